/*
 * mccb_oracle.c -- CPU fp64 oracle for the masked causal depthwise conv1d backward.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the plain, slow, obviously-correct definition of what the
 * GPU library computes. Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load it. It shares no code, header, table or constant with the HIP library, and the HIP library
 * never calls it.
 *
 * Source of truth: the documentation page "aclnnMaskedCausalConv1dBackward" (Ascend CANN aclnn op).
 *   - section 功能说明 (function description), the three equations:
 *       gradYMasked[i,j] = mask[j,i] * gradY[i,j]
 *       gradX[i,j]       = sum_{k=0}^{W-1} gradYMasked[i+k, j] * weight[W-1-k]
 *       gradWeight[k]    = sum_{j=0}^{B-1} sum_{i=0}^{S-1} gradYMasked[i+W-1-k, j] * x[i,j]
 *     and the note under them: invalid (out-of-range) positions are padded with zeros, W is 3 for
 *     now, and every operation is independent along H (the equations leave h implicit).
 *   - section 参数说明 (parameter table): gradY/x/gradX are [S,B,H], weight/gradWeight are [W,H],
 *     mask is an optional bool [B,S]; the float tensors are BFLOAT16 or FLOAT16.
 *   - section 约束说明 (constraints): B in 1..32, B*S in 1..512K, H in 384..24576 and a multiple of
 *     64, W = 3. The oracle does NOT enforce these limits: it is the definition and accepts any
 *     positive S, B, H so that tiny hand-worked cases can be checked. The *_w entry points take the
 *     window W as written in the equations (any W >= 1; the page's is 3), for the kernels' W != 3
 *     extension.
 *
 * Readings where the page is silent (the same readings the library documents):
 *   - mask "true" keeps the gradient (the equation multiplies by it); a null mask means all-true
 *     (the parameter table gives nullptr as the default); one byte per element, nonzero = true,
 *     stored row-major [B,S], so mask[j,i] is byte j*S + i.
 *   - only row indices i' >= S are invalid in the backward (the stencil looks ahead, never behind);
 *     row i' always belongs to the same batch j.
 *   - outputs are correctly rounded (round to nearest, ties to even) from the fp64 value.
 *
 * Arithmetic: everything in fp64. Decoding a 16-bit value to fp64 is exact, every product of two
 * decoded 16-bit values is exact in fp64, and sums follow the loop order written below. Build with
 * -ffp-contract=off so that no multiply-add is fused and the bits are reproducible.
 *
 * Parity pins (tests/test_oracle.py): hand-worked cases derived from the equations, the page's
 * all-zero call example, PyTorch CPU fp64 autograd of the causal depthwise forward, the adjoint
 * (dot-product) identity against oracle_forward, invariants (linearity, batch permutation, null
 * mask == all-true mask) and an exhaustive codec check against numpy / torch casts.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_BF16 0
#define OR_FP16 1
#define OR_TAPS 3 /* W: the constraints section fixes the window at 3 (for now) */

/* ------------------------------------------------------------------------------------------------
 * Codec, written from the IEEE 754 binary16 layout (1 sign, 5 exponent, 10 fraction bits, bias 15)
 * and the bfloat16 layout (1 sign, 8 exponent, 7 fraction bits, bias 127).
 * --------------------------------------------------------------------------------------------- */

static void layout_of(int dtype, int *exp_bits, int *frac_bits) {
    if (dtype == OR_FP16) {
        *exp_bits = 5;
        *frac_bits = 10;
    } else {
        *exp_bits = 8;
        *frac_bits = 7;
    }
}

/* Exact decode: value = (-1)^s * 2^(e-bias) * (1 + f/2^p) for normal e, 2^(1-bias) * f/2^p for
 * e == 0 (subnormal), inf/NaN for the all-ones exponent. */
static double decode_one(int dtype, uint16_t bits) {
    int eb, pb;
    layout_of(dtype, &eb, &pb);
    const int bias = (1 << (eb - 1)) - 1;
    const int sign = bits >> 15;
    const int e = (bits >> pb) & ((1 << eb) - 1);
    const int f = bits & ((1 << pb) - 1);
    double v;
    if (e == (1 << eb) - 1) {
        v = f ? NAN : INFINITY;
    } else if (e == 0) {
        v = ldexp((double)f, 1 - bias - pb);
    } else {
        v = ldexp((double)(f + (1 << pb)), e - bias - pb);
    }
    return sign ? -v : v;
}

/* Round-to-nearest-even encode. In the binade [2^E, 2^(E+1)) (E clamped to the minimum normal
 * exponent, which also covers subnormals) representable magnitudes are the integer multiples of
 * q = 2^(E-p). n = |v|/q is exact (scaling by a power of two); round it to the nearest integer r,
 * ties to even. The encoding is then ((E + bias - 1) << p) + r: for a normal r in [2^p, 2^(p+1))
 * that is the biased exponent field plus the fraction, for a subnormal (E = 1 - bias) it is r itself,
 * and a carry r == 2^(p+1) rolls into the next exponent with a zero fraction. */
static uint16_t encode_one(int dtype, double v) {
    int eb, pb;
    layout_of(dtype, &eb, &pb);
    const int bias = (1 << (eb - 1)) - 1;
    const uint16_t sign = signbit(v) ? 0x8000u : 0u;
    const uint32_t inf_field = ((1u << eb) - 1u) << pb;
    if (isnan(v)) return (uint16_t)(inf_field | (1u << (pb - 1))); /* quiet NaN */
    double a = fabs(v);
    if (isinf(a)) return (uint16_t)(sign | inf_field);
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2); /* a = m * 2^e2, m in [0.5, 1): a lies in the binade of exponent e2 - 1 */
    int E = e2 - 1;
    const int emin = 1 - bias;
    if (E < emin) E = emin;
    const double n = ldexp(a, pb - E); /* |v| / q */
    double r = floor(n);
    const double frac = n - r; /* exact: n and floor(n) share the binade's ulp */
    if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
    const double field = ldexp((double)(E + bias - 1), pb) + r;
    if (field >= (double)inf_field) return (uint16_t)(sign | inf_field); /* overflow */
    return (uint16_t)(sign | (uint16_t)field);
}

void oracle_decode(int dtype, const uint16_t *in, double *out, int64_t n) {
    for (int64_t t = 0; t < n; ++t) out[t] = decode_one(dtype, in[t]);
}

void oracle_encode(int dtype, const double *in, uint16_t *out, int64_t n) {
    for (int64_t t = 0; t < n; ++t) out[t] = encode_one(dtype, in[t]);
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads of the following calls (n >= 1); the results do not depend on it: each thread owns
   whole channels and sums them in the same order. */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------------------------------------
 * The backward (function description section, all three equations).
 * --------------------------------------------------------------------------------------------- */

/* gradYMasked[i,j] (for one h) = mask[j,i] * gradY[i,j], zero for padded rows i >= S. */
static double grad_y_masked(const double *gy, const uint8_t *mask, int64_t S, int64_t B, int64_t H,
                            int64_t i, int64_t j, int64_t h) {
    if (i >= S) return 0.0; /* zero padding of invalid positions */
    const double m = (mask == NULL || mask[j * S + i] != 0) ? 1.0 : 0.0;
    return m * gy[(i * B + j) * H + h];
}

/*
 * Inputs: gY, x [S,B,H] and w [3,H] as 16-bit patterns of `dtype`, mask [B,S] bytes or NULL.
 * Outputs (each may be NULL):
 *   gx64  [S,B,H] fp64 gradX            gx16 [S,B,H] gradX rounded to dtype
 *   gw64  [3,H]   fp64 gradWeight       gw16 [3,H]   gradWeight rounded to dtype
 *   gwrss [3,H]   sqrt(sum of the squared gradWeight terms), a scale for the gradWeight tolerance
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
int oracle_backward_w(int dtype, int W, int64_t S, int64_t B, int64_t H, const uint16_t *gY,
                      const uint16_t *x, const uint16_t *w, const uint8_t *mask, double *gx64,
                      uint16_t *gx16, double *gw64, double *gwrss, uint16_t *gw16) {
    if (S < 1 || B < 1 || H < 1 || W < 1 || !gY || !x || !w) return -1;
    if (dtype != OR_BF16 && dtype != OR_FP16) return -1;
    const int64_t N = S * B * H;
    double *gyd = (double *)malloc(sizeof(double) * (size_t)N);
    double *xd = (double *)malloc(sizeof(double) * (size_t)N);
    double *wd = (double *)malloc(sizeof(double) * (size_t)(W * H));
    if (!gyd || !xd || !wd) {
        free(gyd);
        free(xd);
        free(wd);
        return -1;
    }
    oracle_decode(dtype, gY, gyd, N);
    oracle_decode(dtype, x, xd, N);
    oracle_decode(dtype, w, wd, (int64_t)W * H);

    /* Every h is independent (the H axis is elementwise), so threads split h and each thread owns
     * its outputs: the result does not depend on the thread count. */
#pragma omp parallel for schedule(static)
    for (int64_t h = 0; h < H; ++h) {
        /* gradX[i,j] = sum_{k=0}^{W-1} gradYMasked[i+k,j] * weight[W-1-k] */
        for (int64_t i = 0; i < S; ++i) {
            for (int64_t j = 0; j < B; ++j) {
                double acc = 0.0;
                for (int k = 0; k < W; ++k) {
                    acc += grad_y_masked(gyd, mask, S, B, H, i + k, j, h) * wd[(W - 1 - k) * H + h];
                }
                const int64_t o = (i * B + j) * H + h;
                if (gx64) gx64[o] = acc;
                if (gx16) gx16[o] = encode_one(dtype, acc);
            }
        }
        /* gradWeight[k] = sum_{j=0}^{B-1} sum_{i=0}^{S-1} gradYMasked[i+W-1-k,j] * x[i,j] */
        for (int k = 0; k < W; ++k) {
            double acc = 0.0, sq = 0.0;
            for (int64_t j = 0; j < B; ++j) {
                for (int64_t i = 0; i < S; ++i) {
                    const double term =
                        grad_y_masked(gyd, mask, S, B, H, i + W - 1 - k, j, h) * xd[(i * B + j) * H + h];
                    acc += term;
                    sq += term * term;
                }
            }
            if (gw64) gw64[k * H + h] = acc;
            if (gwrss) gwrss[k * H + h] = sqrt(sq);
            if (gw16) gw16[k * H + h] = encode_one(dtype, acc);
        }
    }
    free(gyd);
    free(xd);
    free(wd);
    return 0;
}

/*
 * The same three equations over a range of rows, for tensors too large to hold whole on the host:
 * gradX rows r0 .. r1-1, and the gradWeight terms of those rows (gradX rows i in [r0, r1) in the
 * gradWeight equation) added into caller-held fp64 sums. Running it over consecutive ranges that
 * cover 0 .. S-1 gives every gradX row and the whole gradWeight sum (summed range by range; within
 * a range j outer, i inner, as above).
 *   gY_rows: [n_gy, B, H] 16-bit patterns of gradY rows r0 .. r0+n_gy-1, where
 *            n_gy = min(r1 + W - 1, S) - r0 (the range and the W-1 rows after it, up to S)
 *   x_rows : [r1 - r0, B, H] rows r0 .. r1-1 of x
 *   w      : [W, H]; mask: the whole [B,S] mask, or NULL
 *   gx16   : [r1 - r0, B, H] gradX rows r0 .. r1-1 rounded to dtype (may be NULL)
 *   gw_acc, gw_sq: [W, H] fp64, incremented by the terms and by their squares (either may be NULL)
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
int oracle_backward_rows_w(int dtype, int W, int64_t S, int64_t B, int64_t H, int64_t r0,
                           int64_t r1, const uint16_t *gY_rows, const uint16_t *x_rows,
                           const uint16_t *w, const uint8_t *mask, uint16_t *gx16, double *gw_acc,
                           double *gw_sq) {
    if (S < 1 || B < 1 || H < 1 || W < 1 || !gY_rows || !x_rows || !w) return -1;
    if (dtype != OR_BF16 && dtype != OR_FP16) return -1;
    if (r0 < 0 || r1 <= r0 || r1 > S) return -1;
    const int64_t n_gy = (r1 + W - 1 < S ? r1 + W - 1 : S) - r0, n_x = r1 - r0;
    double *gyd = (double *)malloc(sizeof(double) * (size_t)(n_gy * B * H));
    double *xd = (double *)malloc(sizeof(double) * (size_t)(n_x * B * H));
    double *wd = (double *)malloc(sizeof(double) * (size_t)(W * H));
    if (!gyd || !xd || !wd) {
        free(gyd);
        free(xd);
        free(wd);
        return -1;
    }
    oracle_decode(dtype, gY_rows, gyd, n_gy * B * H);
    oracle_decode(dtype, x_rows, xd, n_x * B * H);
    oracle_decode(dtype, w, wd, (int64_t)W * H);
#pragma omp parallel for schedule(static)
    for (int64_t h = 0; h < H; ++h) {
        /* gradYMasked of absolute row i, batch j (zero for i >= S); row i sits at i - r0 */
#define GYM(i, j) ((i) >= S ? 0.0                                                           \
                   : ((mask == NULL || mask[(j) * S + (i)] != 0) ? 1.0 : 0.0) *            \
                         gyd[(((i) - r0) * B + (j)) * H + h])
        for (int64_t i = r0; i < r1; ++i) {
            for (int64_t j = 0; j < B; ++j) {
                double acc = 0.0;
                for (int k = 0; k < W; ++k) acc += GYM(i + k, j) * wd[(W - 1 - k) * H + h];
                if (gx16) gx16[((i - r0) * B + j) * H + h] = encode_one(dtype, acc);
            }
        }
        for (int k = 0; k < W; ++k) {
            double acc = 0.0, sq = 0.0;
            for (int64_t j = 0; j < B; ++j) {
                for (int64_t i = r0; i < r1; ++i) {
                    const double term = GYM(i + W - 1 - k, j) * xd[((i - r0) * B + j) * H + h];
                    acc += term;
                    sq += term * term;
                }
            }
            if (gw_acc) gw_acc[k * H + h] += acc;
            if (gw_sq) gw_sq[k * H + h] += sq;
        }
#undef GYM
    }
    free(gyd);
    free(xd);
    free(wd);
    return 0;
}

/* The page's window, W = 3. */
int oracle_backward(int dtype, int64_t S, int64_t B, int64_t H, const uint16_t *gY,
                    const uint16_t *x, const uint16_t *w, const uint8_t *mask, double *gx64,
                    uint16_t *gx16, double *gw64, double *gwrss, uint16_t *gw16) {
    return oracle_backward_w(dtype, OR_TAPS, S, B, H, gY, x, w, mask, gx64, gx16, gw64, gwrss,
                             gw16);
}

/*
 * The forward that these gradients belong to, used only by the adjoint (dot-product) test. The
 * page prints only the backward; the forward is the causal depthwise convolution whose adjoint the
 * equations are: y[i,j] = mask[j,i] * sum_{k=0}^{W-1} weight[k] * x[i-(W-1)+k, j], x[<0] = 0.
 * Operates on fp64 arrays (x [S,B,H], w [W,H], y [S,B,H]).
 */
int oracle_forward_w(int W, int64_t S, int64_t B, int64_t H, const double *x, const double *w,
                     const uint8_t *mask, double *y) {
    if (S < 1 || B < 1 || H < 1 || W < 1 || !x || !w || !y) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t h = 0; h < H; ++h) {
        for (int64_t i = 0; i < S; ++i) {
            for (int64_t j = 0; j < B; ++j) {
                double acc = 0.0;
                for (int k = 0; k < W; ++k) {
                    const int64_t src = i - (W - 1) + k;
                    if (src < 0) continue; /* causal: nothing before the first token */
                    acc += w[k * H + h] * x[(src * B + j) * H + h];
                }
                const double m = (mask == NULL || mask[j * S + i] != 0) ? 1.0 : 0.0;
                y[(i * B + j) * H + h] = m * acc;
            }
        }
    }
    return 0;
}

/* The page's window, W = 3. */
int oracle_forward(int64_t S, int64_t B, int64_t H, const double *x, const double *w,
                   const uint8_t *mask, double *y) {
    return oracle_forward_w(OR_TAPS, S, B, H, x, w, mask, y);
}

/* ------------------------------------------------------------------------------------------------
 * Packed variable-length layout. The sibling operators' pages describe a TND layout: the tokens of
 * all sequences packed along one axis T, with an INT64 array of per-sequence lengths given as
 * cumulative sums (the actualSeqLengths parameter). Here gY, x, gX and y are [T,H], the mask, if
 * any, is one byte per token [T], and cu[b] is the end of sequence b: sequence b holds the tokens
 * cu[b-1] .. cu[b]-1 (cu[-1] = 0), and cu[nseq-1] must equal T. Each sequence is its own
 * [S = length, B = 1] problem: the stencil never reads across a sequence boundary (rows past the
 * end of a sequence, or before its start for the forward, are zero), and gradWeight sums the terms
 * of every sequence.
 * --------------------------------------------------------------------------------------------- */

static int check_cu(int64_t T, int64_t nseq, const int64_t *cu) {
    if (nseq < 1 || !cu) return -1;
    int64_t prev = 0;
    for (int64_t b = 0; b < nseq; ++b) {
        if (cu[b] < prev) return -1;
        prev = cu[b];
    }
    return prev == T ? 0 : -1;
}

int oracle_backward_varlen(int dtype, int W, int64_t T, int64_t H, int64_t nseq, const int64_t *cu,
                           const uint16_t *gY, const uint16_t *x, const uint16_t *w,
                           const uint8_t *mask, double *gx64, uint16_t *gx16, double *gw64,
                           double *gwrss, uint16_t *gw16) {
    if (T < 1 || H < 1 || W < 1 || W > 8 || !gY || !x || !w) return -1;
    if (dtype != OR_BF16 && dtype != OR_FP16) return -1;
    if (check_cu(T, nseq, cu) != 0) return -1;
    double *gyd = (double *)malloc(sizeof(double) * (size_t)(T * H));
    double *xd = (double *)malloc(sizeof(double) * (size_t)(T * H));
    double *wd = (double *)malloc(sizeof(double) * (size_t)(W * H));
    if (!gyd || !xd || !wd) {
        free(gyd);
        free(xd);
        free(wd);
        return -1;
    }
    oracle_decode(dtype, gY, gyd, T * H);
    oracle_decode(dtype, x, xd, T * H);
    oracle_decode(dtype, w, wd, (int64_t)W * H);
#pragma omp parallel for schedule(static)
    for (int64_t h = 0; h < H; ++h) {
        double acc_w[8] = {0}, sq_w[8] = {0}; /* W <= 8 (checked above) */
        for (int64_t b = 0; b < nseq; ++b) {
            const int64_t start = b == 0 ? 0 : cu[b - 1], end = cu[b];
            for (int64_t t = start; t < end; ++t) {
                /* gradX[t] = sum_k gYm[t+k] * w[W-1-k], rows past the sequence end are zero */
                double acc = 0.0;
                for (int k = 0; k < W; ++k) {
                    const int64_t r = t + k;
                    if (r >= end) break;
                    const double m = (mask == NULL || mask[r] != 0) ? 1.0 : 0.0;
                    acc += m * gyd[r * H + h] * wd[(W - 1 - k) * H + h];
                }
                if (gx64) gx64[t * H + h] = acc;
                if (gx16) gx16[t * H + h] = encode_one(dtype, acc);
                /* gradWeight[k] += gYm[t+W-1-k] * x[t], within the sequence */
                for (int k = 0; k < W; ++k) {
                    const int64_t r = t + W - 1 - k;
                    if (r >= end) continue;
                    const double m = (mask == NULL || mask[r] != 0) ? 1.0 : 0.0;
                    const double term = m * gyd[r * H + h] * xd[t * H + h];
                    acc_w[k] += term;
                    sq_w[k] += term * term;
                }
            }
        }
        for (int k = 0; k < W; ++k) {
            if (gw64) gw64[k * H + h] = acc_w[k];
            if (gwrss) gwrss[k * H + h] = sqrt(sq_w[k]);
            if (gw16) gw16[k * H + h] = encode_one(dtype, acc_w[k]);
        }
    }
    free(gyd);
    free(xd);
    free(wd);
    return 0;
}

int oracle_forward_varlen(int W, int64_t T, int64_t H, int64_t nseq, const int64_t *cu,
                          const double *x, const double *w, const uint8_t *mask, double *y) {
    if (T < 1 || H < 1 || W < 1 || !x || !w || !y) return -1;
    if (check_cu(T, nseq, cu) != 0) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t h = 0; h < H; ++h) {
        for (int64_t b = 0; b < nseq; ++b) {
            const int64_t start = b == 0 ? 0 : cu[b - 1], end = cu[b];
            for (int64_t t = start; t < end; ++t) {
                double acc = 0.0;
                for (int k = 0; k < W; ++k) {
                    const int64_t src = t - (W - 1) + k;
                    if (src < start) continue; /* nothing before the sequence's first token */
                    acc += w[k * H + h] * x[src * H + h];
                }
                const double m = (mask == NULL || mask[t] != 0) ? 1.0 : 0.0;
                y[t * H + h] = m * acc;
            }
        }
    }
    return 0;
}
