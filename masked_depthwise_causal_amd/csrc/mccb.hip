// mccb.hip -- masked causal depthwise conv1d backward for MI355X (gfx950).
//
// Computes, for gradY/x/gradX [S,B,H], weight/gradWeight [3,H] and an optional mask [B,S]
// (page "aclnnMaskedCausalConv1dBackward", section 功能说明 / function description):
//   gYm[i,j]     = mask[j,i] * gradY[i,j]                       (zero for i >= S)
//   gradX[i,j]   = gYm[i,j]*w[2] + gYm[i+1,j]*w[1] + gYm[i+2,j]*w[0]
//   gradW[k]     = sum_j sum_i gYm[i+2-k,j] * x[i,j]
// independently for every channel h.
//
// Storage view: with C = B*H, the [S,B,H] tensors are an [S, C] row-major matrix; column
// c = j*H + h never mixes with another column except that gradWeight sums the columns that share h.
// So the whole op is a 3-tap stencil down the rows of that matrix plus a column-group reduction.
// The same kernels take windows of W = 1..4 taps (weight [W,H], look-ahead W-1 rows), gradY and x
// read in place with their own row and batch strides, and the packed variable-length layout
// ([T,H] tokens with cumulative sequence lengths, the stencil cut at each sequence's end); the
// forward y = mask * causal conv(x, w) is a separate one-pass kernel further down.
//
// Kernel 1 (fused): the rows are cut into strips and the columns into blocks; a block walks its
// strip down the rows, a wavefront holding one wave-wide load (64 lanes x V columns, a "column
// group") of each row it handles. Two lane layouts, chosen from the shape alone:
//   wide (B*H at least 32768, a multiple of 4096): 8-byte lanes, 4 column groups per block
//     placed 16 KiB apart in the row (adjacent in a row's last, partial 64 KiB), one wave per
//     group. Four wave-wide loads that far apart are served faster by the HBM than four adjacent
//     ones, fastest when the block's super-chunk (groups x spacing) tiles the row an odd number
//     of times: rows that 64 KiB does not tile so take 4 groups 32 KiB apart or 3 groups 32 KiB
//     apart where those do.
//   ring (everything else): 4-byte lanes, column groups of adjacent columns with 2 waves each,
//     which take the strip's rows round robin; 4 groups per block, or 2 (the narrow ring) where
//     the plan's grid would otherwise stay small (a column's sums do not depend on the count).
// Either way a wave takes kTurnRows rows per round, and the block's waves pass a barrier each
// round, so the block's loads of a row reach the HBM together; each row of gradY, x and gradX
// crosses HBM once. A wave forms gradX for its kTurnRows rows from the masked gradY rows
// i..i+kTurnRows+W-2 it holds in registers (the first W-1 are the previous turn's look-ahead rows:
// in the wide layout the same wave's, kept in its fp64 window; in the ring loaded again and served
// from L2), and accumulates its gradWeight terms in fp64 across all its rounds. Rounds are software-pipelined: a wave issues the loads of its next turn before computing
// the current one, so HBM requests stay in flight through the arithmetic and across the
// (fence-free) round barrier. The strip's mask bytes are staged in LDS once. At the end each column
// group writes one fp64 partial per (strip, tap, column) to the caller's workspace (the ring
// layout first adds its two waves in LDS, in a fixed order). Kernel 2 (reduce) adds the partials
// of each (tap, channel) over strips and batches in a fixed order and rounds once. No atomics
// anywhere: the result bits depend only on the inputs and the plan, and the plan only on
// (S, B, H, dtype, W).
//
// Precision: every product of two 16-bit values is exact in fp64 (and in fp32). gradX's three
// products are summed in fp64 in the equation's order and the sum is rounded once to the dtype
// (round-to-odd to fp32, then round-to-nearest-even, which equals direct rounding of the fp64 sum).
// gradWeight sums stay in fp64 until the final rounding.
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>
#include <vector>

#include "mccb.h"

// Tuning constants (compile-time; every value here gives the same results, except that the lane
// layout of the fused kernel and the strip plan fix the order in which gradWeight's fp64 partial
// sums are formed).
// The wide layout of the fused kernel: MCCB_WIDE_VEC columns per lane, MCCB_WIDE_COL_GROUPS
// column groups MCCB_GROUP_SPACING bytes apart with MCCB_WIDE_RING waves each. The ring layout
// is fixed: 2 columns per lane, 4 adjacent column groups (2 where registers run short) of 2 waves.
#ifndef MCCB_WIDE_VEC
#define MCCB_WIDE_VEC 4  // columns per lane: 4 -> 8-byte loads
#endif
#ifndef MCCB_RING_COL_GROUPS
#define MCCB_RING_COL_GROUPS 4  // column groups of a ring block (2 where registers run short)
#endif
#ifndef MCCB_WIDE_COL_GROUPS
#define MCCB_WIDE_COL_GROUPS 4
#endif
#ifndef MCCB_WIDE_RING
#define MCCB_WIDE_RING 1
#endif
#ifndef MCCB_WIDE_WAVES_PER_SIMD
#define MCCB_WIDE_WAVES_PER_SIMD 2  // occupancy the wide layout is compiled for (caps its VGPRs)
#endif
#ifndef MCCB_GROUP_SPACING
#define MCCB_GROUP_SPACING 16384  // bytes between the column groups of a wide block
#endif
#ifndef MCCB_TURN_ROWS
#define MCCB_TURN_ROWS 8  // rows a wave handles per turn (loads kept in flight together)
#endif
#ifndef MCCB_NT_LOAD
#define MCCB_NT_LOAD 1  // streaming (non-temporal) hint on gradY / x loads read once
#endif
#ifndef MCCB_NT_GY
#define MCCB_NT_GY 1  // ... also on the gradY rows of a backward turn that no other turn reads
#endif
#ifndef MCCB_FWD_NT_X
#define MCCB_FWD_NT_X 1  // ... and on the x rows of a forward tile that no other tile reads
#endif
#ifndef MCCB_REDUCE_VEC
#define MCCB_REDUCE_VEC 1  // gradWeight reduction: channels per lane (1: more blocks across the CUs)
#endif
#ifndef MCCB_NT_STORE
#define MCCB_NT_STORE 1  // streaming (non-temporal) hint on gradX stores
#endif
#ifndef MCCB_EXACT_GRADX
#define MCCB_EXACT_GRADX 1  // 1: gradX correctly rounded from fp64; 0: fp64 -> fp32 -> dtype
#endif
#ifndef MCCB_LDS_FLOOR
#define MCCB_LDS_FLOOR 0  // dynamic LDS bytes the fused kernel reserves at least (caps blocks per CU)
#endif
#ifndef MCCB_STRIP_ROWS
#define MCCB_STRIP_ROWS 1024  // the plan aims for strips about this many rows long ...
#endif
#ifndef MCCB_MIN_BLOCKS
#define MCCB_MIN_BLOCKS 2048  // ... splitting further until the grid has this many blocks ...
#endif
#ifndef MCCB_MIN_STRIP_ROWS
#define MCCB_MIN_STRIP_ROWS 128  // ... but not below this many rows per strip
#endif
#ifndef MCCB_FWD_VEC
#define MCCB_FWD_VEC 8  // forward: channels per lane (8 = 16-byte loads)
#endif
#ifndef MCCB_FWD_WAVES
#define MCCB_FWD_WAVES 4  // forward: wavefronts per block, side by side across the columns
#endif
#ifndef MCCB_FWD_ROWS
#define MCCB_FWD_ROWS 8  // forward: rows one block covers
#endif
#ifndef MCCB_FWD_LDS
#define MCCB_FWD_LDS 0  // forward: LDS reserved per block to cap blocks per CU (0: no cap)
#endif

// Fixed device scratch of mccb_backward_noalloc (the fp64 gradWeight partials), in place of a
// caller's workspace; see scratch_on() below for how host code reaches it.
constexpr uint64_t kScratchBytes = MCCB_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch holds whole 256-byte lines");
static __device__ __align__(256) double scratch[kScratchBytes / sizeof(double)];

namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef double f64x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;  // lanes per wavefront on CDNA
constexpr int kTurnRows = MCCB_TURN_ROWS;
constexpr int kPlanRound = 16;  // strips are a whole number of this many rows (any layout's round)
// Longest strip the plan makes: ceil(S / ceil(S / MCCB_STRIP_ROWS)) <= MCCB_STRIP_ROWS rows,
// rounded up to a whole round (the mask staging is unrolled for it).
constexpr int kPlanMaxStripRows = (MCCB_STRIP_ROWS + kPlanRound - 1) / kPlanRound * kPlanRound;
// Bytes a staged mask slot holds beyond the strip's rows: a whole turn (kTurnRows + W - 1 <= 16
// rows, starting 8-aligned) reads 16 bytes, so the last one reaches 8 bytes past the strip.
constexpr int kMaskPad = 8;
static_assert(kTurnRows == 8 && kTurnRows + 3 <= 16, "a turn's mask bytes are two 8-byte words");
constexpr int kReduceWaves = 16;        // wavefronts per reduce block
constexpr int kReduceVec = MCCB_REDUCE_VEC;          // channels per reduce lane (1 or 2)
constexpr int kReduceCols = kWave * kReduceVec;      // channels per reduce block
static_assert(kReduceVec == 1 || kReduceVec == 2, "reduce lanes own 1 or 2 channels");

// Lane vector of V 16-bit values (V/2 words): one load per row.
template <int V>
struct Vec {
    typedef uint32_t t __attribute__((ext_vector_type(V / 2)));
};

// Lane layouts of the fused kernel (all give each column's gradX bit for bit; gradWeight's fp64
// partials are summed in the layout's order, and the layout is a function of the shape only):
//   WIDE (rows of at least one super-chunk, a multiple of 4096 columns): 8-byte lanes, a block is
//        4 column groups spaced MCCB_GROUP_SPACING bytes apart (adjacent past the row's last whole
//        super-chunk), one wave per group;
//        Two more spacings, for rows the 64 KiB super-chunk tiles an even number of times or
//        not at all: 4 groups 32 KiB apart (128 KiB super-chunks) and 3 groups 32 KiB apart
//        (96 KiB);
//   ring: 4-byte lanes, a block is column groups of adjacent columns with 2 ring waves each
//        (fewer groups, one wave less per SIMD, when the registers run short: strided 3-tap and
//        4-tap windows). The wide layout's 4-tap window keeps fp32 weights widened per use.
constexpr int kLayoutRing = 0, kLayoutWide = 1, kLayoutNarrowRing = 2, kLayoutTall = 3,
              kLayoutWide4x32 = 4, kLayoutWide3x32 = 5;
// group spacing of the two other wide layouts, in bytes
constexpr int64_t kWide32Spacing = 32768;
// The tall layout (sequences of at most kTallRows rows, one strip): 8 ring waves on one column group
// take every row of the strip in a single round, so a block's loads all go out together.
constexpr int kTallWaves = 8;
constexpr int kTallRows = kTallWaves * kTurnRows;
template <int W, bool STRIDED, int LAYOUT>
struct FusedCfg {
    static constexpr bool WIDE =
        LAYOUT == kLayoutWide || LAYOUT == kLayoutWide4x32 || LAYOUT == kLayoutWide3x32;
    static constexpr bool TALL = LAYOUT == kLayoutTall;
    static constexpr bool tight = (STRIDED && W >= 3) || W > 3;
    static constexpr int V = WIDE ? MCCB_WIDE_VEC : 2;  // columns per lane
    static constexpr int CG = LAYOUT == kLayoutWide3x32 ? 3
                              : WIDE ? MCCB_WIDE_COL_GROUPS
                              : TALL ? 1
                                     : ((tight || LAYOUT == kLayoutNarrowRing) ? 2 : MCCB_RING_COL_GROUPS);
    static constexpr int RG = WIDE ? MCCB_WIDE_RING : TALL ? kTallWaves : 2;  // waves per column group
    static constexpr int WPS = WIDE ? MCCB_WIDE_WAVES_PER_SIMD : (tight ? 3 : 4);
    static constexpr int GC = kWave * V;       // columns of one column group
    static constexpr int BW = CG * RG;         // waves per block
    static constexpr int RR = RG * kTurnRows;  // rows a block advances per round
    // longest strip a block of this layout walks (the mask staging is unrolled for it)
    static constexpr int MAX_STRIP = TALL ? kTallRows
                                     : LAYOUT == kLayoutNarrowRing ? (int)MCCB_MIN_STRIP_ROWS
                                                                   : kPlanMaxStripRows;
    // column groups spaced this many lane vectors apart (0: adjacent)
    static constexpr int64_t DLV =
        (LAYOUT == kLayoutWide4x32 || LAYOUT == kLayoutWide3x32) ? kWide32Spacing / (V * 2)
        : WIDE                                                   ? (int64_t)MCCB_GROUP_SPACING / (V * 2)
                                                                 : 0;
    static_assert(!WIDE || W <= 4, "the wide layout holds at most 4 taps");
    static_assert(V == 2 || V == 4, "lane vector must be 4 or 8 bytes");
    static_assert(GC < 384, "a column group spans at most 2 batches (H >= 384)");
    static_assert(CG <= 8, "the staged mask holds two batches for each of at most 8 groups");
    // a turn never straddles the end of a strip other than the tensor's last row: strips are whole
    // rounds (the tall layout has a single strip)
    static_assert(TALL || kPlanRound % RR == 0, "strips must be whole rounds");
    static_assert(BW * kWave <= 1024, "block too large");
    static_assert(DLV % kWave == 0, "group spacing must be a whole number of wave-wide loads");
};

constexpr int64_t kMinH = 384, kMaxH = 24576, kHAlign = 64;
constexpr int64_t kMaxB = 32, kMaxBS = 524288;
constexpr int64_t kMinW = 1, kMaxW = 4;  // window taps supported by the kernels
constexpr int64_t kStripRows = MCCB_STRIP_ROWS;
static_assert(kStripRows <= kPlanMaxStripRows, "strips longer than the mask staging");
constexpr int64_t kMinBlocks = MCCB_MIN_BLOCKS;
constexpr int64_t kMinStripRows = MCCB_MIN_STRIP_ROWS;
constexpr int64_t kMaxMaskLds = 48 * 1024;  // bytes of LDS for the staged mask, at most
// The strip rule counts column blocks of this many columns (its tuning predates the wide layout;
// the strips, not the launch width, fix gradWeight's summation order).
constexpr int64_t kPlanBlockCols = 512;
// Columns of the widest column group (one wave-wide load) of the fused kernel.
constexpr int64_t kMaxGroupCols = (int64_t)kWave * (MCCB_WIDE_VEC > 2 ? MCCB_WIDE_VEC : 2);
// Staged mask batches per block: two per column group (a group's columns span at most two).
constexpr int kMaxStagedBatches =
    2 * (MCCB_WIDE_COL_GROUPS > MCCB_RING_COL_GROUPS ? MCCB_WIDE_COL_GROUPS : MCCB_RING_COL_GROUPS);

// ---------------------------------------------------------------------------------------------
// 16-bit formats
// ---------------------------------------------------------------------------------------------
template <int DT>
struct Fmt;

template <>
struct Fmt<MCCB_BF16> {
    __device__ static inline void unpack(uint32_t u, float &lo, float &hi) {
        lo = __uint_as_float(u << 16);
        hi = __uint_as_float(u & 0xffff0000u);
    }
    __device__ static inline uint32_t pack(float lo, float hi) {  // round to nearest even
        f32x2 f = {lo, hi};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
    }
};

template <>
struct Fmt<MCCB_FP16> {
    __device__ static inline void unpack(uint32_t u, float &lo, float &hi) {
        f16x2 h = __builtin_bit_cast(f16x2, u);
        lo = (float)h.x;
        hi = (float)h.y;
    }
    __device__ static inline uint32_t pack(float lo, float hi) {  // round to nearest even
        f32x2 f = {lo, hi};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
    }
};

// fp64 -> fp32 with round-to-odd: truncate toward zero, then force the last bit to 1 if the value
// was inexact. Rounding the result to nearest-even in a format with at least two fewer significand
// bits (bf16: 8, fp16: 11, against fp32's 24) gives the correctly rounded fp64 value.
__device__ static inline float round_to_odd_f32(double d) {
    const float f = (float)d;  // round to nearest even
    const double back = (double)f;
    const uint32_t b = __float_as_uint(f);
    const uint32_t toward_zero = b - (__builtin_fabs(back) > __builtin_fabs(d) ? 1u : 0u);
    return __uint_as_float(back != d ? (toward_zero | 1u) : b);
}

template <int DT, int V>
__device__ static inline void unpack_vec(const typename Vec<V>::t q, float (&f)[V]) {
#pragma unroll
    for (int p = 0; p < V / 2; ++p) Fmt<DT>::unpack(q[p], f[2 * p], f[2 * p + 1]);
}

template <typename T>
__device__ static inline T load_vec(const T *p) {
#if MCCB_NT_LOAD
    return __builtin_nontemporal_load(p);
#else
    return *p;
#endif
}
template <typename T>
__device__ static inline T load_vec_cached(const T *p) {
    return *p;
}
// gradY rows a turn of the fused kernel reads once (neither look-ahead row of a turn)
template <typename T>
__device__ static inline T load_gy_stream(const T *p) {
#if MCCB_NT_GY
    return load_vec(p);
#else
    return *p;
#endif
}
// x rows of a forward tile that no other tile reads (not the tile's last W-1 rows)
template <typename T>
__device__ static inline T load_fwd_stream(const T *p) {
#if MCCB_FWD_NT_X
    return load_vec(p);
#else
    return *p;
#endif
}
// A global address as a wave-uniform row base plus a 32-bit lane offset. The empty asm keeps the
// base in scalar registers, so that the load or store takes the scalar-base + vector-offset form;
// without it the compiler folds the loop-invariant lane offset into the base ahead of the loop and
// forms every row's address with a 64-bit vector multiply-add. The base is cast back to the global
// address space (the asm hides where it came from). Unoptimized device builds (the host-sanitizer
// test) keep the plain sum: there the base is not kept uniform and cannot be pinned to SGPRs.
template <typename P>
__device__ static inline P *lane_at(P *row_base, uint32_t lane_off) {
#if defined(__OPTIMIZE__)
    asm("" : "+s"(row_base));
    typedef __attribute__((address_space(1))) P gP;
    return (P *)((gP *)row_base + lane_off);
#else
    return row_base + lane_off;
#endif
}

template <typename T>
__device__ static inline void store_vec(T *p, T v) {
#if MCCB_NT_STORE
    __builtin_nontemporal_store(v, p);
#else
    *p = v;
#endif
}

// gradX for one lane's V columns at row i from the masked gradY rows i .. i+W-1 (fp64, d[k] =
// gYm[i+k]), and the gradWeight terms of row i: a[k] += gYm[i+W-1-k] * x[i]. Returns the packed
// gradX row. LIMITED (packed variable-length layout): only d[k] with k < lim belong to row i's
// sequence; the rest count as zero.
template <int DT, int W, int V, bool LIMITED = false, typename WT = double>
__device__ static inline typename Vec<V>::t stencil_row(const double (&d)[W][V],
                                                       const typename Vec<V>::t x_row,
                                                       const WT (&wt)[W][V],
                                                       double (&a)[W][V], int lim = W) {
    float xf[V];
    unpack_vec<DT, V>(x_row, xf);
    float out[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
        // gradX[i] = sum_k gYm[i+k] * w[W-1-k], in k order (each product exact in fp64)
        double s = d[0][e] * (double)wt[W - 1][e];
#pragma unroll
        for (int k = 1; k < W; ++k)
            s = __builtin_fma((!LIMITED || k < lim) ? d[k][e] : 0.0, (double)wt[W - 1 - k][e], s);
#if MCCB_EXACT_GRADX
        out[e] = round_to_odd_f32(s);
#else
        out[e] = (float)s;
#endif
        // gradWeight[k] += gYm[i+W-1-k] * x[i]
        const double xd = (double)xf[e];
#pragma unroll
        for (int k = 0; k < W; ++k)
            a[k][e] = __builtin_fma((!LIMITED || W - 1 - k < lim) ? d[W - 1 - k][e] : 0.0, xd,
                                    a[k][e]);
    }
    typename Vec<V>::t r;
#pragma unroll
    for (int p = 0; p < V / 2; ++p) r[p] = Fmt<DT>::pack(out[2 * p], out[2 * p + 1]);
    return r;
}

// gradWeight entries, rounded once: round-to-odd to fp32, then nearest-even to the dtype.
template <int DT>
__device__ static inline void store_gw(uint16_t *p, double t) {
    *p = (uint16_t)(Fmt<DT>::pack(round_to_odd_f32(t), 0.0f) & 0xFFFFu);
}
template <int DT>
__device__ static inline void store_gw(uint16_t *p, f64x2 t) {  // p 4-byte aligned
    *reinterpret_cast<uint32_t *>(p) = Fmt<DT>::pack(round_to_odd_f32(t[0]), round_to_odd_f32(t[1]));
}

template <int DT, int V>
__device__ static inline void widen(const typename Vec<V>::t q, double (&d)[V]) {
    float f[V];
    unpack_vec<DT, V>(q, f);
#pragma unroll
    for (int e = 0; e < V; ++e) d[e] = (double)f[e];
}

// ---------------------------------------------------------------------------------------------
// Kernel 1: mask + gradX + gradWeight partials in one HBM pass, for a window of W taps (the
// look-ahead is W-1 rows).
// grid.x = n_col_blocks * n_strips (column block fastest), block = CG * RG waves (FusedCfg<W>).
// Dynamic LDS (masked launches): CG * 2 * (rows_per_strip + W - 1) mask bytes, then (VARLEN) the
// strip's rows_per_strip + W - 1 `ahead` bytes.
// Workspace: fp64 partials [n_strips][W][C].
//
// Columns of a block: a column group is one wave-wide load of each row (64 lanes x V columns).
// Column blocks below `n_sp_blocks` place their CG groups DLV lane vectors apart (a super-chunk of
// CG*DLV lane vectors is covered by DLV/64 such blocks); the rest of the row is cut into blocks of
// CG adjacent groups. Every lane vector of a row belongs to exactly one lane of one block.
// ---------------------------------------------------------------------------------------------
// Input strides (in elements; channels contiguous, so only the row and batch strides vary): a
// contiguous [S,B,H] tensor has row stride B*H and batch stride H. With STRIDED false the kernel
// assumes that layout for gradY and x; with STRIDED true it takes each tensor's own strides. Either
// way a load address is a wave-uniform 64-bit base (row, and for STRIDED the wave's first batch)
// plus a 32-bit lane offset; a wave's columns span at most two batches, and the host reads an
// input in place only when the lane offset fits. The mask is always addressed through its strides
// (batch, row), which cost nothing in the once-per-strip staging loop.
struct InStrides {
    int64_t gy_row, gy_batch, x_row, x_batch, m_batch, m_row;
};

// First lane vector (lane 0) of column group g of column block cb.
template <int CG>
__device__ static inline int64_t group_first_vec(int64_t cb, int g, int64_t n_sp_blocks,
                                                 int64_t dlv) {
    if (cb < n_sp_blocks) {
        const int64_t per = dlv / kWave;  // blocks per super-chunk
        const int64_t sup = cb / per, k = cb - sup * per;
        return sup * CG * dlv + g * dlv + k * kWave;
    }
    return n_sp_blocks * CG * kWave + ((cb - n_sp_blocks) * CG + g) * kWave;
}

// VARLEN (packed variable-length layout, B = 1): `ahead[i]` holds the number of rows i, i+1, ...
// that belong to row i's sequence (at least 1); the stencil of row i uses only those.
template <int DT, bool HAS_MASK, bool STRIDED, int W, bool VARLEN, int LAYOUT>
__global__ void __launch_bounds__((FusedCfg<W, STRIDED, LAYOUT>::BW * kWave))
    __attribute__((amdgpu_waves_per_eu((FusedCfg<W, STRIDED, LAYOUT>::WPS))))
    mccb_fused_bwd(const void *__restrict__ gy_, const void *__restrict__ x_,
                   const void *__restrict__ w_, const uint8_t *__restrict__ mask,
                   void *__restrict__ gx_, double *__restrict__ ws, int64_t S, int64_t B, int64_t H,
                   int64_t rows_per_strip, int64_t n_col_blocks, int64_t n_sp_blocks,
                   InStrides st, const uint8_t *__restrict__ ahead, int lim_lds,
                   uint16_t *__restrict__ gw_direct) {
    typedef FusedCfg<W, STRIDED, LAYOUT> Cfg;
    static_assert(!(Cfg::TALL && VARLEN), "the packed layout does not take the tall blocks");
    constexpr int V = Cfg::V, CG = Cfg::CG, RG = Cfg::RG, TR = kTurnRows, RR = Cfg::RR;
    typedef typename Vec<V>::t vec_t;
    constexpr int L = W - 1;  // look-ahead rows
    extern __shared__ __attribute__((aligned(16))) uint8_t smask[];
    // Whether a wave's turns overlap (the next turn's loads in flight while the current turn is
    // computed; see issue_sel). Measured per layout: the plain ring (a padded tensor, many blocks
    // of adjacent column groups with two ring waves each) runs faster without, every other layout
    // with.
    constexpr bool kPipe = LAYOUT != kLayoutRing || VARLEN;

    const int lane = threadIdx.x & (kWave - 1);
    // The wave index is the same on every lane of a wave; saying so keeps everything derived from
    // it (row ranges, row addresses) in scalar registers.
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int ring = wave / CG;   // position along rows
    const int group = wave % CG;  // column group
    const int64_t C = B * H;
    const int64_t CV = C / V;  // lane vectors per row
    // (block, row and column indices are below 2^31: 32-bit divisions, a few instructions each
    // instead of a 64-bit division's hundred)
    const int64_t col_block = (int64_t)(blockIdx.x % (uint32_t)n_col_blocks);
    const int64_t strip = (int64_t)(blockIdx.x / (uint32_t)n_col_blocks);
    const int64_t rs0 = strip * rows_per_strip;
    const int64_t rs1 = (rs0 + rows_per_strip < S) ? rs0 + rows_per_strip : S;

    // Lanes past the last column load a valid column (the last one) and store nothing.
    const int64_t v0 = group_first_vec<CG>(col_block, group, n_sp_blocks, Cfg::DLV);
    const int64_t v_raw = v0 + lane;
    const bool active = v_raw < CV;
    const int64_t v = active ? v_raw : CV - 1;
    const int64_t c = v * V;
    const int64_t j = (int64_t)((uint32_t)c / (uint32_t)H);
    const int64_t h = c - j * H;
    // the wave's first batch
    const int64_t jg = (int64_t)((uint32_t)((v0 < CV ? v0 : CV - 1) * V) / (uint32_t)H);

    const int span = (int)(rows_per_strip + L);  // rows of the strip and its look-ahead
    const int mspan = (int)(rows_per_strip + kMaskPad);  // bytes of one staged mask slot
    // Wave-uniform row addresses plus one 32-bit lane offset: loads and stores take the
    // scalar-base + vector-offset form, with no per-lane 64-bit address arithmetic.
    const int64_t row_bytes = C * 2;
    const uint32_t lane_off = (uint32_t)(v * (V * 2));
    // STRIDED: the wave's first batch goes into the uniform base, the lane keeps the rest
    const char *gy_base = reinterpret_cast<const char *>(gy_) + (STRIDED ? jg * st.gy_batch * 2 : 0);
    const char *x_base = reinterpret_cast<const char *>(x_) + (STRIDED ? jg * st.x_batch * 2 : 0);
    const int64_t gy_rb = STRIDED ? st.gy_row * 2 : row_bytes;
    const int64_t x_rb = STRIDED ? st.x_row * 2 : row_bytes;
    const uint32_t gy_lane = STRIDED ? (uint32_t)(((j - jg) * st.gy_batch + h) * 2) : lane_off;
    const uint32_t x_lane = STRIDED ? (uint32_t)(((j - jg) * st.x_batch + h) * 2) : lane_off;
    // Row base in scalar registers plus the lane's offset (lane_at); the 4-tap window keeps the
    // compiler's own form (measured: 3-tap headline backward 75.3-75.4 -> 75.7-76.1 % of 8 TB/s,
    // 4-tap 73.3-73.5 -> 72.4-72.8 %, four alternating runs).
    auto at_lane = [&](auto *row_base, uint32_t lane) {
        if constexpr (W <= 3) return lane_at(row_base, lane);
        return row_base + lane;
    };
    auto at_gy = [&](int64_t row) -> const vec_t * {
        return reinterpret_cast<const vec_t *>(at_lane(gy_base + row * gy_rb, gy_lane));
    };
    auto at_x = [&](int64_t row) -> const vec_t * {
        return reinterpret_cast<const vec_t *>(at_lane(x_base + row * x_rb, x_lane));
    };
    auto out_at = [&](int64_t row) -> vec_t * {
        return reinterpret_cast<vec_t *>(
            at_lane(reinterpret_cast<char *>(gx_) + row * row_bytes, lane_off));
    };
    // The loads of one turn (gradY rows i0 .. i0+TR+L-1, x rows i0 .. i0+TR-1); CLAMP: a row past
    // the tensor's last row S-1 is read at row S-1, a valid address, and cleared before use.
    auto issue_rows = [&](auto clamp_tag, int64_t i0, vec_t(&qy)[TR + L], vec_t(&qx)[TR]) {
        constexpr bool CLAMP = decltype(clamp_tag)::value;
        auto row = [&](int64_t r) -> int64_t {
            if constexpr (CLAMP) return r < S - 1 ? r : S - 1;
            return r;
        };
#pragma unroll
        for (int k = 0; k < L; ++k) qy[k] = load_vec_cached(at_gy(row(i0 + k)));
#pragma unroll
        for (int u = 0; u < TR - L; ++u) qy[u + L] = load_gy_stream(at_gy(row(i0 + L + u)));
#pragma unroll
        for (int u = TR - L; u < TR; ++u) qy[u + L] = load_vec_cached(at_gy(row(i0 + L + u)));
#pragma unroll
        for (int u = 0; u < TR; ++u) qx[u] = load_vec(at_x(row(i0 + u)));
    };
    // Every round issues one turn of loads, with no condition around them: behind a condition the
    // compiler's wait counts before each row of the current turn must also hold on the path
    // without those loads, so on the path with them each row would wait for the next turn's loads
    // as well and the two turns would not overlap. Without a next turn (`real` false, the same on
    // every lane) the loads read the first row of the weights, which is in L2, and are not used.
    const uint32_t w_lane = (uint32_t)(h * 2);
    auto issue_sel = [&](auto clamp_tag, bool real, int64_t i0, vec_t(&qy)[TR + L],
                         vec_t(&qx)[TR], auto lead_tag) {
        constexpr bool CLAMP = decltype(clamp_tag)::value;
        constexpr bool LEAD = decltype(lead_tag)::value;  // the turn's first L gradY rows too
        const int s1 = (int)(S - 1);  // rows are below 2^31
        auto row = [&](int r) -> int {
            if constexpr (CLAMP) return r < s1 ? r : s1;
            return r;
        };
        const int r0 = (int)i0;
        const char *gb = real ? gy_base : reinterpret_cast<const char *>(w_);
        const char *xb = real ? x_base : reinterpret_cast<const char *>(w_);
        const int64_t grb = real ? gy_rb : 0, xrb = real ? x_rb : 0;
        const uint32_t gl = real ? gy_lane : w_lane, xl = real ? x_lane : w_lane;
        auto gy_at = [&](int r) {
            return reinterpret_cast<const vec_t *>(at_lane(gb + (int64_t)row(r) * grb, gl));
        };
        auto x_at = [&](int r) {
            return reinterpret_cast<const vec_t *>(at_lane(xb + (int64_t)row(r) * xrb, xl));
        };
        if constexpr (LEAD) {
#pragma unroll
            for (int k = 0; k < L; ++k) qy[k] = load_vec_cached(gy_at(r0 + k));
        }
#pragma unroll
        for (int u = 0; u < TR - L; ++u) qy[u + L] = load_gy_stream(gy_at(r0 + L + u));
#pragma unroll
        for (int u = TR - L; u < TR; ++u) qy[u + L] = load_vec_cached(gy_at(r0 + L + u));
#pragma unroll
        for (int u = 0; u < TR; ++u) qx[u] = load_vec(x_at(r0 + u));
    };
    // A turn is "whole" when this wave's TR rows and their look-ahead rows all exist.
    auto whole = [&](int64_t r0) {
        if constexpr (kPipe) {
            // rows are below 2^31: 32-bit compares stay in scalar registers
            const int i0 = (int)r0 + ring * TR;
            return i0 + TR <= (int)rs1 && i0 + TR + L <= (int)S;
        } else {
            const int64_t i0 = r0 + ring * TR;
            return i0 + TR <= rs1 && i0 + TR + L <= S;
        }
    };
    // Whether this wave has a turn in the round that starts at row r0 (its first row inside the
    // strip).
    auto has_turn = [&](int r0) { return r0 + ring * TR < (int)rs1; };
    // The weights and the first turn's loads go out before the mask staging (every layout but the
    // plain ring), so that one round trip covers all three at the start of a block.
    const vec_t *w = reinterpret_cast<const vec_t *>(w_);
    vec_t ay[TR + L], ax[TR], wraw[W];
    const int64_t t_i0 = rs0 + ring * TR;
    if constexpr (kPipe) {
#pragma unroll
        for (int k = 0; k < W; ++k) wraw[k] = w[(k * H + h) / V];
        if constexpr (Cfg::TALL) {
            if (t_i0 < rs1) issue_rows(std::true_type{}, t_i0, ay, ax);
        } else if constexpr (LAYOUT == kLayoutNarrowRing) {
            issue_sel(std::true_type{}, has_turn((int)rs0), t_i0, ay, ax, std::true_type{});
        } else {
            issue_sel(std::false_type{}, whole(rs0), t_i0, ay, ax, std::true_type{});
        }
    }

    int moff = 0;  // offset of this lane's batch in the staged mask
    if constexpr (HAS_MASK) {
        // Each column group stages the bytes of its (at most two) batches: [CG][2][mspan], 0xFF
        // where the mask keeps the row and 0 where it drops it (or the row is past S); the second
        // slot only when the group's columns reach into the next batch. A slot is a multiple of 8
        // bytes and holds 8 bytes past the strip's look-ahead, so that a whole turn reads its
        // rows' bytes as two aligned 8-byte words. A thread loads all of its bytes from clamped,
        // always valid addresses before it writes any of them to LDS, and decides afterwards
        // which of them count: no load depends on a branch, so they issue back to back and the
        // thread waits once instead of once per byte.
        int64_t jf[CG];
        bool two[CG];
#pragma unroll
        for (int gg = 0; gg < CG; ++gg) {
            const int64_t vg = group_first_vec<CG>(col_block, gg, n_sp_blocks, Cfg::DLV);
            const int64_t va = vg < CV ? vg : CV - 1, vb = vg + kWave - 1 < CV ? vg + kWave - 1 : CV - 1;
            jf[gg] = (int64_t)((uint32_t)(va * V) / (uint32_t)H);
            two[gg] = (int64_t)((uint32_t)(vb * V + V - 1) / (uint32_t)H) != jf[gg];
        }
        // Slot (gg, b) holds bytes rs0 .. rs0+mspan-1 of mask row jf[gg] + b; a thread takes bytes
        // tid, tid + kThreads, ... of every slot. The slot's batch is the same for the whole block.
        constexpr int kThreads = Cfg::BW * kWave;
        constexpr int kPer = (Cfg::MAX_STRIP + kMaskPad + kThreads - 1) / kThreads;
        uint8_t vals[2 * CG][kPer];
#pragma unroll
        for (int slot = 0; slot < 2 * CG; ++slot) {
            const int gg = slot >> 1;
            const bool second = (slot & 1) != 0;
            const uint8_t *src = mask + (jf[gg] + ((second && two[gg]) ? 1 : 0)) * st.m_batch;
#pragma unroll
            for (int q = 0; q < kPer; ++q) {
                const int64_t row = rs0 + (int)threadIdx.x + q * kThreads;
                vals[slot][q] = src[(row < S ? row : S - 1) * st.m_row];
            }
        }
#pragma unroll
        for (int slot = 0; slot < 2 * CG; ++slot) {
            const bool used = (slot & 1) == 0 || two[slot >> 1];
#pragma unroll
            for (int q = 0; q < kPer; ++q) {
                const int t = (int)threadIdx.x + q * kThreads;
                if (t < mspan)
                    smask[slot * mspan + t] =
                        (used && rs0 + t < S && vals[slot][q] != 0) ? (uint8_t)0xFF : (uint8_t)0;
            }
        }
        moff = (group * 2 + (int)(j - jg)) * mspan;
        if constexpr (!VARLEN) __syncthreads();
    }
    if constexpr (VARLEN) {
        for (int t = threadIdx.x; t < span; t += blockDim.x) {
            const int64_t row = rs0 + t;
            smask[lim_lds + t] = (row < S) ? ahead[row] : (uint8_t)1;
        }
        __syncthreads();
    }
    // rows of the output row's sequence from that row on (VARLEN), the same for every lane
    auto lim_of = [&](int64_t row) -> int {
        if constexpr (VARLEN) return __builtin_amdgcn_readfirstlane(smask[lim_lds + (int)(row - rs0)]);
        return W;
    };

    // The wide layout's 4-tap window keeps its weights in fp32 (exact for 16-bit values) and
    // widens them at each use: fp64 copies of 4 taps x 4 columns would not fit beside its state.
    constexpr bool kNarrowW = Cfg::WIDE && W > 3;
    typedef typename std::conditional<kNarrowW, float, double>::type wt_t;
    wt_t wt[W][V];
#pragma unroll
    for (int k = 0; k < W; ++k) {
        float t[V];
        unpack_vec<DT, V>(kPipe ? wraw[k] : w[(k * H + h) / V], t);
#pragma unroll
        for (int e = 0; e < V; ++e) wt[k][e] = (wt_t)t[e];
    }
    // an empty asm that "changes" the fp32 weights, so that their widening is redone after it
    // instead of being hoisted into fp64 copies that live through the loop (which spills). Once
    // per whole turn: 4-tap headline backward 68.0-68.2 -> 72.1-72.2 % of 8 TB/s against once per
    // row (70.4-70.5 every 2 rows, 71.7 every 4), 249-256 VGPRs and no spill; the row-at-a-time
    // turns keep one per row.
    auto refresh_wt = [&]() {
        if constexpr (kNarrowW) {
#pragma unroll
            for (int k = 0; k < W; ++k)
#pragma unroll
                for (int e = 0; e < V; ++e) asm volatile("" : "+v"(wt[k][e]));
        }
    };

    double a[W][V];
#pragma unroll
    for (int k = 0; k < W; ++k)
#pragma unroll
        for (int e = 0; e < V; ++e) a[k][e] = 0.0;

    vec_t zero;
#pragma unroll
    for (int p = 0; p < V / 2; ++p) zero[p] = 0u;
    // Whether the mask keeps gradY row `row` of this lane's batch (rows < S only).
    auto keep = [&](int64_t row) -> bool {
        if constexpr (HAS_MASK) return smask[moff + (int)(row - rs0)] != 0;
        return true;
    };
    // A whole turn's mask: the staged bytes of rows i0 .. i0+15 (i0 - rs0 is a multiple of 8);
    // `masked(q, mw, k)` is gradY row i0+k's lane vector with every word cleared where the mask
    // drops the row (the byte, sign-extended, is the word mask).
    auto turn_mask = [&](int64_t i0, uint32_t (&mw)[4]) {
        if constexpr (HAS_MASK) {
            const uint8_t *mp = smask + moff + (int)(i0 - rs0);
            const uint2 lo = *reinterpret_cast<const uint2 *>(mp);
            const uint2 hi = *reinterpret_cast<const uint2 *>(mp + 8);
            mw[0] = lo.x;
            mw[1] = lo.y;
            mw[2] = hi.x;
            mw[3] = hi.y;
        }
    };
    auto masked = [&](const vec_t &q, const uint32_t (&mw)[4], int k) -> vec_t {
        if constexpr (!HAS_MASK) return q;
        const uint32_t m = (uint32_t)((int32_t)(mw[k >> 2] << (24 - 8 * (k & 3))) >> 24);
        vec_t r;
#pragma unroll
        for (int p = 0; p < V / 2; ++p) r[p] = q[p] & m;
        return r;
    };

    // Issue the loads of a whole turn: gradY rows i0 .. i0+TR+L-1 and x rows i0 .. i0+TR-1. The
    // first L gradY rows were the previous turn's last look-ahead rows (this wave's own with one
    // wave per group, the other ring wave's otherwise), and this turn's last L are the next turn's
    // first: cached loads, so those come from L2; the rest stream.
    // (Each kind of load has a loop of its own: a choice between a cached and a streaming load
    // of one address inside one loop body is merged into a single plain load by the compiler.)
    auto issue = [&](int64_t r0, vec_t (&qy)[TR + L], vec_t (&qx)[TR]) {
        issue_rows(std::false_type{}, r0 + ring * TR, qy, qx);
    };
    // A turn's rows; its fp64 window `d` either starts from the turn's first L gradY rows (LEAD)
    // or holds them already: the wave's previous turn ends with exactly those rows in it.
    auto compute_w = [&](int64_t r0, const vec_t (&qy)[TR + L], const vec_t (&qx)[TR],
                         double (&d)[W][V], auto lead_tag) {
        const int64_t i0 = r0 + ring * TR;
        uint32_t mw[4];
        turn_mask(i0, mw);
        if constexpr (decltype(lead_tag)::value) {
#pragma unroll
            for (int k = 0; k < L; ++k) widen<DT, V>(masked(qy[k], mw, k), d[k]);
        }
#pragma unroll
        for (int u = 0; u < TR; ++u) {
            widen<DT, V>(masked(qy[u + L], mw, u + L), d[L]);
            if (u == 0) refresh_wt();
            vec_t r;
            if constexpr (VARLEN) {
                // a uniform branch: only the last W-1 rows of a sequence take the limited form
                const int lim = lim_of(i0 + u);
                if (lim >= W)
                    r = stencil_row<DT, W, V>(d, qx[u], wt, a);
                else
                    r = stencil_row<DT, W, V, true>(d, qx[u], wt, a, lim);
            } else {
                r = stencil_row<DT, W, V>(d, qx[u], wt, a);
            }
            if (active) store_vec(out_at(i0 + u), r);
#pragma unroll
            for (int k = 0; k < L; ++k)
#pragma unroll
                for (int e = 0; e < V; ++e) d[k][e] = d[k + 1][e];
        }
    };
    auto compute = [&](int64_t r0, const vec_t (&qy)[TR + L], const vec_t (&qx)[TR]) {
        double d[W][V];
        compute_w(r0, qy, qx, d, std::true_type{});
    };
    // Partial turn at the end of the strip or of the tensor: one row at a time, gradY rows past S
    // read as zero.
    auto partial = [&](int64_t r0) {
        const int64_t i0 = r0 + ring * TR;
        if (i0 >= rs1) return;
        const int64_t i1 = (i0 + TR < rs1) ? i0 + TR : rs1;
        double d[W][V];
#pragma unroll
        for (int k = 0; k < L; ++k)
            widen<DT, V>((i0 + k < S && keep(i0 + k)) ? load_vec_cached(at_gy(i0 + k)) : zero, d[k]);
        for (int64_t i = i0; i < i1; ++i) {
            widen<DT, V>((i + L < S && keep(i + L)) ? load_vec_cached(at_gy(i + L)) : zero, d[L]);
            refresh_wt();
            const vec_t r = VARLEN ? stencil_row<DT, W, V, true>(d, load_vec(at_x(i)), wt, a, lim_of(i))
                                   : stencil_row<DT, W, V>(d, load_vec(at_x(i)), wt, a);
            if (active) store_vec(out_at(i), r);
#pragma unroll
            for (int k = 0; k < L; ++k)
#pragma unroll
                for (int e = 0; e < V; ++e) d[k][e] = d[k + 1][e];
        }
    };
    // One round: prefetch the next round's whole turn into `nxt`, then compute this round from
    // `cur` (loaded one round earlier) while those loads are in flight.
    auto round = [&](int64_t r0, const vec_t (&cy)[TR + L], const vec_t (&cx)[TR],
                     vec_t (&ny)[TR + L], vec_t (&nx)[TR]) {
        const int64_t rn = r0 + RR;
        if (rn < rs1 && whole(rn)) issue(rn, ny, nx);
        if (whole(r0))
            compute(r0, cy, cx);
        else
            partial(r0);
        // Keep the block's waves on the same round: ring waves share look-ahead rows through L2,
        // and the column groups' loads of a row reach the HBM together. A bare barrier, without a
        // memory fence, so the prefetched loads stay in flight across it.
        __builtin_amdgcn_s_barrier();
    };

    // A turn that may reach past the tensor's last row S-1 (its loads clamped there): the rows past
    // S-1 are cleared (the staged mask already holds 0 for them) and only rows inside the strip
    // are stored; its x rows past S-1 meet only cleared gradY rows and add nothing to gradWeight.
    auto turn_clear = [&](int64_t i0, const vec_t (&qy)[TR + L], const vec_t (&qx)[TR]) {
        uint32_t mw[4];
        turn_mask(i0, mw);
        if constexpr (!HAS_MASK) {
            const int64_t nv = S - i0;  // rows of the turn that exist, >= 1
            const uint64_t lo = nv >= 8 ? ~0ull : (1ull << (8 * nv)) - 1u;
            const uint64_t hi = nv >= 16 ? ~0ull : nv <= 8 ? 0ull : (1ull << (8 * (nv - 8))) - 1u;
            mw[0] = (uint32_t)lo;
            mw[1] = (uint32_t)(lo >> 32);
            mw[2] = (uint32_t)hi;
            mw[3] = (uint32_t)(hi >> 32);
        }
        auto clear = [&](const vec_t &q, int k) -> vec_t {
            const uint32_t m = (uint32_t)((int32_t)(mw[k >> 2] << (24 - 8 * (k & 3))) >> 24);
            vec_t r;
#pragma unroll
            for (int p = 0; p < V / 2; ++p) r[p] = q[p] & m;
            return r;
        };
        double d[W][V];
#pragma unroll
        for (int k = 0; k < L; ++k) widen<DT, V>(clear(qy[k], k), d[k]);
#pragma unroll
        for (int u = 0; u < TR; ++u) {
            widen<DT, V>(clear(qy[u + L], u + L), d[L]);
            refresh_wt();
            vec_t r;
            if constexpr (VARLEN) {
                const int lim = lim_of(i0 + u);
                if (lim >= W)
                    r = stencil_row<DT, W, V>(d, qx[u], wt, a);
                else
                    r = stencil_row<DT, W, V, true>(d, qx[u], wt, a, lim);
            } else {
                r = stencil_row<DT, W, V>(d, qx[u], wt, a);
            }
            if (active && i0 + u < rs1) store_vec(out_at(i0 + u), r);
#pragma unroll
            for (int k = 0; k < L; ++k)
#pragma unroll
                for (int e = 0; e < V; ++e) d[k][e] = d[k + 1][e];
        }
    };
    if constexpr (Cfg::TALL) {
        // one round covers the strip
        if (t_i0 < rs1) turn_clear(t_i0, ay, ax);
    } else if constexpr (LAYOUT == kLayoutNarrowRing) {
        // Small grids: every turn's loads are clamped (a scalar operation per row), so the last
        // strip's last turns need no separate, slower form; with a mask every turn takes the
        // clearing form (one copy of the turn code keeps the registers in bounds).
        auto turn_c = [&](int r0, const vec_t (&cy)[TR + L], const vec_t (&cx)[TR]) {
            const int64_t i0 = r0 + ring * TR;
            if (HAS_MASK || i0 + TR + L > S)
                turn_clear(i0, cy, cx);
            else
                compute(r0, cy, cx);
        };
        // The rounds in which this wave has a turn come first (a turn exists while its first row
        // is inside the strip); every round loads the next turn (see issue_sel) and computes
        // this one, with no other path through the loop, so the compiler's wait counts are
        // exact. Unrolled by two so that the two register buffers swap roles without copies.
        // Then one barrier for each round left (every wave passes one barrier per round).
        vec_t by[TR + L], bx[TR];
        int r0 = (int)rs0;
        for (; has_turn(r0); r0 += 2 * RR) {
            issue_sel(std::true_type{}, has_turn(r0 + RR), r0 + RR + ring * TR, by, bx,
                      std::true_type{});
            turn_c(r0, ay, ax);
            __builtin_amdgcn_s_barrier();  // as in round()
            if (!has_turn(r0 + RR)) {
                r0 += RR;
                break;
            }
            issue_sel(std::true_type{}, has_turn(r0 + 2 * RR), r0 + 2 * RR + ring * TR, ay, ax,
                      std::true_type{});
            turn_c(r0 + RR, by, bx);
            __builtin_amdgcn_s_barrier();
        }
        for (; r0 < (int)rs1; r0 += RR) __builtin_amdgcn_s_barrier();
    } else if constexpr (kPipe) {
        // As in the narrow ring: first the rounds in which this wave's turn is whole, each loading
        // the next turn and computing this one with no other path through the loop, then the rest
        // of the strip (the last strip's turns that reach past row S-1, or none) row by row, one
        // barrier per round.
        // With one wave per column group (the wide layouts) a turn's first L gradY rows are the
        // wave's previous turn's last ones: its fp64 window carries them over, and only the
        // strip's first turn loads them (16 loads a turn instead of 18 at 3 taps). Measured:
        // headline 74.6-75.5 -> 76.4-76.7 % of 8 TB/s per call, 4 taps 73.4-73.8 -> 75.4-75.6 %
        // (249 VGPRs, no spill).
        constexpr bool kCarry = Cfg::RG == 1 && !VARLEN;
        const auto lead = std::integral_constant<bool, !kCarry>{};
        vec_t by[TR + L], bx[TR];
        double dc[W][V];  // the carried window (kCarry)
        auto turn_w = [&](int r, const vec_t (&cy)[TR + L], const vec_t (&cx)[TR]) {
            if constexpr (kCarry)
                compute_w(r, cy, cx, dc, std::false_type{});
            else
                compute(r, cy, cx);
        };
        auto next_whole = [&](int r) { return r < (int)rs1 && whole(r); };
        int r0 = (int)rs0;
        if constexpr (kCarry) {
            if (whole(r0)) {
                uint32_t mw[4];
                turn_mask(r0 + ring * TR, mw);
#pragma unroll
                for (int k = 0; k < L; ++k) widen<DT, V>(masked(ay[k], mw, k), dc[k]);
            }
        }
        for (; whole(r0); r0 += 2 * RR) {
            issue_sel(std::false_type{}, next_whole(r0 + RR), r0 + RR + ring * TR, by, bx, lead);
            turn_w(r0, ay, ax);
            __builtin_amdgcn_s_barrier();  // as in round()
            if (!next_whole(r0 + RR)) {
                r0 += RR;
                break;
            }
            issue_sel(std::false_type{}, next_whole(r0 + 2 * RR), r0 + 2 * RR + ring * TR, ay, ax,
                      lead);
            turn_w(r0 + RR, by, bx);
            __builtin_amdgcn_s_barrier();
        }
        for (; r0 < (int)rs1; r0 += RR) {
            partial(r0);
            __builtin_amdgcn_s_barrier();
        }
    } else {
        vec_t by[TR + L], bx[TR];
        if (whole(rs0)) issue(rs0, ay, ax);
        // Unrolled by two so that the two register buffers swap roles without copies.
        for (int64_t r0 = rs0; r0 < rs1; r0 += 2 * RR) {
            round(r0, ay, ax, by, bx);
            if (r0 + RR >= rs1) break;
            round(r0 + RR, by, bx, ay, ax);
        }
    }

    // gradWeight partials of the strip, one fp64 value per (tap, column); or, with gw_direct (one
    // strip and one batch: the block's sums are the whole gradWeight of its channels), gradWeight
    // itself, rounded once. The reduction kernel would add the partial to a zero sum: adding +0.0
    // here gives the same bits.
    if constexpr (RG == 1) {
        // one wave per column group: the lane's own sums are the partials
        if (active) {
#pragma unroll
            for (int k = 0; k < W; ++k)
#pragma unroll
                for (int p = 0; p < V / 2; ++p)
                    *reinterpret_cast<f64x2 *>(ws + (strip * W + k) * C + c + 2 * p) =
                        f64x2{a[k][2 * p], a[k][2 * p + 1]};
        }
    } else {
        // add the RG waves of each column group in a fixed order (ring position 0 first)
        __shared__ f64x2 red[Cfg::BW][kWave * V / 2];
#pragma unroll
        for (int k = 0; k < W; ++k) {
            __syncthreads();
#pragma unroll
            for (int p = 0; p < V / 2; ++p)
                red[wave][lane * (V / 2) + p] = f64x2{a[k][2 * p], a[k][2 * p + 1]};
            __syncthreads();
            if (ring == 0 && active) {
#pragma unroll
                for (int p = 0; p < V / 2; ++p) {
                    f64x2 sum = red[group][lane * (V / 2) + p];
#pragma unroll
                    for (int q = 1; q < RG; ++q) sum += red[q * CG + group][lane * (V / 2) + p];
                    if (gw_direct)
                        store_gw<DT>(gw_direct + k * H + c + 2 * p, sum + f64x2{0.0, 0.0});
                    else
                        *reinterpret_cast<f64x2 *>(ws + (strip * W + k) * C + c + 2 * p) = sum;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------------------------
// Kernel 2: gradWeight[k,h] = sum over strips s (outer) and batches j (inner) of
// ws[s][k][j*H + h], in fp64, then one rounding to the dtype.
// grid = (ceil(H / kReduceCols), W), block = kReduceWaves * 64 lanes; a lane owns kReduceVec
// channels. Each wave sums a contiguous range of the (s, j) rows; the waves' sums are then added
// in wave order. The order of every channel's sum depends only on (n_strips, B), not on
// kReduceVec.
// ---------------------------------------------------------------------------------------------
template <int DT>
__global__ void __launch_bounds__(kReduceWaves *kWave)
    mccb_gw_reduce(const double *__restrict__ ws, uint16_t *__restrict__ gw, int64_t n_strips,
                   int64_t B, int64_t H) {
    constexpr int RV = kReduceVec;
    typedef typename std::conditional<RV == 2, f64x2, double>::type rvec_t;
    __shared__ rvec_t red[kReduceWaves][kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int k = blockIdx.y;
    const int W = gridDim.y;  // taps
    const int64_t h = (int64_t)blockIdx.x * kReduceCols + lane * RV;
    const int64_t C = B * H;
    const int64_t rows = n_strips * B;
    const int64_t per = (rows + kReduceWaves - 1) / kReduceWaves;
    const int64_t lo = wave * per;
    const int64_t hi = (lo + per < rows) ? lo + per : rows;

    // The wave's rows in order, kBatch loads in flight at a time. `off` (the same on every lane)
    // is the element offset of row r's partials: row (s, j) sits at (s*W + k)*C + j*H. It stops
    // at the wave's last row, so the loads past it re-read that row (always in bounds) and are
    // not added.
    constexpr int kBatch = 16;
    rvec_t acc = {};
    if (h < H && lo < hi) {
        // (lo and B are below 2^31: 32-bit division)
        int64_t jj = (int64_t)((uint32_t)lo % (uint32_t)B);
        int64_t off = ((int64_t)((uint32_t)lo / (uint32_t)B) * W + k) * C + jj * H;
        const int64_t wrap = W * C - (B - 1) * H;  // from (s, B-1) to (s+1, 0)
        const double *base = ws + h;
        for (int64_t r = lo; r < hi; r += kBatch) {
            rvec_t v[kBatch];
#pragma unroll
            for (int q = 0; q < kBatch; ++q) {
                v[q] = *reinterpret_cast<const rvec_t *>(base + off);
                if (r + q + 1 < hi) {
                    if (++jj == B) {
                        jj = 0;
                        off += wrap;
                    } else {
                        off += H;
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < kBatch; ++q)
                if (r + q < hi) acc += v[q];
        }
    }
    red[wave][lane] = acc;
    __syncthreads();
    if (wave == 0 && h < H) {
        rvec_t t = red[0][lane];
        for (int q = 1; q < kReduceWaves; ++q) t += red[q][lane];
        store_gw<DT>(gw + k * H + h, t);  // gradWeight[k, h ..]: one rounding per channel
    }
}


// ---------------------------------------------------------------------------------------------
// Forward kernel: y[i,c] = mask[j,i] * sum_{k=0}^{W-1} w[k,h] x[i-W+1+k, c], with c = j*H + h and
// rows before 0 read as 0 (the causal depthwise conv the backward above differentiates; W = 3 on
// the page). Pure streaming: read x, write y, nothing to reduce.
//
// A block covers a short tile of contiguous columns (kFwdWaves wavefronts, kFwdVec channels per
// lane; 8 rows x 2048 columns when B*H is large, see `cw` below). Tiles are numbered row-major,
// column tile fastest, so the blocks in flight at any moment sit on a few neighbouring
// rows; the HBM serves such a compact front markedly faster than many independent column walks.
// The W-1 rows before the tile are re-read with cached loads (the tile above loaded them, also
// cached, as its last rows); when the column-tile count is a multiple of the 8 XCDs, which take
// blocks round-robin, a tile and the tile above it run on the same XCD and the re-read hits its L2.
//
// Every output is the exact W-term sum (products of 16-bit values are exact in fp64) rounded once:
// round-to-odd to fp32, then round-to-nearest-even to the dtype.
// ---------------------------------------------------------------------------------------------
constexpr int kFwdVec = MCCB_FWD_VEC;
constexpr int kFwdWords = kFwdVec / 2;
constexpr int kFwdWaves = MCCB_FWD_WAVES;
constexpr int kFwdRows = MCCB_FWD_ROWS;
static_assert(kFwdVec == 2 || kFwdVec == 4 || kFwdVec == 8, "forward lane vector: 4, 8 or 16 bytes");
static_assert(kFwdRows >= 3, "the look-back rows (up to 3) come from the tile above");
static_assert(kFwdWaves * kWave <= 1024, "forward block too large");
static_assert((kFwdWaves & (kFwdWaves - 1)) == 0, "forward waves per block: a power of two");

typedef uint32_t fvec_t __attribute__((ext_vector_type(kFwdWords)));

template <int DT>
__device__ static inline void widen_f(const fvec_t q, double (&d)[kFwdVec]) {
#pragma unroll
    for (int p = 0; p < kFwdWords; ++p) {
        float lo, hi;
        Fmt<DT>::unpack(q[p], lo, hi);
        d[2 * p] = (double)lo;
        d[2 * p + 1] = (double)hi;
    }
}

// VARLEN (packed variable-length layout, B = 1): `behind[i]` holds the number of rows before row i
// that belong to its sequence; the window of row i uses only those.
//
// cw = 2^cw_log2 (1, 2, 4 or kFwdWaves, chosen by the host) is how many of the block's waves sit
// side by side across the columns; the rest stack along the rows, so a block covers
// (kFwdWaves / cw) * kFwdRows rows x cw * kWave * kFwdVec columns. Narrow rows (the packed
// layout's H columns, or a small B*H) use fewer columns per block instead of leaving lanes idle.
// Register budget: 4 wavefronts per SIMD (at most 128 VGPRs) for windows of up to 3 taps; the
// 16-byte lanes of a 4-tap window need more.
constexpr int fwd_waves_per_simd(int w) { return w > 3 ? 3 : 4; }

template <int DT, bool HAS_MASK, bool STRIDED, int W, bool VARLEN = false>
__global__ void __launch_bounds__(kFwdWaves *kWave)
    __attribute__((amdgpu_waves_per_eu(fwd_waves_per_simd(W))))
    mccb_fwd(const fvec_t *__restrict__ x, const fvec_t *__restrict__ w,
             const uint8_t *__restrict__ mask, fvec_t *__restrict__ y, int64_t S, int64_t B,
             int64_t H, int64_t n_ct, int cw_log2, InStrides st,
             const uint8_t *__restrict__ behind = nullptr) {
    constexpr int L = W - 1;  // look-back rows
    extern __shared__ uint8_t fwd_reserved[];  // sized at launch, never used: caps blocks per CU
    if (S < 0) fwd_reserved[threadIdx.x] = 0;   // never taken (S >= 1): keeps the symbol live
    // (tile, column and batch indices are below 2^31: 32-bit divisions, a few instructions each
    // instead of a 64-bit division's hundred)
    const int64_t ct = (int64_t)(blockIdx.x % (uint32_t)n_ct);  // column tile (fastest)
    const int64_t rt = (int64_t)(blockIdx.x / (uint32_t)n_ct);  // row tile
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int wc = wave & ((1 << cw_log2) - 1), wr = wave >> cw_log2;  // column slot, row slot
    const int64_t C = B * H;
    // The wave's wave-wide chunk of the row. Where a block's 4 waves sit side by side and 64 KiB
    // super-chunks tile the row an odd number of times, a block takes 4 chunks 16 KiB apart
    // instead of 4 adjacent ones, as the backward's wide layout does (headline forward 74.1-74.6
    // -> 76.8-77.0 % of 8 TB/s; 128 KiB rows, an even number, 0.5 points slower). Only which
    // columns a block covers changes.
    int64_t q = (ct << cw_log2) + wc;
    if constexpr (!STRIDED && !VARLEN && kFwdWaves == 4) {
        constexpr int64_t kSpace = 16384 / (kWave * kFwdVec * 2);  // chunks per 16 KiB
        const int64_t n_chunks = (B * H) / (kWave * kFwdVec);
        if (cw_log2 == 2 && n_chunks % (4 * kSpace) == 0 && (n_chunks / (4 * kSpace)) % 2 == 1) {
            const int64_t sup = (int64_t)((uint32_t)ct / (uint32_t)kSpace), k = ct - sup * kSpace;
            q = sup * (4 * kSpace) + wc * kSpace + k;
        }
    }
    const int64_t c0 = q * (int64_t)(kWave * kFwdVec) + lane * kFwdVec;
    if (c0 >= C) return;  // no barrier below: lanes past the last column just leave
    const int64_t CV = C / kFwdVec;  // lane vectors per row (C is a multiple of 64)
    const int64_t v = c0 / kFwdVec;
    // the lane's kFwdVec channels share one batch: H % 64 == 0
    const int64_t j = (int64_t)((uint32_t)c0 / (uint32_t)H);
    const int64_t h0 = c0 - j * H;
    const int64_t r0 = (rt * (kFwdWaves >> cw_log2) + wr) * kFwdRows;  // may be >= S: rows guarded

    // Loads are issued before any of them is used, weights first (the first rows' arithmetic
    // needs them), then the mask, then the x rows.
    //
    // Weights: fp64 copies take 2*W*kFwdVec registers for the whole tile. The 4-tap and the
    // packed-layout instantiations, which need the room, keep them in fp32 (exact for 16-bit
    // values) and widen them at each use instead; the others keep fp64 copies, which measured
    // faster for them.
    constexpr bool kNarrowW = W > 3 || VARLEN;
    typedef typename std::conditional<kNarrowW, float, double>::type wt_t;
    fvec_t wq[W];
#pragma unroll
    for (int k = 0; k < W; ++k) wq[k] = w[(k * H + h0) / kFwdVec];

    // Mask of the tile's rows as words of bytes, byte u for row r0+u: 0xFF keeps the row, 0 drops
    // it (or the row is past S); it clears the packed output words of dropped rows. When the
    // tile's bytes are contiguous and 8-byte aligned (unit row stride, batch stride and base
    // multiples of 8, all rows inside S; the same answer on every lane of the wave) they arrive as
    // one 8-byte load per lane, as raw bytes (any nonzero byte keeps its row) turned into 0xFF / 0
    // once the x loads are issued; otherwise byte by byte from clamped addresses, loaded without a
    // branch so that the loads issue together.
    constexpr int kMaskWords = (kFwdRows + 3) / 4;
    uint32_t mk[kMaskWords];
#pragma unroll
    for (int q = 0; q < kMaskWords; ++q) mk[q] = ~0u;
    if constexpr (HAS_MASK) {
        const uint8_t *mcol = mask + j * st.m_batch;
        const bool vec_ok = kFwdRows == 8 && st.m_row == 1 && (st.m_batch & 7) == 0 &&
                            (reinterpret_cast<uintptr_t>(mask) & 7) == 0 && r0 + kFwdRows <= S;
        if (vec_ok) {
            const uint2 mb = load_vec_cached(reinterpret_cast<const uint2 *>(mcol + r0));
            mk[0] = mb.x;
            mk[kMaskWords > 1 ? 1 : 0] = mb.y;
        } else {
            uint8_t mbyte[kFwdRows];
#pragma unroll
            for (int u = 0; u < kFwdRows; ++u)
                mbyte[u] = mcol[((r0 + u < S) ? r0 + u : S - 1) * st.m_row];
#pragma unroll
            for (int q = 0; q < kMaskWords; ++q) mk[q] = 0u;
#pragma unroll
            for (int u = 0; u < kFwdRows; ++u)
                mk[u / 4] |= (r0 + u < S && mbyte[u] != 0) ? 0xFFu << (8 * (u % 4)) : 0u;
        }
    }

    // x rows r0-L .. r0+kFwdRows-1; rows outside [0, S) are zero. The look-back rows and the
    // tile's last L rows (the next tile's look-back) are cached loads, the rest stream. Tiles whose
    // rows all exist (all but the first and the last, a uniform test) load without a branch per
    // row.
    fvec_t xr[kFwdRows + L];
    auto x_at = [&](int64_t row) -> const fvec_t * {
        return STRIDED ? reinterpret_cast<const fvec_t *>(reinterpret_cast<const char *>(x) +
                                                           (row * st.x_row + j * st.x_batch + h0) * 2)
                       : x + row * CV + v;
    };
    // (Each kind of load has a loop of its own: a choice between a cached and a streaming load
    // of one address inside one loop body is merged into a single plain load by the compiler.)
    if (r0 >= L && r0 + kFwdRows <= S) {
#pragma unroll
        for (int u = 0; u < L; ++u) xr[u] = load_vec_cached(x_at(r0 - L + u));
#pragma unroll
        for (int u = L; u < kFwdRows; ++u) xr[u] = load_fwd_stream(x_at(r0 - L + u));
#pragma unroll
        for (int u = kFwdRows; u < kFwdRows + L; ++u) xr[u] = load_vec_cached(x_at(r0 - L + u));
    } else {
        auto guarded = [&](int u, bool stream) {
            const int64_t row = r0 - L + u;
            fvec_t q = {};
            if (row >= 0 && row < S) q = stream ? load_fwd_stream(x_at(row)) : load_vec_cached(x_at(row));
            xr[u] = q;
        };
#pragma unroll
        for (int u = 0; u < L; ++u) guarded(u, false);
#pragma unroll
        for (int u = L; u < kFwdRows; ++u) guarded(u, true);
#pragma unroll
        for (int u = kFwdRows; u < kFwdRows + L; ++u) guarded(u, false);
    }
    if constexpr (HAS_MASK) {
        // any nonzero byte keeps its row: set each byte's top bit where the byte is nonzero (no
        // carry crosses a byte), then widen that bit to the whole byte (0xFF stays 0xFF)
#pragma unroll
        for (int q = 0; q < kMaskWords; ++q) {
            const uint32_t t = (((mk[q] & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | mk[q]) & 0x80808080u;
            mk[q] = (t >> 7) * 0xFFu;
        }
    }
    wt_t wt[W][kFwdVec];
#pragma unroll
    for (int k = 0; k < W; ++k) {
#pragma unroll
        for (int p = 0; p < kFwdWords; ++p) {
            float lo, hi;
            Fmt<DT>::unpack(wq[k][p], lo, hi);
            wt[k][2 * p] = lo;
            wt[k][2 * p + 1] = hi;
        }
    }
    // VARLEN: rows of the tile whose window reaches into another sequence. If the tile's last row
    // has at least kFwdRows-1+L earlier rows in its sequence, no row of the tile does, and the
    // tile takes the unlimited form (a uniform branch; only tiles at sequence starts do not).
    bool limited = false;
    if constexpr (VARLEN) {
        const int64_t last = r0 + kFwdRows - 1;
        limited = __builtin_amdgcn_readfirstlane(
                      (last < S && behind[last] >= kFwdRows - 1 + L) ? 0 : 1) != 0;
    }
    // first window position inside row r0+u's sequence (limited tiles only): window rows before
    // it belong to an earlier sequence
    auto first_of = [&](int u) -> int {
        const int b = (r0 + u < S) ? (int)behind[r0 + u] : L;
        return __builtin_amdgcn_readfirstlane(L - (b < L ? b : L));
    };

    double win[W][kFwdVec];  // win[k] = x row i-L+k
#pragma unroll
    for (int k = 0; k < L; ++k) widen_f<DT>(xr[k], win[k]);
#pragma unroll
    for (int u = 0; u < kFwdRows; ++u) {
        const int64_t row = r0 + u;
        widen_f<DT>(xr[u + L], win[L]);
        if (VARLEN && limited) {
            // Window rows of an earlier sequence count as zero: clear them here, once; the window
            // only slides forward, so later rows of this sequence never see them either.
            const int first = first_of(u);
            if (first > 0) {
#pragma unroll
                for (int k = 0; k < L; ++k)
                    if (k < first)
#pragma unroll
                        for (int e = 0; e < kFwdVec; ++e) win[k][e] = 0.0;
            }
        }
        // fp32 weights: an empty asm that "changes" them, so that their widening is redone after
        // it instead of being hoisted into fp64 copies that live through the tile. 4 taps: once
        // per tile (165 VGPRs, 3 waves/SIMD as before; headline forward 69.0 -> 73.0 % of 8 TB/s
        // against once per row); the packed layout's shorter windows once per row (once per tile
        // spills).
        if (kNarrowW && (W <= 3 || u == 0)) {
#pragma unroll
            for (int k = 0; k < W; ++k)
#pragma unroll
                for (int e = 0; e < kFwdVec; ++e) asm volatile("" : "+v"(wt[k][e]));
        }
        float out[kFwdVec];
#pragma unroll
        for (int e = 0; e < kFwdVec; ++e) {
            // y[i] = sum_k w[k] x[i-L+k], in k order, exact in fp64, rounded once
            double s = win[0][e] * (double)wt[0][e];
#pragma unroll
            for (int k = 1; k < W; ++k) s = __builtin_fma(win[k][e], (double)wt[k][e], s);
            out[e] = round_to_odd_f32(s);
        }
        // all ones where the mask keeps row r0+u, zero (+0.0 in both halves) where it drops it
        const uint32_t keep = (uint32_t)((int32_t)(mk[u / 4] << (24 - 8 * (u % 4))) >> 24);
        fvec_t r;
#pragma unroll
        for (int p = 0; p < kFwdWords; ++p) r[p] = Fmt<DT>::pack(out[2 * p], out[2 * p + 1]) & keep;
        if (row < S) __builtin_nontemporal_store(r, y + row * CV + v);
#pragma unroll
        for (int k = 0; k < L; ++k)
#pragma unroll
            for (int e = 0; e < kFwdVec; ++e) win[k][e] = win[k + 1][e];
    }
}

// ---------------------------------------------------------------------------------------------
// Pack kernel: gathers a strided 16-bit [R0, R1, H] tensor into contiguous rows of the workspace,
// dst[(a*R1 + b)*H + h] = src[a*s0 + b*s1 + h*s2], for inputs the kernels above cannot read in
// place (channels not contiguous, or rows misaligned for their vector loads). One block per
// (a, b) row; each lane writes two channels as one 32-bit store (H is even).
// ---------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
    mccb_pack(const uint16_t *__restrict__ src, uint32_t *__restrict__ dst, int64_t R1, int64_t H,
              int64_t s0, int64_t s1, int64_t s2) {
    const int64_t r = blockIdx.x;
    const int64_t a = r / R1, b = r - a * R1;
    const uint16_t *row = src + a * s0 + b * s1;
    uint32_t *out = dst + r * (H / 2);
    for (int64_t q = threadIdx.x; q < H / 2; q += blockDim.x) {
        const uint32_t lo = row[(2 * q) * s2], hi = row[(2 * q + 1) * s2];
        out[q] = lo | (hi << 16);
    }
}

// ---------------------------------------------------------------------------------------------
// Packed variable-length layout: per-token window limits from the cumulative sequence ends cu[]
// (sequence b holds tokens cu[b-1] .. cu[b]-1, cu[-1] = 0). One thread per token, a binary search
// for the first end past it. ahead[t] = tokens t.. up to its sequence's end (1..255, clamped);
// behind[t] = tokens of its sequence before t (0..255, clamped). A malformed cu (decreasing, or
// not ending at T) gives clamped limits, never an access outside [0, T).
// ---------------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
    mccb_seg_limits(const int64_t *__restrict__ cu, int64_t nseq, int64_t T,
                    uint8_t *__restrict__ ahead, uint8_t *__restrict__ behind) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= T) return;
    int64_t lo = 0, hi = nseq;  // first b with cu[b] > t, or nseq
    while (lo < hi) {
        const int64_t mid = (lo + hi) / 2;
        if (cu[mid] > t) hi = mid;
        else lo = mid + 1;
    }
    int64_t start = lo == 0 ? 0 : cu[lo - 1];
    int64_t end = lo < nseq ? cu[lo] : T;
    if (start > t) start = t;
    if (start < 0) start = 0;
    if (end <= t) end = t + 1;
    if (end > T) end = T;
    const int64_t a = end - t, b = t - start;
    ahead[t] = (uint8_t)(a > 255 ? 255 : a);
    if (behind) behind[t] = (uint8_t)(b > 255 ? 255 : b);
}

// ---------------------------------------------------------------------------------------------
// Host side: validation, plan, launch.
// ---------------------------------------------------------------------------------------------
struct Plan {
    int64_t S, B, H, C;
    int dtype, W;
    int64_t rows_per_strip, n_strips, n_col_blocks;
    // one strip and one batch: the fused kernel's block sums are whole gradWeight entries, so it
    // writes gradWeight itself and the reduction kernel (and the workspace) is not needed
    bool direct;
    uint64_t ws_bytes;
    size_t mask_lds;
};

int check_shape(int64_t S, int64_t B, int64_t H, int dtype) {
    if (dtype != MCCB_BF16 && dtype != MCCB_FP16) return MCCB_ERR_PARAM_INVALID;
    if (B < 1 || B > kMaxB || S < 1 || S > kMaxBS || B * S > kMaxBS) return MCCB_ERR_SHAPE;
    if (H < kMinH || H > kMaxH || H % kHAlign != 0) return MCCB_ERR_SHAPE;
    return MCCB_OK;
}

// Window taps W (the weight's first dimension): 3 on the page; 1..4 here.
int check_taps(int64_t W) { return (W >= kMinW && W <= kMaxW) ? MCCB_OK : MCCB_ERR_SHAPE; }

// Pure function of (S, B, H, dtype, W) -- never of the device -- so gradWeight's summation order,
// and therefore its bits, are the same on every run and every MI355X.
Plan make_plan(int64_t S, int64_t B, int64_t H, int dtype, int W = 3) {
    Plan p;
    p.S = S;
    p.B = B;
    p.H = H;
    p.C = B * H;
    p.dtype = dtype;
    p.W = W;
    p.n_col_blocks = (p.C + kPlanBlockCols - 1) / kPlanBlockCols;
    // Split the rows into strips of about kStripRows rows, more if the grid would have fewer than
    // kMinBlocks blocks (too few to keep every CU busy), but none shorter than kMinStripRows rows;
    // strips are a whole number of rounds long. Short-lived blocks keep the rows in flight across
    // the GPU close together, which the HBM serves faster than long independent column walks; each
    // strip costs 8*W bytes per column of partials written and read back, against 6 bytes per
    // element streamed.
    const int64_t max_strips = (S + kPlanRound - 1) / kPlanRound;
    int64_t strips = (S + kStripRows - 1) / kStripRows;
    const int64_t fill = (kMinBlocks + p.n_col_blocks - 1) / p.n_col_blocks;
    if (strips < fill) strips = fill;
    const int64_t shortest = (S + kMinStripRows - 1) / kMinStripRows;
    if (strips > shortest) strips = shortest;
    if (strips > max_strips) strips = max_strips;
    if (strips < 1) strips = 1;
    for (;;) {
        const int64_t rows = (S + strips - 1) / strips;
        p.rows_per_strip = (rows + kPlanRound - 1) / kPlanRound * kPlanRound;
        p.mask_lds = (size_t)kMaxStagedBatches * (size_t)(p.rows_per_strip + kMaskPad);
        if (p.mask_lds <= (size_t)kMaxMaskLds || strips >= max_strips) break;
        ++strips;  // keep the staged mask within its LDS budget
    }
    p.n_strips = (S + p.rows_per_strip - 1) / p.rows_per_strip;
    p.direct = p.n_strips == 1 && B == 1;
    p.ws_bytes = p.direct ? 0u : (uint64_t)p.n_strips * (uint64_t)W * (uint64_t)p.C * sizeof(double);
    return p;
}

bool overlaps(const void *a, uint64_t na, const void *b, uint64_t nb) {
    const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
    return pa < pb + nb && pb < pa + na;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Optional event-based timing of the two kernels.
struct Profile {
    std::mutex mu;
    bool on = false;
    int cap = 0, n = 0;
    std::vector<hipEvent_t> ev;  // 3 per call: before kernel 1, between, after kernel 2
} g_prof;

// Column blocks of the fused kernel for a W-tap window: `ncb` in all, of which the first `n_sp`
// place their column groups DLV lane vectors apart (whole super-chunks of CG*DLV lane vectors);
// the rest of the row is cut into blocks of adjacent groups. The strips (and with them the
// gradWeight summation order) come from the plan alone.
struct FusedGrid {
    int64_t ncb, n_sp;
};
template <int W, bool STRIDED, int LAYOUT>
FusedGrid fused_grid(int64_t C) {
    typedef FusedCfg<W, STRIDED, LAYOUT> Cfg;
    const int64_t CV = C / Cfg::V;
    FusedGrid g;
    g.n_sp = Cfg::DLV > 0 ? CV / (Cfg::CG * Cfg::DLV) * (Cfg::DLV / kWave) : 0;
    const int64_t rest = CV - g.n_sp * Cfg::CG * kWave;
    g.ncb = g.n_sp + (rest + Cfg::CG * kWave - 1) / (Cfg::CG * kWave);
    return g;
}

// The wide layout is used for the padded layouts (windows of 1..4 taps) when a row of B*H columns
// holds at least one of its super-chunks (CG groups x the group spacing: 32768 columns) and is a
// whole number of 4096 columns (8 KiB); the rest of such a row takes blocks of adjacent groups.
// Elsewhere the ring layouts. (Measured: on rows 6 KiB past a multiple of 8 KiB the ring is
// 4 points faster, on rows a multiple of 8 KiB the wide layout is 2-8 points faster.) A function
// of the shape only, so gradWeight's summation order is too.
bool fused_wide(int64_t C, int64_t W) {
    typedef FusedCfg<3, false, kLayoutWide> Cfg;
    return W <= 4 && Cfg::DLV > 0 && (C / Cfg::V) >= (Cfg::CG * Cfg::DLV) && C % 4096 == 0;
}

// Which wide layout a row takes: the one whose super-chunk (groups x spacing) tiles the row an odd
// number of times, in the order 4 x 16 KiB, 4 x 32 KiB, 3 x 32 KiB; else 4 x 16 KiB with blocks of
// adjacent groups in the row's last, partial super-chunk. Measured per row length (3-tap bf16
// backward, % of 8 TB/s, alternating runs): an even number of super-chunks, or a partial one,
// costs 1-7 points against an odd number (4 x 16 KiB on 128 KiB rows 70.3-71.8 against 4 x 32 KiB
// 72.9-73.4; 3 x 16 KiB on 96 KiB rows 67 against 3 x 32 KiB 74.0 and 4 x 16 KiB 70.4; 3 x 32 KiB
// on 192 KiB rows 72.2 against 4 x 16 KiB 74.5; 4 x 32 KiB on 384 and 640 KiB rows +0.7-0.8).
// Rows a whole number of 256 KiB have no odd tiling here and keep 4 x 16 KiB (ahead of 4 x 32 KiB
// on 1536 KiB rows by 0.5). Contiguous inputs only: the row length is the memory's. Groups enter
// no column's summation order, so every wide layout gives the same bits.
int wide_layout(int64_t C, bool strided) {
    const int64_t L = C * 2;  // bytes of a row
    const int64_t K = 1024;
    if (strided || (L % (64 * K) == 0 && (L / (64 * K)) % 2 == 1)) return kLayoutWide;
    if (L % (128 * K) == 0 && (L / (128 * K)) % 2 == 1) return kLayoutWide4x32;
    if (L % (96 * K) == 0 && (L / (96 * K)) % 2 == 1) return kLayoutWide3x32;
    return kLayoutWide;
}

// Columns per lane of the fused kernel that a call runs (its loads' size and alignment).
int fused_vec(int64_t S, int64_t C, int64_t W) {
    return (S > kTallRows && fused_wide(C, W)) ? FusedCfg<3, false, kLayoutWide>::V
                                               : FusedCfg<3, false, kLayoutRing>::V;
}

// The layout a fused launch takes: tall for sequences of at most kTallRows rows (one strip, which
// its 8 ring waves cover in one round), else wide (above), else the ring; the narrow ring (2 column groups
// instead of 4, so twice the blocks) when the ring's grid would stay under the plan's block target
// (the 128-row floor on strips stopped the plan short of it), and the ring is not already narrow
// (strided 3-tap, 4-tap). The column groups of a block do not enter any column's summation
// order, so the narrow ring's results equal the ring's bit for bit.
int fused_layout(const Plan &p, bool strided, bool varlen) {
    if (!varlen && p.S <= kTallRows) return kLayoutTall;  // one strip, one round
    if (!varlen && fused_wide(p.C, p.W)) return wide_layout(p.C, strided);
    const bool tight = (strided && p.W >= 3) || p.W > 3;
    if (!tight && fused_grid<3, false, kLayoutRing>(p.C).ncb * p.n_strips < kMinBlocks)
        return kLayoutNarrowRing;
    return kLayoutRing;
}

template <int DT, bool M, bool T, int TAPS, bool VL, int LAYOUT>
hipError_t launch_fused(const Plan &p, const void *gy, const void *x, const void *w,
                        const uint8_t *mask, void *gx, void *ws, hipStream_t st, size_t lds,
                        const InStrides &is, const uint8_t *ahead, int lim_lds, void *gw_direct) {
    typedef FusedCfg<TAPS, T, LAYOUT> Cfg;
    // the kernel's assumptions: turns never straddle an inner strip end, the tall layout has one
    // strip, and a direct gradWeight write needs the in-block sum over several ring waves
    if ((!Cfg::TALL && p.rows_per_strip % Cfg::RR != 0) || (Cfg::TALL && p.n_strips != 1) ||
        p.rows_per_strip > Cfg::MAX_STRIP ||
        (gw_direct && Cfg::RG < 2))
        return hipErrorInvalidValue;
    const FusedGrid fg = fused_grid<TAPS, T, LAYOUT>(p.C);
    hipLaunchKernelGGL((mccb_fused_bwd<DT, M, T, TAPS, VL, LAYOUT>),
                       dim3((unsigned)(fg.ncb * p.n_strips)), dim3(Cfg::BW * kWave), lds, st, gy,
                       x, w, mask, gx, (double *)ws, p.S, p.B, p.H, p.rows_per_strip, fg.ncb,
                       fg.n_sp, is, ahead, lim_lds, (uint16_t *)gw_direct);
    return hipGetLastError();
}

template <int DT, bool M, bool T, int TAPS, bool VL>
hipError_t launch_fused_layout(int layout, const Plan &p, const void *gy, const void *x,
                               const void *w, const uint8_t *mask, void *gx, void *ws,
                               hipStream_t st, size_t lds, const InStrides &is,
                               const uint8_t *ahead, int lim_lds, void *gw_direct) {
    if constexpr (!VL) {
        if (layout == kLayoutTall)
            return launch_fused<DT, M, T, TAPS, VL, kLayoutTall>(p, gy, x, w, mask, gx, ws, st,
                                                                 lds, is, ahead, lim_lds, gw_direct);
    }
    if constexpr (!VL) {
        if (layout == kLayoutWide)
            return launch_fused<DT, M, T, TAPS, VL, kLayoutWide>(p, gy, x, w, mask, gx, ws, st,
                                                                 lds, is, ahead, lim_lds, gw_direct);
    }
    if constexpr (!VL && !T) {
        if (layout == kLayoutWide4x32)
            return launch_fused<DT, M, T, TAPS, VL, kLayoutWide4x32>(
                p, gy, x, w, mask, gx, ws, st, lds, is, ahead, lim_lds, gw_direct);
        if (layout == kLayoutWide3x32)
            return launch_fused<DT, M, T, TAPS, VL, kLayoutWide3x32>(
                p, gy, x, w, mask, gx, ws, st, lds, is, ahead, lim_lds, gw_direct);
    }
    if constexpr (!((T && TAPS >= 3) || TAPS > 3)) {  // instantiated where the ring is not narrow
        if (layout == kLayoutNarrowRing)
            return launch_fused<DT, M, T, TAPS, VL, kLayoutNarrowRing>(
                p, gy, x, w, mask, gx, ws, st, lds, is, ahead, lim_lds, gw_direct);
    }
    return launch_fused<DT, M, T, TAPS, VL, kLayoutRing>(p, gy, x, w, mask, gx, ws, st, lds, is,
                                                         ahead, lim_lds, gw_direct);
}

// One fused launch for any (mask, strided, W) of the padded layouts (VL false) or the packed one.
template <int DT, bool VL>
hipError_t launch_fused_any(const Plan &p, const void *gy, const void *x, const void *w,
                            const uint8_t *mask, void *gx, void *ws, hipStream_t st, size_t lds,
                            const InStrides &is, bool strided, const uint8_t *ahead,
                            int lim_lds, void *gw_direct) {
    const int layout = fused_layout(p, strided, VL);
#define MCCB_FUSED(M, T, TAPS)                                                                    \
    return launch_fused_layout<DT, M, T, TAPS, VL>(layout, p, gy, x, w, mask, gx, ws, st, lds, is, \
                                                   ahead, lim_lds, gw_direct)
#define MCCB_FUSED_W(TAPS)                                                                        \
    if constexpr (!VL) {                                                                          \
        if (strided) {                                                                            \
            if (mask) MCCB_FUSED(true, true, TAPS);                                               \
            MCCB_FUSED(false, true, TAPS);                                                        \
        }                                                                                         \
    }                                                                                             \
    if (mask) MCCB_FUSED(true, false, TAPS);                                                      \
    MCCB_FUSED(false, false, TAPS);
    switch (p.W) {
        case 1: MCCB_FUSED_W(1)
        case 2: MCCB_FUSED_W(2)
        case 3: MCCB_FUSED_W(3)
        case 4: MCCB_FUSED_W(4)
        default: return hipErrorInvalidValue;
    }
#undef MCCB_FUSED_W
#undef MCCB_FUSED
}

template <int DT>
hipError_t launch(const Plan &p, const void *gy, const void *x, const void *w, const uint8_t *mask,
                  void *gx, void *gw, void *ws, hipStream_t st, hipEvent_t *ev,
                  const InStrides &is, bool strided) {
    const size_t lds_floor = MCCB_LDS_FLOOR;
    const size_t lds = mask ? (p.mask_lds > lds_floor ? p.mask_lds : lds_floor) : lds_floor;
    if (ev && hipEventRecord(ev[0], st) != hipSuccess) return hipErrorInvalidValue;
    hipError_t e = launch_fused_any<DT, false>(p, gy, x, w, mask, gx, ws, st, lds, is, strided,
                                               nullptr, 0, p.direct ? gw : nullptr);
    if (e != hipSuccess) return e;
    if (ev && hipEventRecord(ev[1], st) != hipSuccess) return hipErrorInvalidValue;
    if (p.direct) {  // gradWeight already written
        if (ev && hipEventRecord(ev[2], st) != hipSuccess) return hipErrorInvalidValue;
        return hipSuccess;
    }
    const dim3 grid2((unsigned)((p.H + kReduceCols - 1) / kReduceCols), (unsigned)p.W);
    const dim3 block2(kReduceWaves * kWave);
    hipLaunchKernelGGL((mccb_gw_reduce<DT>), grid2, block2, 0, st, (const double *)ws,
                       (uint16_t *)gw, p.n_strips, p.B, p.H);
    e = hipGetLastError();
    if (e == hipSuccess && ev && hipEventRecord(ev[2], st) != hipSuccess) return hipErrorInvalidValue;
    return e;
}

// Forward grid: column tiles times row tiles, column tile fastest. The block's waves sit
// side by side across as many columns as the row can fill without idling more than 1/8 of its
// lanes (all kFwdWaves when B*H is large), and stack along the rows otherwise.
struct FwdPlan {
    int64_t n_ct, n_rt, rows, cols;
    int cw, cw_log2;
};

FwdPlan make_fwd_plan(int64_t S, int64_t B, int64_t H) {
    const int64_t C = B * H, wave_cols = kWave * kFwdVec;
    FwdPlan f;
    f.cw = 1;
    for (int cw = kFwdWaves; cw >= 1; cw /= 2) {
        const int64_t span = cw * wave_cols;
        const int64_t waste = (C + span - 1) / span * span - C;
        if (waste * 8 <= C) {
            f.cw = cw;
            break;
        }
    }
    f.cw_log2 = 0;
    while ((1 << f.cw_log2) < f.cw) ++f.cw_log2;
    f.cols = f.cw * wave_cols;
    f.rows = (int64_t)(kFwdWaves / f.cw) * kFwdRows;
    f.n_ct = (C + f.cols - 1) / f.cols;
    f.n_rt = (S + f.rows - 1) / f.rows;
    return f;
}

template <int DT>
hipError_t launch_fwd(int64_t S, int64_t B, int64_t H, int W, const void *x, const void *w,
                      const uint8_t *mask, void *y, hipStream_t st, const InStrides &is,
                      bool strided) {
    const FwdPlan f = make_fwd_plan(S, B, H);
    const dim3 grid((unsigned)(f.n_ct * f.n_rt));
    const dim3 block(kFwdWaves * kWave);
#define MCCB_FWD(M, T, TAPS)                                                                      \
    hipLaunchKernelGGL((mccb_fwd<DT, M, T, TAPS>), grid, block, MCCB_FWD_LDS, st,                \
                       (const fvec_t *)x, (const fvec_t *)w, mask, (fvec_t *)y, S, B, H, f.n_ct,  \
                       f.cw_log2, is)
#define MCCB_FWD_W(TAPS)                                                                          \
    if (mask) {                                                                                   \
        if (strided) MCCB_FWD(true, true, TAPS); else MCCB_FWD(true, false, TAPS);                \
    } else {                                                                                      \
        if (strided) MCCB_FWD(false, true, TAPS); else MCCB_FWD(false, false, TAPS);              \
    }
    switch (W) {
        case 1: MCCB_FWD_W(1); break;
        case 2: MCCB_FWD_W(2); break;
        case 3: MCCB_FWD_W(3); break;
        case 4: MCCB_FWD_W(4); break;
        default: return hipErrorInvalidValue;
    }
#undef MCCB_FWD_W
#undef MCCB_FWD
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Strided inputs. A 3-D input is read in place when its channels are contiguous and its row and
// batch strides and base keep every lane's vector load aligned; otherwise it is first packed into
// a contiguous copy in the workspace (after the gradWeight partials, 256-byte aligned). A
// non-contiguous weight is always packed (3*H elements). The mask is always read in place.
// ---------------------------------------------------------------------------------------------
struct View3 {
    const void *p;
    int64_t s0, s1, s2;  // element strides along S, B, H
};

// `span_limit`: if > 0, the lane-relative byte offset ((batches a block spans - 1) * batch
// stride + H) * 2 must stay below it (the backward kernel keeps it in 32 bits).
bool inplace3(const View3 &v, int vec, int64_t H, uint64_t span_limit) {
    if (!(v.s2 == 1 && v.s0 % vec == 0 && v.s1 % vec == 0 &&
          ((uintptr_t)v.p % (uintptr_t)(vec * 2)) == 0))
        return false;
    if (span_limit == 0) return true;
    const int64_t extra_batches = (kMaxGroupCols - 1) / H + 1;  // j - (wave's first batch), at most
    const unsigned __int128 rel = ((unsigned __int128)extra_batches * (uint64_t)v.s1 + (uint64_t)H) * 2u;
    return rel < span_limit;
}

// Bytes from the base to one past the last element, or 0 if that does not fit in 2^62.
uint64_t extent_bytes(int64_t n0, int64_t s0, int64_t n1, int64_t s1, int64_t n2, int64_t s2,
                      int64_t esz) {
    unsigned __int128 last = (unsigned __int128)(n0 - 1) * (uint64_t)s0 +
                             (unsigned __int128)(n1 - 1) * (uint64_t)s1 +
                             (unsigned __int128)(n2 - 1) * (uint64_t)s2;
    unsigned __int128 bytes = (last + 1) * (uint64_t)esz;
    return bytes >> 62 ? 0 : (uint64_t)bytes;
}

uint64_t align256(uint64_t v) { return (v + 255u) & ~(uint64_t)255u; }

constexpr uint64_t kLaneSpan = (uint64_t)1 << 32;  // backward lane offsets are 32-bit

struct ExLayout {
    bool pack_gy = false, pack_x = false, pack_w = false;
    uint64_t gy_off = 0, x_off = 0, w_off = 0, total = 0;
};

// Workspace layout: `base` bytes of the kernels' own scratch, then the packed copies needed.
ExLayout ex_layout(uint64_t base, int64_t S, int64_t B, int64_t H, int64_t W, const View3 *gy,
                   const View3 &x, const void *w, int64_t w0, int64_t w1, int vec,
                   uint64_t span_limit) {
    ExLayout L;
    const uint64_t nb = (uint64_t)(S * B * H) * 2u;
    uint64_t off = base;
    if (gy && !inplace3(*gy, vec, H, span_limit)) {
        L.pack_gy = true;
        L.gy_off = off = align256(off);
        off += nb;
    }
    if (!inplace3(x, vec, H, span_limit)) {
        L.pack_x = true;
        L.x_off = off = align256(off);
        off += nb;
    }
    if (!(w0 == H && w1 == 1 && ((uintptr_t)w & 15u) == 0)) {
        L.pack_w = true;
        L.w_off = off = align256(off);
        off += (uint64_t)(W * H) * 2u;
    }
    L.total = off;
    return L;
}

hipError_t pack3(const void *src, void *dst, int64_t R0, int64_t R1, int64_t H, int64_t s0,
                 int64_t s1, int64_t s2, hipStream_t st) {
    hipLaunchKernelGGL(mccb_pack, dim3((unsigned)(R0 * R1)), dim3(256), 0, st,
                       (const uint16_t *)src, (uint32_t *)dst, R1, H, s0, s1, s2);
    return hipGetLastError();
}

// Validated strided arguments shared by the _ex entry points.
struct ExArgs {
    View3 gy{}, x{};
    int64_t w0 = 0, w1 = 0, m0 = 0, m1 = 0;  // weight (tap, H) and mask (B, S) strides
    uint64_t gy_ext = 0, x_ext = 0, w_ext = 0, m_ext = 0;
};

// Fills `a` from the strides (NULL = contiguous) and checks them: non-negative, element-aligned
// bases, extents that fit. `gy` may be NULL (forward).
int check_strided(const void *gy, const void *x, const void *w, const uint8_t *mask, int64_t S,
                  int64_t B, int64_t H, int64_t W, const mccb_strides_t *sp, ExArgs &a) {
    const int64_t C = B * H;
    a.gy = View3{gy, C, H, 1};
    a.x = View3{x, C, H, 1};
    a.w0 = H, a.w1 = 1, a.m0 = S, a.m1 = 1;
    if (sp) {
        a.gy = View3{gy, sp->gradY[0], sp->gradY[1], sp->gradY[2]};
        a.x = View3{x, sp->x[0], sp->x[1], sp->x[2]};
        a.w0 = sp->weight[0], a.w1 = sp->weight[1], a.m0 = sp->mask[0], a.m1 = sp->mask[1];
    }
    const int64_t all[10] = {a.gy.s0, a.gy.s1, a.gy.s2, a.x.s0, a.x.s1, a.x.s2, a.w0, a.w1, a.m0, a.m1};
    for (int64_t v : all)
        if (v < 0) return MCCB_ERR_PARAM_INVALID;
    if ((gy && ((uintptr_t)gy & 1u)) || ((uintptr_t)x & 1u) || ((uintptr_t)w & 1u))
        return MCCB_ERR_PARAM_INVALID;
    a.gy_ext = gy ? extent_bytes(S, a.gy.s0, B, a.gy.s1, H, a.gy.s2, 2) : 0;
    a.x_ext = extent_bytes(S, a.x.s0, B, a.x.s1, H, a.x.s2, 2);
    a.w_ext = extent_bytes(W, a.w0, 1, 0, H, a.w1, 2);
    a.m_ext = mask ? extent_bytes(B, a.m0, S, a.m1, 1, 0, 1) : 0;
    if ((gy && !a.gy_ext) || !a.x_ext || !a.w_ext || (mask && !a.m_ext)) return MCCB_ERR_PARAM_INVALID;
    return MCCB_OK;
}

// No output (nor the workspace) may overlap another buffer.
bool any_overlap(const void *const *bufs, const uint64_t *lens, int n, int first_output) {
    for (int o = first_output; o < n; ++o) {
        if (!bufs[o] || lens[o] == 0) continue;
        for (int t = 0; t < n; ++t) {
            if (t == o || !bufs[t] || lens[t] == 0) continue;
            if (overlaps(bufs[o], lens[o], bufs[t], lens[t])) return true;
        }
    }
    return false;
}

// Packed variable-length layout: the backward and forward run with B = 1, S = T, after the
// per-token limits are computed into the workspace.
template <int DT>
hipError_t launch_varlen_bwd(const Plan &p, const void *gy, const void *x, const void *w,
                             const uint8_t *mask, const int64_t *cu, int64_t nseq, void *gx,
                             void *gw, void *ws, uint64_t lim_off, hipStream_t st) {
    uint8_t *ahead = (uint8_t *)ws + lim_off;
    const int64_t T = p.S;
    hipLaunchKernelGGL(mccb_seg_limits, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, st, cu,
                       nseq, T, ahead, (uint8_t *)nullptr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int span = (int)(p.rows_per_strip + p.W - 1);
    const int lim_lds = mask ? (int)p.mask_lds : 0;
    const size_t lds = (size_t)lim_lds + (size_t)span;
    const InStrides is{p.H, p.H, p.H, p.H, T, 1};
    e = launch_fused_any<DT, true>(p, gy, x, w, mask, gx, ws, st, lds, is, false, ahead, lim_lds,
                                   p.direct ? gw : nullptr);
    if (e != hipSuccess || p.direct) return e;
    const dim3 grid2((unsigned)((p.H + kReduceCols - 1) / kReduceCols), (unsigned)p.W);
    const dim3 block2(kReduceWaves * kWave);
    hipLaunchKernelGGL((mccb_gw_reduce<DT>), grid2, block2, 0, st, (const double *)ws,
                       (uint16_t *)gw, p.n_strips, p.B, p.H);
    return hipGetLastError();
}

template <int DT>
hipError_t launch_varlen_fwd(int64_t T, int64_t H, int W, const void *x, const void *w,
                             const uint8_t *mask, const int64_t *cu, int64_t nseq, void *y,
                             void *ws, uint64_t behind_off, hipStream_t st) {
    uint8_t *ahead = (uint8_t *)ws, *behind = (uint8_t *)ws + behind_off;
    hipLaunchKernelGGL(mccb_seg_limits, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, st, cu,
                       nseq, T, ahead, behind);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const FwdPlan f = make_fwd_plan(T, 1, H);
    const dim3 grid((unsigned)(f.n_ct * f.n_rt));
    const dim3 block(kFwdWaves * kWave);
    const InStrides is{H, H, H, H, T, 1};
#define MCCB_VLF(M, TAPS)                                                                         \
    hipLaunchKernelGGL((mccb_fwd<DT, M, false, TAPS, true>), grid, block, MCCB_FWD_LDS, st,      \
                       (const fvec_t *)x, (const fvec_t *)w, mask, (fvec_t *)y, T, (int64_t)1, H, \
                       f.n_ct, f.cw_log2, is, behind)
#define MCCB_VLF_W(TAPS)                                                                          \
    if (mask) MCCB_VLF(true, TAPS); else MCCB_VLF(false, TAPS);
    switch (W) {
        case 1: MCCB_VLF_W(1); break;
        case 2: MCCB_VLF_W(2); break;
        case 3: MCCB_VLF_W(3); break;
        case 4: MCCB_VLF_W(4); break;
        default: return hipErrorInvalidValue;
    }
#undef MCCB_VLF_W
#undef MCCB_VLF
    return hipGetLastError();
}

// Workspace of the packed layout: [fp64 partials][per-token limits], or for the forward
// [ahead][behind]; each part 256-byte aligned.
struct VarlenLayout {
    uint64_t lim_off, total;
};

VarlenLayout varlen_bwd_layout(const Plan &p) {
    VarlenLayout v;
    v.lim_off = align256(p.ws_bytes);
    v.total = v.lim_off + (uint64_t)p.S;
    return v;
}

VarlenLayout varlen_fwd_layout(int64_t T) {
    VarlenLayout v;
    v.lim_off = align256((uint64_t)T);  // behind[]
    v.total = v.lim_off + (uint64_t)T;
    return v;
}

int check_varlen(int64_t T, int64_t nseq, int64_t H, int64_t W, int dtype) {
    int rc = check_shape(T, 1, H, dtype);  // T tokens in [1, 524288], H as usual
    if (rc == MCCB_OK) rc = check_taps(W);
    if (rc == MCCB_OK && (nseq < 1 || nseq > kMaxBS)) rc = MCCB_ERR_SHAPE;
    return rc;
}

// Alignment and overlap checks of the contiguous 3-tap backward (after the entry point's pointer,
// shape and workspace-size checks). `workspace` may be nullptr when the call brings none.
int check_contiguous(const Plan &p, const void *gradY, const void *x, const void *weight,
                     const uint8_t *mask, const void *gradX, const void *gradWeight,
                     const void *workspace) {
    const int64_t S = p.S, B = p.B, H = p.H;
    if (!aligned16(gradY) || !aligned16(x) || !aligned16(weight) || !aligned16(gradX) ||
        !aligned16(gradWeight) || (workspace && p.ws_bytes > 0 && !aligned16(workspace)))
        return MCCB_ERR_PARAM_INVALID;
    const uint64_t nb = (uint64_t)(S * B * H) * 2u, wb = (uint64_t)(3 * H) * 2u;
    const uint64_t mb = mask ? (uint64_t)(B * S) : 0u;
    // No output (nor the workspace) may overlap any other buffer; in particular gradX cannot
    // alias gradY, whose rows the stencil reads ahead of the rows it writes.
    const void *bufs[7] = {gradY, x, weight, mask, gradX, gradWeight, workspace};
    const uint64_t lens[7] = {nb, nb, wb, mb, nb, wb, workspace ? p.ws_bytes : 0u};
    if (any_overlap(bufs, lens, 7, 4)) return MCCB_ERR_PARAM_INVALID;
    return MCCB_OK;
}

// Enqueues the two kernels of the contiguous 3-tap backward on `stream`; `workspace` holds at
// least p.ws_bytes.
int launch_contiguous(const Plan &p, const void *gradY, const void *x, const void *weight,
                      const uint8_t *mask, void *gradX, void *gradWeight, void *workspace,
                      void *stream) {
    hipStream_t st = (hipStream_t)stream;
    hipEvent_t *ev = nullptr;
    {
        std::lock_guard<std::mutex> lk(g_prof.mu);
        if (g_prof.on && g_prof.n < g_prof.cap) ev = &g_prof.ev[3 * (size_t)g_prof.n++];
    }
    const InStrides is{p.B * p.H, p.H, p.B * p.H, p.H, p.S, 1};
    const hipError_t e =
        (p.dtype == MCCB_BF16)
            ? launch<MCCB_BF16>(p, gradY, x, weight, mask, gradX, gradWeight, workspace, st, ev,
                                is, false)
            : launch<MCCB_FP16>(p, gradY, x, weight, mask, gradX, gradWeight, workspace, st, ev,
                                is, false);
    return e == hipSuccess ? MCCB_OK : MCCB_ERR_RUNTIME;
}

// ---------------------------------------------------------------------------------------------
// Fixed scratch of mccb_backward_noalloc: the gradWeight partials live in `scratch`, a device
// array of the library's code object (each device the library runs on holds its own copy until
// the process ends), instead of a caller's workspace. In host code `scratch` names only a host
// stand-in for the symbol; its device address, which differs per device, comes from
// hipGetSymbolAddress, looked up once per device with that device current, and only that address
// reaches a kernel. Every call on one device shares its copy; the fused kernel overwrites every
// partial the reduction reads, so nothing needs clearing between calls.
// ---------------------------------------------------------------------------------------------
constexpr int kMaxDevices = 64;
struct ScratchTable {
    std::mutex mu;
    void *ptr[kMaxDevices] = {};
} g_scratch;

// Device address of `scratch` on the device that runs `stream` (the current device for the null
// stream), or nullptr if a HIP call fails.
void *scratch_on(hipStream_t stream) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return nullptr;
    int dev = cur;
    if (stream) {
        hipDevice_t d = 0;
        if (hipStreamGetDevice(stream, &d) != hipSuccess) return nullptr;
        dev = (int)d;
    }
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lk(g_scratch.mu);
    if (!g_scratch.ptr[dev]) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess) return nullptr;
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur && hipSetDevice(cur) != hipSuccess) return nullptr;
        if (e != hipSuccess || !p) return nullptr;
        g_scratch.ptr[dev] = p;
    }
    return g_scratch.ptr[dev];
}

// The fused kernel's block shape for a layout (the contiguous 3-tap launch).
template <int LAYOUT>
void fill_plan(const Plan &p, mccb_plan_t *plan) {
    typedef FusedCfg<3, false, LAYOUT> Cfg;
    plan->rows_per_round = Cfg::RR;
    plan->cols_per_block = Cfg::CG * Cfg::GC;
    plan->n_col_blocks = fused_grid<3, false, LAYOUT>(p.C).ncb;
    plan->waves_per_block = Cfg::BW;
    plan->group_spacing = Cfg::DLV * Cfg::V * 2;
}

}  // namespace

extern "C" {

int mccb_get_workspace_size(int64_t S, int64_t B, int64_t H, int dtype, uint64_t *workspace_size) {
    if (!workspace_size) return MCCB_ERR_PARAM_NULLPTR;
    const int rc = check_shape(S, B, H, dtype);
    if (rc != MCCB_OK) return rc;
    *workspace_size = make_plan(S, B, H, dtype).ws_bytes;
    return MCCB_OK;
}

int mccb_get_plan(int64_t S, int64_t B, int64_t H, int dtype, mccb_plan_t *plan) {
    if (!plan) return MCCB_ERR_PARAM_NULLPTR;
    const int rc = check_shape(S, B, H, dtype);
    if (rc != MCCB_OK) return rc;
    const Plan p = make_plan(S, B, H, dtype);
    const int layout = fused_layout(p, false, false);  // the contiguous 3-tap launch
    plan->rows_per_turn = kTurnRows;
    plan->rows_per_strip = p.rows_per_strip;
    plan->n_strips = p.n_strips;
    switch (layout) {
        case kLayoutTall: fill_plan<kLayoutTall>(p, plan); break;
        case kLayoutWide: fill_plan<kLayoutWide>(p, plan); break;
        case kLayoutWide4x32: fill_plan<kLayoutWide4x32>(p, plan); break;
        case kLayoutWide3x32: fill_plan<kLayoutWide3x32>(p, plan); break;
        case kLayoutNarrowRing: fill_plan<kLayoutNarrowRing>(p, plan); break;
        default: fill_plan<kLayoutRing>(p, plan); break;
    }
    plan->workspace_size = p.ws_bytes;
    const FwdPlan f = make_fwd_plan(S, B, H);
    plan->fwd_rows_per_tile = f.rows;
    plan->fwd_cols_per_tile = f.cols;
    plan->fwd_n_col_tiles = f.n_ct;
    plan->fwd_n_row_tiles = f.n_rt;
    return MCCB_OK;
}

int mccb_backward(const void *gradY, const void *x, const void *weight, const uint8_t *mask,
                  void *gradX, void *gradWeight, int64_t S, int64_t B, int64_t H, int dtype,
                  void *workspace, uint64_t workspace_size, void *stream) {
    if (!gradY || !x || !weight || !gradX || !gradWeight) return MCCB_ERR_PARAM_NULLPTR;
    const int rc = check_shape(S, B, H, dtype);
    if (rc != MCCB_OK) return rc;
    const Plan p = make_plan(S, B, H, dtype);
    if (p.ws_bytes > 0 && !workspace) return MCCB_ERR_PARAM_NULLPTR;
    if (workspace_size < p.ws_bytes) return MCCB_ERR_PARAM_INVALID;
    const int vr = check_contiguous(p, gradY, x, weight, mask, gradX, gradWeight,
                                    p.ws_bytes > 0 ? workspace : nullptr);
    if (vr != MCCB_OK) return vr;
    return launch_contiguous(p, gradY, x, weight, mask, gradX, gradWeight, workspace, stream);
}

int mccb_backward_noalloc(const void *gradY, const void *x, const void *weight,
                          const uint8_t *mask, void *gradX, void *gradWeight, int64_t S,
                          int64_t B, int64_t H, int dtype, void *stream) {
    if (!gradY || !x || !weight || !gradX || !gradWeight) return MCCB_ERR_PARAM_NULLPTR;
    const int rc = check_shape(S, B, H, dtype);
    if (rc != MCCB_OK) return rc;
    const Plan p = make_plan(S, B, H, dtype);
    if (p.ws_bytes > kScratchBytes) return MCCB_ERR_SCRATCH_LIMIT;
    const int vr = check_contiguous(p, gradY, x, weight, mask, gradX, gradWeight, nullptr);
    if (vr != MCCB_OK) return vr;
    // validation done: the first HIP call comes here
    void *ws = nullptr;
    if (p.ws_bytes > 0) {
        ws = scratch_on((hipStream_t)stream);
        if (!ws) return MCCB_ERR_RUNTIME;
    }
    return launch_contiguous(p, gradY, x, weight, mask, gradX, gradWeight, ws, stream);
}

int mccb_forward(const void *x, const void *weight, const uint8_t *mask, void *y, int64_t S,
                 int64_t B, int64_t H, int dtype, void *stream) {
    if (!x || !weight || !y) return MCCB_ERR_PARAM_NULLPTR;
    const int rc = check_shape(S, B, H, dtype);
    if (rc != MCCB_OK) return rc;
    if (!aligned16(x) || !aligned16(weight) || !aligned16(y)) return MCCB_ERR_PARAM_INVALID;
    const uint64_t nb = (uint64_t)(S * B * H) * 2u, wb = (uint64_t)(3 * H) * 2u;
    const uint64_t mb = mask ? (uint64_t)(B * S) : 0u;
    // y must not overlap any input: a tile reads rows of x that other tiles write in y.
    if (overlaps(y, nb, x, nb) || overlaps(y, nb, weight, wb) || (mask && overlaps(y, nb, mask, mb)))
        return MCCB_ERR_PARAM_INVALID;
    hipStream_t st = (hipStream_t)stream;
    const InStrides is{B * H, H, B * H, H, S, 1};
    const hipError_t e = (dtype == MCCB_BF16)
                             ? launch_fwd<MCCB_BF16>(S, B, H, 3, x, weight, mask, y, st, is, false)
                             : launch_fwd<MCCB_FP16>(S, B, H, 3, x, weight, mask, y, st, is, false);
    return e == hipSuccess ? MCCB_OK : MCCB_ERR_RUNTIME;
}

int mccb_get_workspace_size_ex(const void *gradY, const void *x, const void *weight, int64_t S,
                               int64_t B, int64_t H, int64_t W, int dtype,
                               const mccb_strides_t *strides, uint64_t *workspace_size) {
    if (!gradY || !x || !weight || !workspace_size) return MCCB_ERR_PARAM_NULLPTR;
    int rc = check_shape(S, B, H, dtype);
    if (rc == MCCB_OK) rc = check_taps(W);
    if (rc != MCCB_OK) return rc;
    ExArgs a;
    rc = check_strided(gradY, x, weight, nullptr, S, B, H, W, strides, a);
    if (rc != MCCB_OK) return rc;
    const Plan p = make_plan(S, B, H, dtype, (int)W);
    *workspace_size =
        ex_layout(p.ws_bytes, S, B, H, W, &a.gy, a.x, weight, a.w0, a.w1, fused_vec(S, B * H, W), kLaneSpan).total;
    return MCCB_OK;
}

int mccb_backward_ex(const void *gradY, const void *x, const void *weight, const uint8_t *mask,
                     void *gradX, void *gradWeight, int64_t S, int64_t B, int64_t H, int64_t W,
                     int dtype, const mccb_strides_t *strides, void *workspace,
                     uint64_t workspace_size, void *stream) {
    if (!gradY || !x || !weight || !gradX || !gradWeight) return MCCB_ERR_PARAM_NULLPTR;
    int rc = check_shape(S, B, H, dtype);
    if (rc == MCCB_OK) rc = check_taps(W);
    if (rc != MCCB_OK) return rc;
    ExArgs a;
    rc = check_strided(gradY, x, weight, mask, S, B, H, W, strides, a);
    if (rc != MCCB_OK) return rc;
    const Plan p = make_plan(S, B, H, dtype, (int)W);
    const ExLayout L =
        ex_layout(p.ws_bytes, S, B, H, W, &a.gy, a.x, weight, a.w0, a.w1, fused_vec(S, B * H, W), kLaneSpan);
    if (L.total > 0 && !workspace) return MCCB_ERR_PARAM_NULLPTR;
    if (workspace_size < L.total) return MCCB_ERR_PARAM_INVALID;
    if (!aligned16(gradX) || !aligned16(gradWeight) || (L.total > 0 && !aligned16(workspace)))
        return MCCB_ERR_PARAM_INVALID;
    const uint64_t nb = (uint64_t)(S * B * H) * 2u, wb = (uint64_t)(W * H) * 2u;
    const void *bufs[7] = {gradY, x, weight, mask, gradX, gradWeight, workspace};
    const uint64_t lens[7] = {a.gy_ext, a.x_ext, a.w_ext, a.m_ext, nb, wb, L.total};
    if (any_overlap(bufs, lens, 7, 4)) return MCCB_ERR_PARAM_INVALID;

    hipStream_t st = (hipStream_t)stream;
    char *wsb = (char *)workspace;
    const int64_t C = B * H;
    const void *gy_eff = gradY, *x_eff = x, *w_eff = weight;
    InStrides is{a.gy.s0, a.gy.s1, a.x.s0, a.x.s1, a.m0, a.m1};
    if (L.pack_gy) {
        if (pack3(gradY, wsb + L.gy_off, S, B, H, a.gy.s0, a.gy.s1, a.gy.s2, st) != hipSuccess)
            return MCCB_ERR_RUNTIME;
        gy_eff = wsb + L.gy_off, is.gy_row = C, is.gy_batch = H;
    }
    if (L.pack_x) {
        if (pack3(x, wsb + L.x_off, S, B, H, a.x.s0, a.x.s1, a.x.s2, st) != hipSuccess)
            return MCCB_ERR_RUNTIME;
        x_eff = wsb + L.x_off, is.x_row = C, is.x_batch = H;
    }
    if (L.pack_w) {
        if (pack3(weight, wsb + L.w_off, W, 1, H, a.w0, 0, a.w1, st) != hipSuccess)
            return MCCB_ERR_RUNTIME;
        w_eff = wsb + L.w_off;
    }
    const bool strided = !(is.gy_row == C && is.gy_batch == H && is.x_row == C && is.x_batch == H);
    hipEvent_t *ev = nullptr;
    {
        std::lock_guard<std::mutex> lk(g_prof.mu);
        if (g_prof.on && g_prof.n < g_prof.cap) ev = &g_prof.ev[3 * (size_t)g_prof.n++];
    }
    const hipError_t e =
        (dtype == MCCB_BF16)
            ? launch<MCCB_BF16>(p, gy_eff, x_eff, w_eff, mask, gradX, gradWeight, workspace, st, ev,
                                is, strided)
            : launch<MCCB_FP16>(p, gy_eff, x_eff, w_eff, mask, gradX, gradWeight, workspace, st, ev,
                                is, strided);
    return e == hipSuccess ? MCCB_OK : MCCB_ERR_RUNTIME;
}

int mccb_forward_get_workspace_size_ex(const void *x, const void *weight, int64_t S, int64_t B,
                                       int64_t H, int64_t W, int dtype,
                                       const mccb_strides_t *strides, uint64_t *workspace_size) {
    if (!x || !weight || !workspace_size) return MCCB_ERR_PARAM_NULLPTR;
    int rc = check_shape(S, B, H, dtype);
    if (rc == MCCB_OK) rc = check_taps(W);
    if (rc != MCCB_OK) return rc;
    ExArgs a;
    rc = check_strided(nullptr, x, weight, nullptr, S, B, H, W, strides, a);
    if (rc != MCCB_OK) return rc;
    *workspace_size = ex_layout(0, S, B, H, W, nullptr, a.x, weight, a.w0, a.w1, kFwdVec, 0).total;
    return MCCB_OK;
}

int mccb_forward_ex(const void *x, const void *weight, const uint8_t *mask, void *y, int64_t S,
                    int64_t B, int64_t H, int64_t W, int dtype, const mccb_strides_t *strides,
                    void *workspace, uint64_t workspace_size, void *stream) {
    if (!x || !weight || !y) return MCCB_ERR_PARAM_NULLPTR;
    int rc = check_shape(S, B, H, dtype);
    if (rc == MCCB_OK) rc = check_taps(W);
    if (rc != MCCB_OK) return rc;
    ExArgs a;
    rc = check_strided(nullptr, x, weight, mask, S, B, H, W, strides, a);
    if (rc != MCCB_OK) return rc;
    const ExLayout L = ex_layout(0, S, B, H, W, nullptr, a.x, weight, a.w0, a.w1, kFwdVec, 0);
    if (L.total > 0 && !workspace) return MCCB_ERR_PARAM_NULLPTR;
    if (workspace_size < L.total) return MCCB_ERR_PARAM_INVALID;
    if (!aligned16(y) || (L.total > 0 && !aligned16(workspace))) return MCCB_ERR_PARAM_INVALID;
    const uint64_t nb = (uint64_t)(S * B * H) * 2u;
    const void *bufs[5] = {x, weight, mask, y, L.total ? workspace : nullptr};
    const uint64_t lens[5] = {a.x_ext, a.w_ext, a.m_ext, nb, L.total};
    if (any_overlap(bufs, lens, 5, 3)) return MCCB_ERR_PARAM_INVALID;

    hipStream_t st = (hipStream_t)stream;
    char *wsb = (char *)workspace;
    const int64_t C = B * H;
    const void *x_eff = x, *w_eff = weight;
    InStrides is{C, H, a.x.s0, a.x.s1, a.m0, a.m1};
    if (L.pack_x) {
        if (pack3(x, wsb + L.x_off, S, B, H, a.x.s0, a.x.s1, a.x.s2, st) != hipSuccess)
            return MCCB_ERR_RUNTIME;
        x_eff = wsb + L.x_off, is.x_row = C, is.x_batch = H;
    }
    if (L.pack_w) {
        if (pack3(weight, wsb + L.w_off, W, 1, H, a.w0, 0, a.w1, st) != hipSuccess)
            return MCCB_ERR_RUNTIME;
        w_eff = wsb + L.w_off;
    }
    const bool strided = !(is.x_row == C && is.x_batch == H);
    const hipError_t e =
        (dtype == MCCB_BF16)
            ? launch_fwd<MCCB_BF16>(S, B, H, (int)W, x_eff, w_eff, mask, y, st, is, strided)
            : launch_fwd<MCCB_FP16>(S, B, H, (int)W, x_eff, w_eff, mask, y, st, is, strided);
    return e == hipSuccess ? MCCB_OK : MCCB_ERR_RUNTIME;
}

int mccb_varlen_get_workspace_size(int64_t T, int64_t nseq, int64_t H, int64_t W, int dtype,
                                   uint64_t *workspace_size) {
    if (!workspace_size) return MCCB_ERR_PARAM_NULLPTR;
    const int rc = check_varlen(T, nseq, H, W, dtype);
    if (rc != MCCB_OK) return rc;
    *workspace_size = varlen_bwd_layout(make_plan(T, 1, H, dtype, (int)W)).total;
    return MCCB_OK;
}

int mccb_varlen_backward(const void *gradY, const void *x, const void *weight, const uint8_t *mask,
                         const int64_t *cu_seqlens, void *gradX, void *gradWeight, int64_t T,
                         int64_t nseq, int64_t H, int64_t W, int dtype, void *workspace,
                         uint64_t workspace_size, void *stream) {
    if (!gradY || !x || !weight || !cu_seqlens || !gradX || !gradWeight)
        return MCCB_ERR_PARAM_NULLPTR;
    const int rc = check_varlen(T, nseq, H, W, dtype);
    if (rc != MCCB_OK) return rc;
    const Plan p = make_plan(T, 1, H, dtype, (int)W);
    const VarlenLayout L = varlen_bwd_layout(p);
    if (!workspace) return MCCB_ERR_PARAM_NULLPTR;
    if (workspace_size < L.total) return MCCB_ERR_PARAM_INVALID;
    if (!aligned16(gradY) || !aligned16(x) || !aligned16(weight) || !aligned16(gradX) ||
        !aligned16(gradWeight) || !aligned16(workspace) || ((uintptr_t)cu_seqlens & 7u))
        return MCCB_ERR_PARAM_INVALID;
    const uint64_t nb = (uint64_t)(T * H) * 2u, wb = (uint64_t)(W * H) * 2u;
    const void *bufs[8] = {gradY, x, weight, mask, cu_seqlens, gradX, gradWeight, workspace};
    const uint64_t lens[8] = {nb, nb, wb, mask ? (uint64_t)T : 0u, (uint64_t)nseq * 8u,
                              nb, wb, L.total};
    if (any_overlap(bufs, lens, 8, 5)) return MCCB_ERR_PARAM_INVALID;
    hipStream_t st = (hipStream_t)stream;
    const hipError_t e =
        (dtype == MCCB_BF16)
            ? launch_varlen_bwd<MCCB_BF16>(p, gradY, x, weight, mask, cu_seqlens, nseq, gradX,
                                           gradWeight, workspace, L.lim_off, st)
            : launch_varlen_bwd<MCCB_FP16>(p, gradY, x, weight, mask, cu_seqlens, nseq, gradX,
                                           gradWeight, workspace, L.lim_off, st);
    return e == hipSuccess ? MCCB_OK : MCCB_ERR_RUNTIME;
}

int mccb_varlen_forward_get_workspace_size(int64_t T, int64_t nseq, int64_t H, int64_t W,
                                           int dtype, uint64_t *workspace_size) {
    if (!workspace_size) return MCCB_ERR_PARAM_NULLPTR;
    const int rc = check_varlen(T, nseq, H, W, dtype);
    if (rc != MCCB_OK) return rc;
    *workspace_size = varlen_fwd_layout(T).total;
    return MCCB_OK;
}

int mccb_varlen_forward(const void *x, const void *weight, const uint8_t *mask,
                        const int64_t *cu_seqlens, void *y, int64_t T, int64_t nseq, int64_t H,
                        int64_t W, int dtype, void *workspace, uint64_t workspace_size,
                        void *stream) {
    if (!x || !weight || !cu_seqlens || !y) return MCCB_ERR_PARAM_NULLPTR;
    const int rc = check_varlen(T, nseq, H, W, dtype);
    if (rc != MCCB_OK) return rc;
    const VarlenLayout L = varlen_fwd_layout(T);
    if (!workspace) return MCCB_ERR_PARAM_NULLPTR;
    if (workspace_size < L.total) return MCCB_ERR_PARAM_INVALID;
    if (!aligned16(x) || !aligned16(weight) || !aligned16(y) || ((uintptr_t)cu_seqlens & 7u))
        return MCCB_ERR_PARAM_INVALID;
    const uint64_t nb = (uint64_t)(T * H) * 2u, wb = (uint64_t)(W * H) * 2u;
    const void *bufs[6] = {x, weight, mask, cu_seqlens, y, workspace};
    const uint64_t lens[6] = {nb, wb, mask ? (uint64_t)T : 0u, (uint64_t)nseq * 8u, nb, L.total};
    if (any_overlap(bufs, lens, 6, 4)) return MCCB_ERR_PARAM_INVALID;
    hipStream_t st = (hipStream_t)stream;
    const hipError_t e =
        (dtype == MCCB_BF16)
            ? launch_varlen_fwd<MCCB_BF16>(T, H, (int)W, x, weight, mask, cu_seqlens, nseq, y,
                                           workspace, L.lim_off, st)
            : launch_varlen_fwd<MCCB_FP16>(T, H, (int)W, x, weight, mask, cu_seqlens, nseq, y,
                                           workspace, L.lim_off, st);
    return e == hipSuccess ? MCCB_OK : MCCB_ERR_RUNTIME;
}

const char *mccb_status_string(int status) {
    switch (status) {
        case MCCB_OK: return "MCCB_OK";
        case MCCB_ERR_PARAM_NULLPTR: return "MCCB_ERR_PARAM_NULLPTR: a required pointer is NULL";
        case MCCB_ERR_PARAM_INVALID:
            return "MCCB_ERR_PARAM_INVALID: bad dtype, alignment, overlap or workspace size";
        case MCCB_ERR_SHAPE: return "MCCB_ERR_SHAPE: shape outside the supported range";
        case MCCB_ERR_RUNTIME: return "MCCB_ERR_RUNTIME: HIP launch failed";
        case MCCB_ERR_SCRATCH_LIMIT:
            return "MCCB_ERR_SCRATCH_LIMIT: the shape needs more than the fixed scratch of "
                   "mccb_backward_noalloc (call mccb_backward with a workspace)";
        default: return "unknown mccb status";
    }
}

int mccb_profile_begin(int max_calls) {
    std::lock_guard<std::mutex> lk(g_prof.mu);
    for (hipEvent_t e : g_prof.ev)
        if (e) (void)hipEventDestroy(e);
    g_prof.on = false;
    g_prof.cap = g_prof.n = 0;
    g_prof.ev.assign(3 * (size_t)(max_calls > 0 ? max_calls : 0), nullptr);
    for (hipEvent_t &e : g_prof.ev)
        if (hipEventCreate(&e) != hipSuccess) return MCCB_ERR_RUNTIME;
    g_prof.cap = max_calls > 0 ? max_calls : 0;
    g_prof.on = true;
    return MCCB_OK;
}

int mccb_profile_end(double *fused_ms, double *reduce_ms, int *calls) {
    std::lock_guard<std::mutex> lk(g_prof.mu);
    double f = 0.0, r = 0.0;
    int rc = MCCB_OK;
    for (int c = 0; c < g_prof.n; ++c) {
        hipEvent_t *e = &g_prof.ev[3 * (size_t)c];
        float a = 0.f, b = 0.f;
        if (hipEventSynchronize(e[2]) != hipSuccess ||
            hipEventElapsedTime(&a, e[0], e[1]) != hipSuccess ||
            hipEventElapsedTime(&b, e[1], e[2]) != hipSuccess) {
            rc = MCCB_ERR_RUNTIME;
            break;
        }
        f += a;
        r += b;
    }
    if (fused_ms) *fused_ms = f;
    if (reduce_ms) *reduce_ms = r;
    if (calls) *calls = g_prof.n;
    for (hipEvent_t e : g_prof.ev)
        if (e) (void)hipEventDestroy(e);
    g_prof.ev.clear();
    g_prof.on = false;
    g_prof.cap = g_prof.n = 0;
    return rc;
}

}  // extern "C"
