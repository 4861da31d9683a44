/*
 * mccb.h -- masked causal depthwise conv1d backward on AMD Instinct MI355X (gfx950).
 *
 * The operation is the one documented on the page "aclnnMaskedCausalConv1dBackward" (Ascend CANN
 * aclnn operator), section 功能说明 (function description). With gradY, x and gradX of shape
 * [S,B,H], weight and gradWeight of shape [W=3,H] and an optional bool mask of shape [B,S]:
 *
 *   gradYMasked[i,j] = mask[j,i] * gradY[i,j]
 *   gradX[i,j]       = sum_{k=0}^{2} gradYMasked[i+k, j] * weight[2-k]
 *   gradWeight[k]    = sum_{j=0}^{B-1} sum_{i=0}^{S-1} gradYMasked[i+2-k, j] * x[i,j]
 *
 * Rows past the end (i' >= S) are zero. Every operation is independent per channel h (the
 * equations leave h implicit). The window W is fixed at 3 (constraints section), so the API has no
 * W argument.
 *
 * The interface keeps the page's two-phase shape (function prototype section): a first call that
 * validates the arguments and reports the device workspace size, and a second call that enqueues
 * the computation on a stream. There is no executor object: the second call takes the tensors
 * again and re-validates them.
 *
 * Tensors are raw device pointers to contiguous row-major storage:
 *   gradY, x, gradX : [S,B,H], element (i,j,h) at (i*B + j)*H + h
 *   weight          : [3,H],   element (k,h)   at k*H + h
 *   gradWeight      : [3,H]
 *   mask            : [B,S] one byte per element, element (j,i) at j*S + i, nonzero = true (keep);
 *                     NULL means every position is kept (the page's default for the optional mask).
 * All five floating-point tensors share one dtype, bfloat16 or float16 (parameter table).
 *
 * Results: gradX is written once, correctly rounded (round to nearest, ties to even) from the exact
 * three-term sum. gradWeight is accumulated in fp64 and reduced in a fixed order, then rounded
 * once to the dtype, so repeated calls with the same inputs give bit-identical outputs
 * (constraints section: deterministic by default). Both outputs are overwritten, never accumulated.
 *
 * Preconditions that are NOT checked (constraints section): inputs contain no inf or NaN, and
 * neither inputs nor intermediate results exceed the range of the dtype.
 */
#ifndef MCCB_H
#define MCCB_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of gradY, x, weight, gradX and gradWeight (parameter table: BFLOAT16, FLOAT16). */
typedef enum { MCCB_BF16 = 0, MCCB_FP16 = 1 } mccb_dtype_t;

/* Status codes. The first three take the numbers of the page's return-code table (section 返回值)
 * for the same three error classes. */
enum {
    MCCB_OK = 0,
    /* a required pointer (input, output, out-parameter, or a workspace that is needed) is NULL */
    MCCB_ERR_PARAM_NULLPTR = 161001,
    /* dtype out of range, misaligned pointer, overlapping buffers, workspace too small */
    MCCB_ERR_PARAM_INVALID = 161002,
    /* shape out of the supported range: B in [1,32], S >= 1, B*S in [1, 524288],
     * H in [384, 24576] and H % 64 == 0 (constraints section) */
    MCCB_ERR_SHAPE = 561002,
    /* a HIP runtime call or kernel launch failed (the page names no code for this) */
    MCCB_ERR_RUNTIME = -1,
    /* mccb_backward_noalloc: the shape needs more workspace than its fixed scratch holds */
    MCCB_ERR_SCRATCH_LIMIT = -2
};

/*
 * Phase 1 (the page's ...GetWorkspaceSize). Validates the shape and dtype and stores in
 * *workspace_size the number of device bytes the caller must provide to mccb_backward for this
 * (S, B, H, dtype). The size depends on nothing else. Host-only; makes no HIP call.
 * Returns MCCB_OK, MCCB_ERR_PARAM_NULLPTR (workspace_size NULL), MCCB_ERR_PARAM_INVALID (dtype)
 * or MCCB_ERR_SHAPE.
 */
int mccb_get_workspace_size(int64_t S, int64_t B, int64_t H, int dtype, uint64_t *workspace_size);

/*
 * Phase 2 (the page's second call). Enqueues the backward on `stream` (a hipStream_t; NULL = the
 * default stream) and returns without waiting; the caller synchronizes the stream before reading
 * gradX or gradWeight.
 *
 *   gradY, x, weight : inputs, device memory, 16-byte aligned, not modified
 *   mask             : optional input, device memory, any alignment, or NULL (= all true)
 *   gradX, gradWeight: outputs, device memory, 16-byte aligned, overwritten
 *   workspace        : device scratch of at least the phase-1 size, 16-byte aligned, owned by the
 *                      caller (may be NULL only when the phase-1 size is 0). Its contents need no
 *                      initialisation and are meaningless afterwards. It must not be used by
 *                      another call that is in flight at the same time.
 *
 * The library allocates nothing and keeps no state between calls (apart from the optional
 * profiling record below). gradX must not overlap gradY or x; no output or the workspace may
 * overlap any other buffer.
 *
 * Validation happens on the host before any HIP call, in this order: NULL pointers
 * (MCCB_ERR_PARAM_NULLPTR), dtype (MCCB_ERR_PARAM_INVALID), shape (MCCB_ERR_SHAPE), workspace,
 * alignment and overlap (MCCB_ERR_PARAM_INVALID / MCCB_ERR_PARAM_NULLPTR). On any error nothing is
 * enqueued. MCCB_ERR_RUNTIME reports a failed kernel launch.
 */
int mccb_backward(const void *gradY, const void *x, const void *weight, const uint8_t *mask,
                  void *gradX, void *gradWeight, int64_t S, int64_t B, int64_t H, int dtype,
                  void *workspace, uint64_t workspace_size, void *stream);

/*
 * mccb_backward for callers that cannot allocate device memory: code recorded under HIP graph
 * capture, serving loops and harnesses that forbid hipMalloc. Same arguments, results (bit for
 * bit), validation and error codes as mccb_backward, without the workspace: the gradWeight
 * partials go to a fixed scratch array of MCCB_NOALLOC_SCRATCH_BYTES that the library's device
 * code holds on every device it runs on (allocated when the library's code is loaded on that
 * device, kept until the process ends). This call allocates nothing: no hipMalloc, no hipFree.
 *
 * A shape whose workspace (mccb_get_workspace_size) exceeds MCCB_NOALLOC_SCRATCH_BYTES returns
 * MCCB_ERR_SCRATCH_LIMIT and enqueues nothing (S=16384 B=32 H=5120 needs 62,914,560 bytes and
 * fits; S=262144 B=2 H=24576 needs 301,989,888 and does not). The scratch needs no clearing: every
 * call overwrites the part it reads. All calls on one device share that device's scratch, so two
 * calls that can run at the same time on one device (on different streams, or from different
 * threads without ordering) race and give wrong gradWeight; calls ordered on one stream do not.
 * The kernels run on the device of `stream` (NULL = the current device's default stream). The
 * first call on a device also looks up the scratch address there (hipGetSymbolAddress), so that
 * call must not itself be under graph capture; MCCB_ERR_RUNTIME if the lookup fails.
 */
#define MCCB_NOALLOC_SCRATCH_BYTES (64ull << 20)
int mccb_backward_noalloc(const void *gradY, const void *x, const void *weight,
                          const uint8_t *mask, void *gradX, void *gradWeight, int64_t S,
                          int64_t B, int64_t H, int dtype, void *stream);

/*
 * The forward operation whose gradients mccb_backward computes: the masked causal depthwise
 * convolution named beside the backward on the same page (the MaskedCausalConv1d operator),
 *
 *   y[i,j] = mask[j,i] * sum_{k=0}^{2} weight[k] * x[i-2+k, j]      (x rows < 0 are zero),
 *
 * per channel h, i.e. the operator whose adjoint in x is the gradX equation above and whose
 * derivative in weight is the gradWeight equation. The page documents only the backward; this
 * reading of the forward is the one its three equations imply.
 *
 *   x      : input [S,B,H], device memory, 16-byte aligned, not modified
 *   weight : input [3,H], device memory, 16-byte aligned
 *   mask   : optional [B,S] bytes as for mccb_backward (NULL = all true); masked outputs are 0
 *   y      : output [S,B,H], device memory, 16-byte aligned, overwritten; must not overlap x,
 *            weight or mask
 *
 * Each output is the exact three-term sum rounded once to nearest-even in the dtype. Same shape
 * limits and error codes as mccb_backward; needs no workspace. Enqueues on `stream` (NULL = the
 * default stream) and returns without waiting; MCCB_ERR_RUNTIME reports a failed launch.
 */
int mccb_forward(const void *x, const void *weight, const uint8_t *mask, void *y, int64_t S,
                 int64_t B, int64_t H, int dtype, void *stream);

/*
 * Strided (non-contiguous) inputs. The parameter table marks gradY, x, weight and mask as
 * accepting non-contiguous tensors; the outputs gradX, gradWeight (and the forward's y) stay
 * contiguous. Strides are in elements and >= 0 (0 repeats an element, e.g. a broadcast batch).
 * Contiguous values: gradY and x {B*H, H, 1}, weight {H, 1}, mask {S, 1}.
 */
typedef struct {
    int64_t gradY[3];  /* along S, B, H */
    int64_t x[3];      /* along S, B, H */
    int64_t weight[2]; /* along the tap k, then H */
    int64_t mask[2];   /* along B, then S */
} mccb_strides_t;

/*
 * Extended calls: strided inputs and a window of W taps.
 *
 * W: the weight and gradWeight are [W,H]; the equations of the function description with 2 (and
 * the forward's look-back) replaced by W-1. The constraints section supports only W = 3 "for
 * now"; the kernels here take W = 1..4 (other values: MCCB_ERR_SHAPE). W = 3 with NULL strides is
 * exactly mccb_get_workspace_size / mccb_backward / mccb_forward.
 *
 * Strides (NULL = all contiguous): the backward reads gradY or x in place when its channels are
 * contiguous (H stride 1), its row and batch strides are multiples of the fused kernel's lane
 * width in elements, its base is aligned to the lane width in bytes, and a wave's columns span
 * less than 4 GiB of it. The lane width is 8 bytes (4 elements) on shapes with S > 64 and B*H at
 * least 32768 and a multiple of 4096, and 4 bytes (2 elements) on all others. Any other gradY or x is first
 * packed into a contiguous copy inside the workspace (one extra read and write of that tensor),
 * and a weight that is not contiguous and 16-byte aligned is packed too; phase 1 includes those
 * copies in the size it reports. The mask is read through its strides. Phase 1 therefore takes the input pointers as well (as the page's
 * phase 1 takes the tensors): they are inspected for alignment only, never dereferenced. Input
 * bases need 2-byte alignment; gradX, gradWeight and the workspace stay contiguous and 16-byte
 * aligned. Negative strides, or an input extent past 2^62 bytes, give MCCB_ERR_PARAM_INVALID; no
 * output or the workspace may overlap any input's extent. Otherwise as mccb_get_workspace_size /
 * mccb_backward.
 */
int mccb_get_workspace_size_ex(const void *gradY, const void *x, const void *weight, int64_t S,
                               int64_t B, int64_t H, int64_t W, int dtype,
                               const mccb_strides_t *strides, uint64_t *workspace_size);
int mccb_backward_ex(const void *gradY, const void *x, const void *weight, const uint8_t *mask,
                     void *gradX, void *gradWeight, int64_t S, int64_t B, int64_t H, int64_t W,
                     int dtype, const mccb_strides_t *strides, void *workspace,
                     uint64_t workspace_size, void *stream);

/*
 * mccb_forward with strided x, weight and mask (strides->gradY is ignored) and W taps:
 * y[i] = mask[j,i] * sum_{k=0}^{W-1} weight[k] * x[i-W+1+k]. x is read in place when its channels
 * are contiguous, its row and batch strides are multiples of 8 and its base is 16-byte aligned;
 * otherwise it (and a non-contiguous weight) is packed into the workspace, whose size phase 1
 * returns (0 when nothing needs packing; the workspace may then be NULL).
 */
int mccb_forward_get_workspace_size_ex(const void *x, const void *weight, int64_t S, int64_t B,
                                       int64_t H, int64_t W, int dtype,
                                       const mccb_strides_t *strides, uint64_t *workspace_size);
int mccb_forward_ex(const void *x, const void *weight, const uint8_t *mask, void *y, int64_t S,
                    int64_t B, int64_t H, int64_t W, int dtype, const mccb_strides_t *strides,
                    void *workspace, uint64_t workspace_size, void *stream);

/*
 * Packed variable-length layout (the TND convention of the sibling operators' pages: the tokens of
 * all sequences packed along one axis, with an INT64 array of cumulative sequence lengths).
 *
 *   gradY, x, gradX, y : [T,H] packed tokens, contiguous, 16-byte aligned
 *   weight, gradWeight : [W,H]
 *   mask               : optional, one byte per token [T] (nonzero = keep), NULL = all kept
 *   cu_seqlens         : device int64 [nseq], 8-byte aligned: cu_seqlens[b] is the end of
 *                        sequence b, which holds tokens cu_seqlens[b-1] .. cu_seqlens[b]-1
 *                        (cu_seqlens[-1] = 0). Preconditions, not checked (the values live on
 *                        the device): non-decreasing, last value = T. Violating them gives
 *                        unspecified outputs but no access outside the buffers.
 *
 * Every sequence is its own masked causal conv: the equations of the function description apply
 * within a sequence, and no stencil reads a token of another sequence (rows past a sequence's end,
 * or before its start for the forward, are zero); gradWeight sums the terms of all sequences.
 * This equals the padded [S,B,H] layout with each batch's mask cut at its sequence length.
 * Limits: T in [1, 524288], nseq in [1, 524288] (empty sequences allowed), H and W as for the
 * extended calls. Both calls need a workspace (per-token window limits; the backward also holds
 * its gradWeight partials); sizes from the *_get_workspace_size functions. Same error codes.
 */
int mccb_varlen_get_workspace_size(int64_t T, int64_t nseq, int64_t H, int64_t W, int dtype,
                                   uint64_t *workspace_size);
int mccb_varlen_backward(const void *gradY, const void *x, const void *weight, const uint8_t *mask,
                         const int64_t *cu_seqlens, void *gradX, void *gradWeight, int64_t T,
                         int64_t nseq, int64_t H, int64_t W, int dtype, void *workspace,
                         uint64_t workspace_size, void *stream);
int mccb_varlen_forward_get_workspace_size(int64_t T, int64_t nseq, int64_t H, int64_t W,
                                           int dtype, uint64_t *workspace_size);
int mccb_varlen_forward(const void *x, const void *weight, const uint8_t *mask,
                        const int64_t *cu_seqlens, void *y, int64_t T, int64_t nseq, int64_t H,
                        int64_t W, int dtype, void *workspace, uint64_t workspace_size,
                        void *stream);

/* The tiling chosen for a shape, for mccb_backward (fwd_* excepted) and mccb_forward (fwd_*);
 * a pure function of (S, B, H, dtype). Exposed so that tests can place edge cases on tile
 * boundaries. */
typedef struct {
    int64_t rows_per_turn;   /* rows one wavefront handles per round */
    int64_t rows_per_round;  /* rows a fused-kernel block advances per round */
    int64_t rows_per_strip;  /* rows of [S, B*H] one fused-kernel block covers (whole rounds) */
    int64_t n_strips;        /* ceil(S / rows_per_strip) */
    int64_t cols_per_block;  /* columns of [S, B*H] one fused-kernel block covers */
    int64_t n_col_blocks;    /* ceil(B*H / cols_per_block) */
    int64_t waves_per_block;
    uint64_t workspace_size; /* same value as mccb_get_workspace_size */
    int64_t fwd_rows_per_tile; /* rows one mccb_forward block covers */
    int64_t fwd_cols_per_tile; /* columns of [S, B*H] one mccb_forward block covers */
    int64_t fwd_n_col_tiles;   /* ceil(B*H / fwd_cols_per_tile) */
    int64_t fwd_n_row_tiles;   /* ceil(S / fwd_rows_per_tile) */
    int64_t group_spacing;     /* bytes between the column groups of a fused-kernel block
                                  (0: adjacent groups) */
} mccb_plan_t;

/* Fills *plan for a valid shape. Same return codes as mccb_get_workspace_size. Host-only. */
int mccb_get_plan(int64_t S, int64_t B, int64_t H, int dtype, mccb_plan_t *plan);

/* Human-readable name of a status code (static storage, never NULL). */
const char *mccb_status_string(int status);

/*
 * Optional per-kernel timing, for benchmarks. After mccb_profile_begin(n), each of the next n
 * mccb_backward calls records HIP events on its stream around its two kernels (the fused
 * mask/gradX/gradWeight-partials kernel and the gradWeight reduction). mccb_profile_end waits for
 * the recorded events, returns the summed milliseconds of each kernel and the number of calls
 * recorded, and turns recording off. Returns MCCB_OK or MCCB_ERR_RUNTIME. Not thread-safe with
 * respect to concurrent mccb_backward calls.
 */
int mccb_profile_begin(int max_calls);
int mccb_profile_end(double *fused_ms, double *reduce_ms, int *calls);

#ifdef __cplusplus
}
#endif

#endif /* MCCB_H */
