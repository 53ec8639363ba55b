/*
 * moe_route.h -- C ABI of the MI355X (gfx950) MoE layer hot path:
 *   routing metadata preprocessing -> dispatch-permute -> grouped SwiGLU MLP
 *   -> probability-weighted combine-unpermute, all experts on one GPU.
 *
 * Operations follow these pages (cited by title and section):
 *   [P1] Megatron-LM PR #6800 "Reuse caller-owned HybridEP dispatch and expert
 *        output buffers"
 *   [P2] DeepEP PR #716 "perf: reuse HybridEP routing allgather buffer"
 *   [P3] NeMo-Automodel PR #3931 "perf(moe): sync-free HybridEP dispatch
 *        (capacity mode, equal token counts)"
 *   [P4] Megatron-LM PR #4632 "moe: add DeepEP V2 ElasticBuffer support to MoE
 *        flex dispatcher"
 *   [P5] TensorRT-LLM PR #16190 "Update CuTeDSL MegaMoE kernels"
 *
 * Conventions for every call below:
 *   - Pointers prefixed d_ are device memory owned by the caller; the library
 *     never allocates, frees or keeps them beyond the call (the workspace is
 *     only referenced through the handle until it is re-initialised).
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream).
 *     Device work is enqueued on it asynchronously; no call synchronises the
 *     host with the device, so every sequence is capturable in a HIP graph.
 *   - Shapes are fixed when a handle is initialised (static-shape rule of
 *     [P4] "What changed": the per-rank token ceiling is pinned at
 *     construction).  Host-side argument checks return a negative status and
 *     enqueue nothing; device-side problems are reported only through the
 *     overflow flag word.
 *   - bf16 tensors are raw 16-bit patterns; fp8 is OCP e4m3 ("fn") with one
 *     fp32 scale per 128 consecutive columns of a row.
 *   - Device pointers to token rows must be 16-byte aligned.
 */
#ifndef MOE_ROUTE_H
#define MOE_ROUTE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

/* ---- status codes --------------------------------------------------------- */
enum moe_status {
    MOE_OK = 0,
    MOE_EINVAL = -1,        /* null required pointer, unknown enum value      */
    MOE_ESHAPE = -2,        /* sizes outside the supported ranges             */
    MOE_EDTYPE = -3,        /* dtype / format combination not supported       */
    MOE_EALIGN = -4,        /* a device pointer is not 16-byte aligned         */
    MOE_ESTALE = -5,        /* handle's workspace was re-initialised, or the   */
                            /* handle has no routing metadata yet             */
    MOE_EHIP = -6,          /* a HIP runtime call failed                       */
    MOE_EUNSUPPORTED = -7,  /* legal but not implemented                       */
    MOE_ENOSPC = -8,        /* workspace or scratch smaller than required      */
    MOE_EBUSY = -9,         /* ring slot still in use (reuse before release)   */
    MOE_ESTATE = -10        /* ring slot released twice / never acquired       */
};

/* ---- routing formats ([P2] "Memory impact", "Implementation") -------------
 * DENSE_*: top-k expert indices [T, K], -1 marks an empty slot.
 * SPARSE_BOOL: Boolean map [T, E], one byte per (token, expert), nonzero =
 * routed; K then bounds the experts per token. */
enum moe_route_fmt {
    MOE_ROUTE_DENSE_I16 = 0,
    MOE_ROUTE_DENSE_I32 = 1,
    MOE_ROUTE_SPARSE_BOOL = 2
};

/* ---- payload / weight dtypes ([P2] "Full HybridEP reference validation":
 * BF16 and FP8 dispatch; [P5] first commit message: low-precision weights) */
enum moe_dtype {
    MOE_BF16 = 0,
    MOE_FP8E4M3_B128 = 1    /* e4m3 codes + fp32 scale per 128 columns         */
};

/* ---- overflow flag bits ([P3] "What does this PR do ?", "Validation": the
 * real counts stay on the device and an overflow flag reports truncation).
 * The flag word is written fresh (not accumulated) by every preprocess. */
#define MOE_FLAG_CAPACITY   1  /* some expert count exceeds the capacity          */
#define MOE_FLAG_OUT_ROWS   2  /* padded segments need more rows than out_rows    */
#define MOE_FLAG_BAD_EXPERT 4  /* a dense index outside [-1, E)                   */
#define MOE_FLAG_DUPLICATE  8  /* repeated expert in a dense row, or more than K  */
                               /* experts in a sparse row                          */

/* Static description of one dispatch/combine problem. */
typedef struct moe_desc {
    int32_t T;             /* tokens (rows of x), >= 0                           */
    int32_t H;             /* hidden size; bf16: multiple of 8, fp8: of 128      */
    int32_t E;             /* experts, 1..1024                                   */
    int32_t K;             /* top-k slots (dense) / max experts per row (sparse) */
    int32_t route_fmt;     /* enum moe_route_fmt                                 */
    int32_t payload;       /* enum moe_dtype of the permuted rows                */
    int32_t pad_multiple;  /* >= 1; each expert segment is padded to a multiple  */
    int32_t capacity;      /* rows kept per expert; < 0 = unbounded              */
    int64_t out_rows;      /* rows R of the permuted / expert-output buffers;    */
                           /* 0 = moe_out_rows_bound(desc)                        */
} moe_desc;

/* Dispatch handle: plain data.  Host ints plus device pointers carved from
 * the caller's workspace; it owns nothing.  Fields are read-only for the
 * caller.  Device arrays (all in the workspace):
 *   seg_off[E+1]  int64  first row of each expert segment (exclusive scan of
 *                        the padded kept counts); seg_off[E] = rows needed
 *   kept[E]       int32  copies kept per expert (min(count, capacity))
 *   row_id[T*K]   int32  destination row of copy (t, j), -1 if none
 *   copy_prob[T*K] f32   probability of copy (t, j) (1 without probs, 0 if
 *                        dropped)
 *   src_row[R]    int32  source token of each row, -1 for rows with no copy */
typedef struct moe_handle {
    moe_desc desc;         /* resolved copy (out_rows filled in)                 */
    uint64_t epoch;        /* workspace generation                               */
    int32_t n_tiles;       /* 64-token tiles                                      */
    int32_t state;         /* 0 = initialised, 1 = routing metadata enqueued     */
    void* ws;
    size_t ws_bytes;
    uint64_t* tile_mask;   /* [n_tiles, E] per-tile expert membership bitmasks    */
    int32_t* tile_base;    /* [n_tiles, E] copies of each expert in earlier tiles */
    int32_t* tile_err;     /* [n_tiles] per-tile flag bits                        */
    int64_t* seg_off;
    int32_t* kept;
    int64_t* rows_needed;  /* [1]                                                 */
    int32_t* row_id;
    float* copy_prob;
    int32_t* src_row;
} moe_handle;

/* ---- host-only helpers (no device access) ---------------------------------- */

/* Text for a status code. */
const char* moe_status_string(int status);

/* Largest number of rows the padded segments can need:
 * min(E * roundup(capacity, p), T*K + E*(p-1)); the second term alone when
 * capacity < 0.  This is the static output bound of [P3] "What does this PR
 * do ?" (the permuted buffer sized from host-known numbers so that no device
 * count is read back).  Returns -1 for an invalid descriptor. */
int64_t moe_out_rows_bound(const moe_desc* desc);

/* Bytes of one routing tensor of this descriptor: T*E for the Boolean map,
 * T*K*2 (int16) or T*K*4 (int32) for dense indices.  [P2] "Memory impact". */
int64_t moe_routing_bytes(const moe_desc* desc);

/* Caller-side static bound from a calibrated row count: ceil(rows * factor)
 * rounded up to a multiple of 4.  [P3] "What does this PR do ?" and the
 * calibration figure under "Validation".  Returns -1 if rows < 0 or
 * factor <= 0. */
int64_t moe_capacity_from_rows(int64_t rows, double factor);

/* Workspace bytes needed by a handle for this descriptor (0 if invalid): the
 * routing metadata of moe_handle (per-tile masks and bases, per-expert counts
 * and offsets, the row map), sized from the descriptor alone, so the caller
 * can own and reuse it ([P1] "Summary": caller-owned buffers reused across
 * steps; [P2] "Summary": a routing buffer reused instead of reallocated). */
size_t moe_workspace_bytes(const moe_desc* desc);

/* Validate `desc`, resolve out_rows, carve the caller's workspace d_ws
 * (ws_bytes >= moe_workspace_bytes) and fill *h.  Host only: touches no
 * device memory.  Re-initialising a workspace makes earlier handles on it
 * stale (later calls with them return MOE_ESTALE), the explicit early-reuse
 * failure of [P1] "Summary". */
int moe_handle_init(const moe_desc* desc, void* d_ws, size_t ws_bytes, moe_handle* h);

/* ---- device calls (asynchronous on `stream`) -------------------------------- */

/* Routing metadata preprocessing.  [P2] "Summary" (metadata preprocessing
 * consumes the routing map on the dispatch stream), [P3] "What does this PR
 * do ?" (counts and an overflow flag left on the device, no host sync),
 * [P4] "Motivation" (layout inferred from the top-k indices).
 *   d_routing            [T,K] int16/int32 or [T,E] uint8 per desc.route_fmt
 *   d_probs              nullable; fp32 with the routing's shape
 *   d_T_live             nullable; device int32 count of live tokens, tokens
 *                        at or beyond it are unrouted (decode bucket trim,
 *                        [P5] review-fix commit)
 *   d_tokens_per_expert  [E] int32 out: raw per-expert copy counts
 *   d_out_probs          nullable [R] fp32 out: probability of each row's copy,
 *                        0 for rows holding no copy
 *   d_flag               [1] int32 out: MOE_FLAG_* bits, written fresh
 * Rows inside an expert segment follow token order; an expert keeps its first
 * `capacity` copies; copies that would land at or beyond out_rows are
 * dropped. */
int moe_route_preprocess(moe_handle* h, const void* d_routing, const float* d_probs,
                         const int32_t* d_T_live, int32_t* d_tokens_per_expert,
                         float* d_out_probs, int32_t* d_flag, void* stream);

/* Permute: copy every kept token row to its destination row.  [P1]
 * "Summary"/"Configuration" (dispatch writes permuted tokens into a
 * caller-provided output buffer), [P2] "Full HybridEP reference validation"
 * (dispatch with permutation, BF16 and FP8).
 *   d_x         [T,H] bf16, or [T,H] e4m3 codes for desc.payload = FP8
 *   d_x_scales  fp8 only: [T, H/128] fp32; else NULL
 *   d_out       [R,H] same dtype as d_x; rows without a copy are not written
 *   d_out_scales fp8 only: [R, H/128] fp32 */
int moe_permute(const moe_handle* h, const void* d_x, const float* d_x_scales, void* d_out,
                float* d_out_scales, void* stream);

/* Quantise-on-dispatch: the permute of bf16 token rows into fp8 rows.  Each
 * token row is quantised once per 1x128 block (scale = block amax / 448, 1
 * for an all-zero block; code = e4m3(x / scale), nearest-even, saturating at
 * 448: the expert MLP's own activation rule) and the codes and scales are
 * written to every kept copy's row.  [P2] "Full HybridEP reference
 * validation" (FP8 dispatch), [P1] "Configuration" (FP8 expert GEMMs behind
 * the dispatch).  Requires desc.payload = MOE_FP8E4M3_B128 (the permuted
 * rows' format).
 *   d_x          [T,H] bf16
 *   d_out        [R,H] e4m3 codes; rows without a copy are not written
 *   d_out_scales [R,H/128] fp32 */
int moe_permute_quantize(const moe_handle* h, const void* d_x, void* d_out, float* d_out_scales, void* stream);

/* moe_route_preprocess followed by moe_permute on the same stream. */
int moe_dispatch(moe_handle* h, const void* d_routing, const float* d_probs,
                 const int32_t* d_T_live, const void* d_x, const float* d_x_scales, void* d_out,
                 float* d_out_scales, float* d_out_probs, int32_t* d_tokens_per_expert,
                 int32_t* d_flag, void* stream);

/* Scratch bytes moe_grouped_swiglu_mlp needs for FFN width F and weight
 * dtype wdtype (the FC1 -> activation -> FC2 intermediate of [P1]
 * "Configuration", owned by the caller): MOE_BF16 holds the bf16 FC1
 * activations of all R rows;
 * MOE_FP8E4M3_B128 holds the fp32 FC1 activations plus the e4m3 codes and
 * fp32 1x128 scales of the permuted rows and of the activations (each input
 * is quantised once per call).  0 if invalid. */
size_t moe_mlp_scratch_bytes(const moe_handle* h, int32_t F, int32_t wdtype);

/* Grouped expert MLP over the permuted rows: for every expert e and every
 * kept row r of its segment, g = W1[e][0:F] x_r, u = W1[e][F:2F] x_r,
 * a = silu(g) * u, y_r = W2[e] a, y_r stored as bf16 into the caller-owned
 * d_expert_out.  [P1] "Summary" and "Configuration" (grouped MLP writing FC2
 * into a caller-provided reusable buffer), [P5] streaming-load commit (FC1
 * weight is the concatenated gate/up matrix).
 *   d_perm        [R,H] bf16 permuted rows (output of moe_permute); for a
 *                 handle with fp8 payload, [R,H] e4m3 codes quantised on
 *                 dispatch (moe_permute_quantize), fp8 weights only
 *   d_perm_scales NULL for bf16 rows; [R,H/128] fp32 scales of fp8 rows,
 *                 which FC1 then consumes without re-quantising
 *   wdtype MOE_BF16: d_w1 [E,2F,H] bf16, d_w2 [E,H,F] bf16, scales NULL;
 *          requires H % 256 == 0 and F % 128 == 0.
 *   wdtype MOE_FP8E4M3_B128: d_w1 [E,2F,H] e4m3, d_w1_scales [E,2F/128,H/128]
 *          fp32, d_w2 [E,H,F] e4m3, d_w2_scales [E,H/128,F/128] fp32; the
 *          bf16 rows are quantised per 1x128 block on load (scale = block
 *          amax / 448, 1 for an all-zero block; code = e4m3(x / scale),
 *          nearest-even, saturating) and a is re-quantised the same way
 *          before FC2; requires H, F multiples of 128.  Built for decode-sized
 *          batches (few rows per expert; weight streaming bound).
 *   d_scratch     >= moe_mlp_scratch_bytes bytes
 *   d_expert_out  [R,H] bf16; rows that hold no kept copy are unspecified */
int moe_grouped_swiglu_mlp(const moe_handle* h, int32_t F, int32_t wdtype, const void* d_perm,
                           const float* d_perm_scales, const void* d_w1, const float* d_w1_scales,
                           const void* d_w2, const float* d_w2_scales, void* d_scratch,
                           size_t scratch_bytes, void* d_expert_out, void* stream);

/* The two halves of moe_grouped_swiglu_mlp, for callers that schedule or
 * time them separately.  FC1 + SwiGLU writes the activations of every kept
 * row into d_scratch; FC2 reads them from d_scratch (with fp8 weights it
 * first writes their 1x128 codes and scales into d_scratch as well) and
 * writes d_expert_out.
 * Arguments and requirements as for moe_grouped_swiglu_mlp; FC2 must run
 * after FC1 on the same handle and scratch (same stream or ordered). */
int moe_grouped_fc1_swiglu(const moe_handle* h, int32_t F, int32_t wdtype, const void* d_perm,
                           const float* d_perm_scales, const void* d_w1, const float* d_w1_scales,
                           void* d_scratch, size_t scratch_bytes, void* stream);
int moe_grouped_fc2(const moe_handle* h, int32_t F, int32_t wdtype, const void* d_w2,
                    const float* d_w2_scales, void* d_scratch, size_t scratch_bytes,
                    void* d_expert_out, void* stream);

/* Grouped expert MLP that allocates nothing, for callers that cannot call
 * hipMalloc or take a caller-provided scratch buffer (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).  Same
 * operation, arguments and requirements as moe_grouped_swiglu_mlp, minus the
 * scratch: the FC1 -> FC2 activations live in a file-scope device array of
 * MOE_NOALLOC_SCRATCH_BYTES bytes that the library holds on every GPU it runs
 * on until the process ends (its address is looked up once per device, at the
 * first call with that device current).
 *   Returns MOE_ENOSPC, with nothing enqueued, when
 *   moe_mlp_scratch_bytes(h, F, wdtype) exceeds MOE_NOALLOC_SCRATCH_BYTES
 *   (128 MiB: the bf16 path up to R*F = 64 Mi activations, the fp8 path up to
 *   about 7,500 rows at H = 7168, F = 2048, which holds the 5,888-row bound
 *   of a 256-token decode bucket with 256 experts top-8 and padding 16).
 *   Every call on one GPU shares that GPU's array, which keeps the last
 *   call's contents (nothing in it needs to start at zero): calls that can
 *   overlap on one GPU (different streams without ordering between them)
 *   race on it and must be serialised by the caller. */
#define MOE_NOALLOC_SCRATCH_BYTES (128ll << 20)
int moe_grouped_swiglu_mlp_noalloc(const moe_handle* h, int32_t F, int32_t wdtype, const void* d_perm,
                                   const float* d_perm_scales, const void* d_w1, const float* d_w1_scales,
                                   const void* d_w2, const float* d_w2_scales, void* d_expert_out,
                                   void* stream);

/* FC2 into the fp8 combine format: as moe_grouped_fc2 (bf16 weights), but each
 * kept row's fp32 output is quantised per 1x128 block (scale = block amax /
 * 448, 1 for an all-zero block; code = e4m3(y / scale), nearest-even,
 * saturating) instead of being rounded to bf16, halving the expert-output
 * bytes that FC2 writes and the combine reads.  [P2] "Full HybridEP reference
 * validation" (FP8 token payloads), [P1] "Configuration" (FP8 expert GEMMs).
 *   wdtype        MOE_BF16 only (else MOE_EUNSUPPORTED)
 *   d_out_q       [R,H] e4m3 codes out; rows without a kept copy not written
 *   d_out_scales  [R,H/128] fp32 out */
int moe_grouped_fc2_fp8out(const moe_handle* h, int32_t F, int32_t wdtype, const void* d_w2,
                           const float* d_w2_scales, void* d_scratch, size_t scratch_bytes, void* d_out_q,
                           float* d_out_scales, void* stream);

/* Combine-unpermute: y[t] = bf16( sum over the token's surviving copies j, in
 * slot order, of p_tj * expert_out[row_id[t,j]] ) accumulated in fp32;
 * p_tj = copy probability if apply_probs else 1; a token with no surviving
 * copy gets 0.  [P1] "Summary"/"Motivation" (combine is the final read of the
 * expert output), [P5] review-fix commit (top-k reduction).
 *   d_expert_out  [R,H] bf16
 *   d_y           [T,H] bf16 out */
int moe_combine(const moe_handle* h, const void* d_expert_out, int32_t apply_probs, void* d_y,
                void* stream);

/* Combine from the fp8 format: as moe_combine, with each copy's row
 * dequantised (code value * its block's scale, in fp32) before the weighted
 * sum.  Requires H % 128 == 0.
 *   d_expert_out_q       [R,H] e4m3 codes (moe_grouped_fc2_fp8out)
 *   d_expert_out_scales  [R,H/128] fp32
 *   d_y                  [T,H] bf16 out */
int moe_combine_fp8(const moe_handle* h, const void* d_expert_out_q, const float* d_expert_out_scales,
                    int32_t apply_probs, void* d_y, void* stream);

/* ---- persistent decode layer ----------------------------------------------------
 * [P5] first commit message (dispatch, FC1, FC2 and combine fused in one kernel
 * for decode, stages handing work to each other through flags instead of
 * separate launches) and review-fix commit (live-token trim; an empty batch
 * launches nothing that computes).  After moe_route_preprocess on the handle,
 * one call runs the rest of the layer with fp8 weights: quantise-on-dispatch
 * of the bf16 token rows (as moe_permute_quantize), FC1 + SwiGLU, the 1x128
 * re-quantisation of the activations, FC2 into d_expert_out, and the combine
 * into d_y (as moe_combine), as one persistent kernel after a small reset of
 * its control block.  Work items are handed out by device-side queues and
 * wait on the items they depend on; the result is bit-identical to
 * moe_permute_quantize + moe_grouped_swiglu_mlp (fp8) + moe_combine.
 *   Requires desc.payload = MOE_BF16, H and F multiples of 128.
 *   d_x            [T,H] bf16 tokens
 *   d_w1, d_w1_scales, d_w2, d_w2_scales  as moe_grouped_swiglu_mlp, fp8
 *   d_scratch      >= moe_decode_layer_scratch_bytes(h, F) bytes
 *   d_expert_out   [R,H] bf16, caller-owned and reused; rows holding no kept
 *                  copy are unspecified
 *   d_y            [T,H] bf16 out
 *   d_status       [1] int32 in/out.  The call clears bits 0 and 1 and keeps
 *                  bit 2.  On return: bit 0 set if a wait of the kernel ran
 *                  past its bound (0.25 s, see moe_decode_layer_set_wait_bound),
 *                  bit 1 set if a workgroup ran on an XCD numbered 8 or more
 *                  (the work queues assume XCDs 0-7); the outputs are then
 *                  unspecified.  Bit 2 is the caller's abort request: set
 *                  before the call, or while the kernel runs (e.g. by a copy
 *                  on another stream), it makes every wait return at once;
 *                  the outputs are then unspecified.  Once any bit is set,
 *                  every later wait returns at once, so the kernel always runs
 *                  to its end. */
size_t moe_decode_layer_scratch_bytes(const moe_handle* h, int32_t F);
int moe_decode_layer_fp8(const moe_handle* h, int32_t F, const void* d_x, const void* d_w1, const float* d_w1_scales,
                         const void* d_w2, const float* d_w2_scales, void* d_scratch, size_t scratch_bytes,
                         void* d_expert_out, int32_t apply_probs, void* d_y, int32_t* d_status, void* stream);

/* Bound of every wait of moe_decode_layer_fp8, in ticks of the GPU's 100 MHz
 * real-time counter, for calls made after this one in the process; ticks <= 0
 * restores the default (25,000,000 = 0.25 s).  For tests of the time-out
 * path and for callers that want a failed dependency reported sooner. */
void moe_decode_layer_set_wait_bound(int64_t ticks);

/* ---- fused decode layer ------------------------------------------------------------
 * [P5] first commit message (dispatch, FC1, FC2 and combine of a decode batch
 * fused into one persistent kernel with block-scaled low-precision expert
 * weights) and review-fix commit (work trimmed to the live tokens; an empty
 * batch launches nothing).  After moe_route_preprocess on the handle, one call
 * runs the rest of the layer with fp8 weights in two launches: a small one
 * that quantises every token row into its kept copies (as
 * moe_permute_quantize), zeroes the output rows of tokens without a kept copy
 * and clears the completion counters; then one persistent kernel whose work
 * units are (touched expert, 128-feature slice of the FFN).  A unit computes
 * FC1 + SwiGLU for its slice, quantises the slice as one 1x128 activation
 * block, and adds its FC2 share through a partial buffer; the last unit of an
 * expert reduces the expert's rows into d_expert_out, and the last expert of a
 * token combines the token into d_y.  No work unit waits for another.  The
 * result is bit-identical to moe_permute_quantize + moe_grouped_swiglu_mlp
 * (fp8) + moe_combine on the same handle.
 *   Requires desc.payload = MOE_BF16, H and F multiples of 128, H <= 8192
 *   (MOE_ESHAPE otherwise).
 *   d_x            [T,H] bf16 tokens
 *   d_w1, d_w1_scales, d_w2, d_w2_scales  as moe_grouped_swiglu_mlp, fp8
 *   d_scratch      >= moe_decode_fused_scratch_bytes(h, F) bytes (token codes
 *                  per row, FC2 partials [F/128, T*K, H] fp32, counters);
 *                  contents on entry are ignored
 *   d_expert_out   [R,H] bf16, caller-owned and reused; rows holding no kept
 *                  copy are not written
 *   d_y            [T,H] bf16 out
 * Two calls that share d_scratch must not overlap.  Returns MOE_ENOSPC if the
 * scratch is too small; nothing is enqueued on any error. */
size_t moe_decode_fused_scratch_bytes(const moe_handle* h, int32_t F);
int moe_decode_fused_fp8(const moe_handle* h, int32_t F, const void* d_x, const void* d_w1, const float* d_w1_scales,
                         const void* d_w2, const float* d_w2_scales, void* d_scratch, size_t scratch_bytes,
                         void* d_expert_out, int32_t apply_probs, void* d_y, void* stream);

/* ---- backward (gradients of dispatch and combine) ---------------------------
 * [P2] "Full HybridEP reference validation" (hidden-state and probability
 * gradients of the backward-of-dispatch and of the backward-of-combine), [P3]
 * "What does this PR do ?" (the combine's backward is a dispatch sized by the
 * same host-known row count: no host sync).  Both reuse the handle of the
 * forward dispatch; gradients are bf16 rows whatever the forward payload.
 * Probability gradients have the routing's shape: [T,K] fp32 by slot for
 * dense routing, [T,E] fp32 by expert for a Boolean map; entries of copies
 * that were not kept (empty, invalid, duplicate, over capacity, beyond
 * out_rows) and unrouted entries are 0. */

/* Backward of dispatch.  A token's gradient is the sum, in fp32 and slot
 * order, of its kept copies' row gradients (one rounding to bf16; 0 if none
 * was kept), i.e. moe_combine with apply_probs = 0 applied to d_grad_out.
 *   d_grad_out        [R,H] bf16: gradient of the permuted rows
 *   d_grad_out_probs  nullable [R] fp32: gradient of the dispatch's per-row
 *                     probabilities (d_out_probs)
 *   d_grad_x          [T,H] bf16 out
 *   d_grad_probs      nullable out (requires d_grad_out_probs): each kept
 *                     copy's row gradient at its routing position */
int moe_dispatch_backward(const moe_handle* h, const void* d_grad_out, const float* d_grad_out_probs,
                          void* d_grad_x, float* d_grad_probs, void* stream);

/* Backward of combine.  With w_tj = the copy probability if apply_probs else
 * 1, for every kept copy (t, j) at row r = row_id[t,j]:
 *   d_grad_expert_out[r] = w_tj * d_grad_y[t]   (exact product, one rounding
 *                          to bf16); rows holding no kept copy are not written
 *   d_grad_probs at (t, j) = sum over h of d_grad_y[t,h] * d_expert_out[r,h]
 *                          in fp32 when apply_probs, else 0.
 *   d_grad_y          [T,H] bf16: gradient of the combine output
 *   d_expert_out      [R,H] bf16: the forward combine's input; read only for
 *                     the probability gradient (may be NULL otherwise)
 *   d_grad_expert_out [R,H] bf16 out
 *   d_grad_probs      nullable out, the routing's shape */
int moe_combine_backward(const moe_handle* h, const void* d_grad_y, const void* d_expert_out,
                         int32_t apply_probs, void* d_grad_expert_out, float* d_grad_probs, void* stream);

/* ---- caller-owned buffer ring ------------------------------------------------
 * [P1] "Summary", "Motivation", "Known limitations": dispatch outputs and FC2
 * outputs live in a fixed ring of persistent slots owned by the application;
 * the final consumer of a slot releases it by recording an event on its own
 * stream, and the next producer of that slot waits for the event on the
 * device (no host or stream-wide synchronisation), so the storage stays
 * bounded.  Reuse before release and double release fail explicitly.
 * Host-side logic: slots are carved from the caller's device buffer; the only
 * HIP calls are event create (lazily, at a slot's first release), record,
 * stream-wait and destroy.  Not thread-safe: one ring per host thread.
 * Graph capture: a release recorded during a capture is waited on only by
 * acquires inside the same capture; a release recorded outside any capture
 * is not waited on inside one (capture begins after the caller's
 * synchronisation, so the eager warm-up has completed). */
#define MOE_RING_MAX_SLOTS 32
typedef struct moe_ring {
    void* base;                                  /* caller's storage, n_slots * slot_bytes */
    size_t slot_bytes;                           /* multiple of 256                        */
    int32_t n_slots;                             /* 1 .. MOE_RING_MAX_SLOTS                */
    int32_t next;                                /* next slot in rotation                  */
    uint64_t acquisitions;
    int32_t state[MOE_RING_MAX_SLOTS];           /* 0 free, 1 acquired                     */
    int32_t event_kind[MOE_RING_MAX_SLOTS];      /* 0 none, 1 eager, 2 recorded in capture */
    unsigned long long event_capture[MOE_RING_MAX_SLOTS];  /* capture id of kind 2         */
    void* event[MOE_RING_MAX_SLOTS];             /* hipEvent_t of the last release         */
} moe_ring;

/* Set up a ring over d_base (256-byte aligned, >= n_slots * slot_bytes bytes,
 * owned by the caller).  Host only.  MOE_ESHAPE for n_slots outside
 * 1..MOE_RING_MAX_SLOTS or slot_bytes not a positive multiple of 256. */
int moe_ring_init(moe_ring* r, void* d_base, size_t slot_bytes, int32_t n_slots);

/* Take the next slot in rotation for a producer on `stream`: *d_slot is its
 * device address, *slot its index.  If the slot was released before, `stream`
 * waits (on the device) for that release.  MOE_EBUSY if the slot's previous
 * acquisition has not been released: the ring is too small for the schedule
 * (early reuse, [P1] "Known limitations"). */
int moe_ring_acquire(moe_ring* r, void* stream, void** d_slot, int32_t* slot);

/* The final consumer on `stream` is done with `slot` once the work enqueued on
 * `stream` so far has run: records the slot's release event there.
 * MOE_ESTATE if the slot is not currently acquired (double release). */
int moe_ring_release(moe_ring* r, int32_t slot, void* stream);

/* Destroy the ring's events (the caller's storage is untouched). */
int moe_ring_destroy(moe_ring* r);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ROUTE_H */
