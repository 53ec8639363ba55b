// Internal declarations shared by the HIP translation units of libmoe_route.
// Not part of the public ABI (that is include/moe_route.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "moe_route.h"

namespace moe {

constexpr int kMaxE = 1024;      // experts supported by the routing kernels
constexpr int kTileTok = 64;     // tokens per routing tile = one wavefront

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// float -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}
// Two floats -> two bf16 bits (lo in the low half) by gfx950's packed
// conversion (v_cvt_pk_bf16_f32): round to nearest even, the same result as
// f32_to_bf16 for every finite value.
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{lo, hi}, bf16x2v));
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ---- e4m3 block quantisation (1 x 128 blocks) ------------------------------
// scale = block amax / 448 (1 for an all-zero block; a correctly rounded fp32
// division), code = e4m3(v / scale), nearest even, saturating at 448.
__device__ __forceinline__ float e4m3_prep(float v) {   // saturate to the e4m3 range
    return fminf(fmaxf(v, -448.f), 448.f);
}
__device__ __forceinline__ float e4m3_scale(float amax) { return amax > 0.f ? amax / 448.f : 1.f; }
// Four values -> four e4m3 codes in one 32-bit word (value i in byte i).
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d, float sc) {
    int p = 0;
    p = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_prep(a / sc), e4m3_prep(b / sc), p, false);
    p = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_prep(c / sc), e4m3_prep(d / sc), p, true);
    return (uint32_t)p;
}

// Every host-side argument check of moe_grouped_swiglu_mlp except those of
// the scratch buffer (no device access); returns a moe_status.
int check_mlp_host(const moe_handle* h, int32_t F, int32_t wdtype, const void* d_perm, const float* d_perm_scales,
                   const void* d_w1, const float* d_w1_scales, const void* d_w2, const float* d_w2_scales,
                   const void* d_expert_out);

// ---- launchers (each returns a hipError_t) --------------------------------
hipError_t launch_route(const moe_handle* h, const void* routing, const float* probs,
                        const int32_t* T_live, int32_t* tokens_per_expert, float* out_probs,
                        int32_t* flag, hipStream_t s);
// Column slices per token row for the row-copy kernels: one wavefront per
// (token, slice).  Few tokens get more slices (whole 64-chunk groups) so that
// at least ~4096 wavefronts run; large batches keep one slice per row.
inline void row_slices(int T, int nch, int* nsplit, int* slice_ch) {
    const int groups = (nch + 63) / 64;
    int n = T > 0 ? (4096 + T - 1) / T : 1;
    if (n > groups) n = groups;
    if (n < 1) n = 1;
    const int gps = (groups + n - 1) / n;          // 64-chunk groups per slice
    *slice_ch = gps * 64;
    *nsplit = (nch + *slice_ch - 1) / *slice_ch;
}

hipError_t launch_permute(const moe_handle* h, const void* x, const float* x_scales, void* out,
                          float* out_scales, hipStream_t s);
// bf16 token rows -> e4m3 codes + 1x128 scales at every kept copy's row
hipError_t launch_permute_quant(const moe_handle* h, const void* x, void* out, float* out_scales, hipStream_t s);
hipError_t launch_combine(const moe_handle* h, const void* y_in, int apply_probs, void* y_out,
                          hipStream_t s);
// combine from fp8 expert-output rows (e4m3 codes [R,H] + 1x128 scales)
hipError_t launch_combine_fp8(const moe_handle* h, const void* yq, const float* ys, int apply_probs, void* y_out,
                              hipStream_t s);
// backward: probability gradients of a dispatch (row gradients gathered to
// the routing's shape) and the combine backward (row and probability grads)
hipError_t launch_probs_gather(const moe_handle* h, const float* grad_row_probs, float* grad_probs,
                               hipStream_t s);
hipError_t launch_combine_backward(const moe_handle* h, const void* grad_y, const void* expert_out,
                                   int apply_probs, void* grad_expert_out, float* grad_probs, hipStream_t s);
// stage 0: FC1 + SwiGLU (in -> act), stage 1: FC2 (act -> expert_out); with
// out_scales non-null, FC2 writes e4m3 codes to `out` and 1x128 scales
hipError_t launch_gemm_bf16(const moe_handle* h, int stage, int F, const void* in, const void* w,
                            void* out, float* out_scales, int num_cu, hipStream_t s);
// stage 0: FC1 + SwiGLU (bf16 rows -> fp32 activations), stage 1: FC2
// (fp32 activations -> bf16 expert output); e4m3 weights with 128x128 scales
// fp8 path: stage 0 quantises the permuted rows `in` into the scratch and
// writes fp32 activations there; stage 1 quantises those and writes `out`.
// With in_scales non-null, stage 0 takes `in` as already quantised rows
// (e4m3 codes [R,H] with 1x128 scales) and skips the row quantiser.
hipError_t launch_gemm_fp8(const moe_handle* h, int stage, int F, const void* in, const float* in_scales,
                           const void* w, const float* ws, void* scratch, void* out, hipStream_t s);
size_t fp8_mlp_scratch_bytes(long long R, int H, int F);
// persistent decode layer (quantise-on-dispatch, FC1, activation quantiser,
// FC2, combine in one launch after a control-block reset)
size_t decode_layer_scratch_bytes(long long R, int H, int F);
size_t decode_fused_scratch_bytes(long long R, int T, int K, int H, int F, int E);
bool decode_fused_shape_ok(int H, int F);
hipError_t launch_decode_fused(const moe_handle* h, int F, const void* x, const void* w1, const float* w1s,
                               const void* w2, const float* w2s, void* scratch, void* expert_out, int apply_probs,
                               void* y, int num_cu, hipStream_t s);
hipError_t launch_decode_layer(const moe_handle* h, int F, const void* x, const void* w1, const float* w1s,
                               const void* w2, const float* w2s, void* scratch, void* expert_out, int apply_probs,
                               void* y, int32_t* status, long long wait_ticks, int num_cu, hipStream_t s);

}  // namespace moe
