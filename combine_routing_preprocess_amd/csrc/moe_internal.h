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

// float -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

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
hipError_t launch_combine(const moe_handle* h, const void* y_in, int apply_probs, void* y_out,
                          hipStream_t s);
// backward: probability gradients of a dispatch (row gradients gathered to
// the routing's shape) and the combine backward (row and probability grads)
hipError_t launch_probs_gather(const moe_handle* h, const float* grad_row_probs, float* grad_probs,
                               hipStream_t s);
hipError_t launch_combine_backward(const moe_handle* h, const void* grad_y, const void* expert_out,
                                   int apply_probs, void* grad_expert_out, float* grad_probs, hipStream_t s);
// stage 0: FC1 + SwiGLU (in -> act), stage 1: FC2 (act -> expert_out)
hipError_t launch_gemm_bf16(const moe_handle* h, int stage, int F, const void* in, const void* w,
                            void* out, int num_cu, hipStream_t s);
// stage 0: FC1 + SwiGLU (bf16 rows -> fp32 activations), stage 1: FC2
// (fp32 activations -> bf16 expert output); e4m3 weights with 128x128 scales
// fp8 path: stage 0 quantises the permuted rows `in` into the scratch and
// writes fp32 activations there; stage 1 quantises those and writes `out`.
hipError_t launch_gemm_fp8(const moe_handle* h, int stage, int F, const void* in, const void* w,
                           const float* ws, void* scratch, void* out, hipStream_t s);
size_t fp8_mlp_scratch_bytes(long long R, int H, int F);

}  // namespace moe
