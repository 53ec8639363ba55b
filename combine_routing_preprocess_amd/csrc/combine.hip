// Combine-unpermute (K5): each token gathers its surviving expert-output rows
// and reduces them, weighted by the copy probabilities, in fp32; one
// round-to-nearest-even to bf16 at the end.
//
// Operation: Megatron-LM PR #6800 "Reuse caller-owned HybridEP dispatch and
// expert output buffers" (sections "Summary", "Motivation": combine with
// unpermute is the final read of the expert output) and TensorRT-LLM PR
// #16190 "Update CuTeDSL MegaMoE kernels" (review-fix commit: the per-token
// top-k reduction, which must cope with an empty token set).
//
// Token-major: one wavefront per token; each lane owns 16-byte column chunks
// and sums the token's copies in slot order with fused multiply-adds, so the
// result does not depend on scheduling.  Expert-output rows are read once
// (non-temporal); output rows are written once.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kCombU = 4;   // 16-byte chunks per lane per pass

__global__ __launch_bounds__(256) void k_combine(const u32x4* __restrict__ Y, int T, int K, int nch, int R,
                                                 const int32_t* __restrict__ row_id,
                                                 const float* __restrict__ copy_prob, int apply,
                                                 u32x4* __restrict__ y) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const int32_t* rid = row_id + (size_t)t * K;
    const float* cp = copy_prob + (size_t)t * K;
    for (int c0 = 0; c0 < nch; c0 += 64 * kCombU) {
        float acc[kCombU][8];
#pragma unroll
        for (int u = 0; u < kCombU; ++u)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[u][i] = 0.f;
        for (int j = 0; j < K; ++j) {
            const int r = rid[j];
            if (r < 0 || r >= R) continue;
            const float p = apply ? cp[j] : 1.f;
            const u32x4* src = Y + (size_t)r * nch;
            u32x4 v[kCombU];
#pragma unroll
            for (int u = 0; u < kCombU; ++u) {
                const int c = c0 + u * 64 + lane;
                v[u] = c < nch ? __builtin_nontemporal_load(src + c) : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < kCombU; ++u)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    acc[u][2 * w] = fmaf(p, bf16_lo(v[u][w]), acc[u][2 * w]);
                    acc[u][2 * w + 1] = fmaf(p, bf16_hi(v[u][w]), acc[u][2 * w + 1]);
                }
        }
#pragma unroll
        for (int u = 0; u < kCombU; ++u) {
            const int c = c0 + u * 64 + lane;
            if (c < nch) {
                u32x4 o;
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    o[w] = f32_to_bf16(acc[u][2 * w]) | (f32_to_bf16(acc[u][2 * w + 1]) << 16);
                y[(size_t)t * nch + c] = o;
            }
        }
    }
}

}  // namespace

hipError_t launch_combine(const moe_handle* h, const void* y_in, int apply_probs, void* y_out,
                          hipStream_t s) {
    const moe_desc& d = h->desc;
    if (d.T == 0) return hipSuccess;
    const int nch = d.H * 2 / 16;
    hipLaunchKernelGGL(k_combine, dim3((d.T + 3) / 4), dim3(256), 0, s, (const u32x4*)y_in, d.T, d.K, nch,
                       (int)d.out_rows, h->row_id, h->copy_prob, apply_probs, (u32x4*)y_out);
    return hipGetLastError();
}

}  // namespace moe
