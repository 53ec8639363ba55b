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
// Token-major.  Each lane owns 16-byte column chunks and sums the token's
// copies in slot order with fused multiply-adds, so the result does not
// depend on scheduling.  The loads of four copies are issued before their
// multiply-adds.  Expert-output rows are read once (non-temporal); output
// rows are written once.
//  * Large batches (k_combine_wg): one workgroup of four wavefronts per
//    token, the row's 1 KB pieces dealt to the wavefronts in turn, so each
//    expert-output row is read in 4 KB bursts (0.182 against 0.195 ms for
//    one wavefront per token at 8192 x 7168, top-8, on MI355X).
//  * Small batches (k_combine): a token's row is cut into `nsplit` column
//    slices so that enough wavefronts run; one wavefront per (token, slice).
#include "device_ops.h"

namespace moe {
namespace {

using namespace ops;

__global__ __launch_bounds__(256) void k_combine(const u32x4* __restrict__ Y, int T, int K, int nch, int R,
                                                 int nsplit, int slice_ch, const int32_t* __restrict__ row_id,
                                                 const float* __restrict__ copy_prob, int apply,
                                                 u32x4* __restrict__ y) {
    const int lane = threadIdx.x & 63;
    const int wv = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int t = wv / nsplit;
    if (t >= T) return;
    const int cs = (wv - t * nsplit) * slice_ch;
    const int ce = min(nch, cs + slice_ch);
    const int32_t* rid = row_id + (size_t)t * K;
    const float* cp = copy_prob + (size_t)t * K;
    for (int c0 = cs; c0 < ce; c0 += 64 * kCombU) {
        float acc[kCombU][8];
#pragma unroll
        for (int u = 0; u < kCombU; ++u)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[u][i] = 0.f;
        for (int j0 = 0; j0 < K; j0 += kCombJ) {
            u32x4 v[kCombJ][kCombU];
            float pj[kCombJ];
            bool ok[kCombJ];
#pragma unroll
            for (int jj = 0; jj < kCombJ; ++jj) {
                const int j = j0 + jj;
                const int r = j < K ? rid[j] : -1;
                ok[jj] = r >= 0 && r < R;
                pj[jj] = ok[jj] ? (apply ? cp[j] : 1.f) : 0.f;
                const u32x4* src = Y + (size_t)(ok[jj] ? r : 0) * nch;
#pragma unroll
                for (int u = 0; u < kCombU; ++u) {
                    const int c = c0 + u * 64 + lane;
                    v[jj][u] = (ok[jj] && c < ce) ? __builtin_nontemporal_load(src + c) : u32x4{0u, 0u, 0u, 0u};
                }
            }
#pragma unroll
            for (int jj = 0; jj < kCombJ; ++jj) {
                if (!ok[jj]) continue;
#pragma unroll
                for (int u = 0; u < kCombU; ++u)
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        acc[u][2 * w] = fmaf(pj[jj], bf16_lo(v[jj][u][w]), acc[u][2 * w]);
                        acc[u][2 * w + 1] = fmaf(pj[jj], bf16_hi(v[jj][u][w]), acc[u][2 * w + 1]);
                    }
            }
        }
#pragma unroll
        for (int u = 0; u < kCombU; ++u) {
            const int c = c0 + u * 64 + lane;
            if (c < ce) {
                u32x4 o;
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    o[w] = bf16x2_rne(acc[u][2 * w], acc[u][2 * w + 1]);
                y[(size_t)t * nch + c] = o;
            }
        }
    }
}

// Large batches: one workgroup per token; wavefront w owns the row's 1 KB
// pieces w, w+4, w+8, ... (64 16-byte chunks each).  Same arithmetic as
// k_combine.
constexpr int kWgMinTokens = 4096;   // below this, the sliced kernel keeps more wavefronts busy

__global__ __launch_bounds__(256) void k_combine_wg(const u32x4* __restrict__ Y, int T, int K, int nch, int R,
                                                   const int32_t* __restrict__ row_id,
                                                   const float* __restrict__ copy_prob, int apply,
                                                   u32x4* __restrict__ y) {
    const int t = blockIdx.x;
    if (t >= T) return;
    combine_token_wg(Y, K, nch, R, row_id, copy_prob, apply, y, t, threadIdx.x >> 6, threadIdx.x & 63);
}

// Combine from the fp8 format: expert-output rows are e4m3 codes with one
// fp32 scale per 128 columns.  Same work split (a workgroup per token for
// large batches, column slices otherwise) and copy look-ahead as the bf16
// combine; a 16-byte chunk holds 16 codes of one 128-column block,
// dequantised as code value * scale in fp32 before the probability-weighted
// fma.
constexpr int kCombQU = 2;   // 16-byte chunks (16 codes) per lane per pass

__global__ __launch_bounds__(256) void k_combine_fp8(const u32x4* __restrict__ Yq, const float* __restrict__ Ys,
                                                     int T, int K, int nch, int R, int nsplit, int slice_ch,
                                                     const int32_t* __restrict__ row_id,
                                                     const float* __restrict__ copy_prob, int apply,
                                                     u32x4* __restrict__ y) {
    // nsplit == 0: one workgroup per token, the row's 64-chunk pieces dealt
    // to its four wavefronts in turn (as k_combine_wg); else one wavefront per
    // (token, slice of slice_ch chunks)
    const int lane = threadIdx.x & 63, w4 = threadIdx.x >> 6;
    const bool wg = nsplit == 0;
    const int wv = blockIdx.x * 4 + w4;
    const int t = wg ? (int)blockIdx.x : wv / nsplit;
    if (t >= T) return;
    const int cs = wg ? 0 : (wv - t * nsplit) * slice_ch;
    const int ce = wg ? nch : min(nch, cs + slice_ch);
    const int step = wg ? 4 * 64 * kCombQU : 64 * kCombQU;
    // chunk of slot u in the pass starting at c0
    auto col = [&](int c0, int u) { return wg ? c0 + (u * 4 + w4) * 64 + lane : c0 + u * 64 + lane; };
    const int nsb = nch / 8;   // scales per row
    const int32_t* rid = row_id + (size_t)t * K;
    const float* cp = copy_prob + (size_t)t * K;
    for (int c0 = cs; c0 < ce; c0 += step) {
        float acc[kCombQU][16];
#pragma unroll
        for (int u = 0; u < kCombQU; ++u)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[u][i] = 0.f;
        for (int j0 = 0; j0 < K; j0 += kCombJ) {
            u32x4 v[kCombJ][kCombQU];
            float sc[kCombJ][kCombQU];
            float pj[kCombJ];
            bool ok[kCombJ];
#pragma unroll
            for (int jj = 0; jj < kCombJ; ++jj) {
                const int j = j0 + jj;
                const int r = j < K ? rid[j] : -1;
                ok[jj] = r >= 0 && r < R;
                pj[jj] = ok[jj] ? (apply ? cp[j] : 1.f) : 0.f;
                const size_t rr = (size_t)(ok[jj] ? r : 0);
#pragma unroll
                for (int u = 0; u < kCombQU; ++u) {
                    const int c = col(c0, u);
                    const bool in = ok[jj] && c < ce;
                    v[jj][u] = in ? __builtin_nontemporal_load(Yq + rr * nch + c) : u32x4{0u, 0u, 0u, 0u};
                    sc[jj][u] = in ? Ys[rr * nsb + (c >> 3)] : 0.f;
                }
            }
#pragma unroll
            for (int jj = 0; jj < kCombJ; ++jj) {
                if (!ok[jj]) continue;
#pragma unroll
                for (int u = 0; u < kCombQU; ++u)
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[jj][u][w], false);
                        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[jj][u][w], true);
                        const float s_ = sc[jj][u];
                        acc[u][4 * w + 0] = fmaf(pj[jj], lo[0] * s_, acc[u][4 * w + 0]);
                        acc[u][4 * w + 1] = fmaf(pj[jj], lo[1] * s_, acc[u][4 * w + 1]);
                        acc[u][4 * w + 2] = fmaf(pj[jj], hi[0] * s_, acc[u][4 * w + 2]);
                        acc[u][4 * w + 3] = fmaf(pj[jj], hi[1] * s_, acc[u][4 * w + 3]);
                    }
            }
        }
#pragma unroll
        for (int u = 0; u < kCombQU; ++u) {
            const int c = col(c0, u);
            if (c < ce) {
                u32x4 o0, o1;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    o0[w] = bf16x2_rne(acc[u][2 * w], acc[u][2 * w + 1]);
                    o1[w] = bf16x2_rne(acc[u][8 + 2 * w], acc[u][8 + 2 * w + 1]);
                }
                y[((size_t)t * nch + c) * 2] = o0;
                y[((size_t)t * nch + c) * 2 + 1] = o1;
            }
        }
    }
}

}  // namespace

hipError_t launch_combine_fp8(const moe_handle* h, const void* yq, const float* ys, int apply_probs, void* y_out,
                              hipStream_t s) {
    const moe_desc& d = h->desc;
    if (d.T == 0) return hipSuccess;
    const int nch = d.H / 16;
    int nsplit, slice_ch;
    row_slices(d.T, nch, &nsplit, &slice_ch);
    long long waves = (long long)d.T * nsplit;
    if (d.T >= kWgMinTokens) {   // one workgroup per token
        nsplit = 0;
        waves = 4LL * d.T;
    }
    hipLaunchKernelGGL(k_combine_fp8, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, (const u32x4*)yq, ys, d.T,
                       d.K, nch, (int)d.out_rows, nsplit, slice_ch, h->row_id, h->copy_prob, apply_probs,
                       (u32x4*)y_out);
    return hipGetLastError();
}

hipError_t launch_combine(const moe_handle* h, const void* y_in, int apply_probs, void* y_out,
                          hipStream_t s) {
    const moe_desc& d = h->desc;
    if (d.T == 0) return hipSuccess;
    const int nch = d.H * 2 / 16;
    if (d.T >= kWgMinTokens) {
        hipLaunchKernelGGL(k_combine_wg, dim3((unsigned)d.T), dim3(256), 0, s, (const u32x4*)y_in, d.T, d.K, nch,
                           (int)d.out_rows, h->row_id, h->copy_prob, apply_probs, (u32x4*)y_out);
        return hipGetLastError();
    }
    int nsplit, slice_ch;
    row_slices(d.T, nch, &nsplit, &slice_ch);
    const long long waves = (long long)d.T * nsplit;
    hipLaunchKernelGGL(k_combine, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, (const u32x4*)y_in, d.T, d.K,
                       nch, (int)d.out_rows, nsplit, slice_ch, h->row_id, h->copy_prob, apply_probs, (u32x4*)y_out);
    return hipGetLastError();
}

}  // namespace moe
