// Dispatch-permute (K2): copy every kept token row to its destination rows.
//
// Operation: Megatron-LM PR #6800 "Reuse caller-owned HybridEP dispatch and
// expert output buffers" (sections "Summary", "Configuration": permuted tokens
// written into a caller-provided output buffer) and DeepEP PR #716 "perf:
// reuse HybridEP routing allgather buffer" (section "Full HybridEP reference
// validation": dispatch with permutation for BF16 and FP8 payloads).
//
// Token-major: each token's row is read once into registers (16-byte loads)
// and stored to each of the token's k destinations, so HBM sees the
// algorithmic minimum, T row reads + (kept copies) row writes.
// The row is cut into 1 KB pieces (64 16-byte chunks), one wavefront per
// (token, piece): a wavefront loads one 16-byte chunk per lane and stores it
// to each kept destination, with at most two stores in flight, then exits.  Consecutive wavefronts hold
// adjacent pieces of a token, so each destination row is written in bursts
// of adjacent 1 KB pieces.  Measured on MI355X, many short wavefronts write
// faster than few long ones: 0.190 ms at 8192 x 7168, top-8, against 0.200
// ms for one workgroup per token and 0.214 ms for one wavefront per token
// (a 1 GiB fill likewise reaches 6.9 TB/s with one 1 KB store per
// wavefront and 5.6 with sixteen).
// Row writes bypass cache residency (non-temporal stores): the permuted
// buffer is far larger than the last-level cache and is consumed by another
// kernel.  Row reads are ordinary loads: measured on MI355X, non-temporal
// loads in this read-once / write-k pattern cost about a fifth of the rate.
// fp8 rows carry their per-128-column fp32 scales along (slice 0).
#include "device_ops.h"

namespace moe {
namespace {

using namespace ops;

constexpr int kPermSlice = 64;   // chunks per wavefront (one 1 KB piece, one chunk per lane)

__global__ __launch_bounds__(256) void k_permute(const u32x4* __restrict__ x, int T, int K, int nch, int R,
                                                 int nsplit, const int32_t* __restrict__ row_id,
                                                 u32x4* __restrict__ out, const float* __restrict__ xs,
                                                 float* __restrict__ outs, int nsc) {
    const int lane = threadIdx.x & 63;
    // token and piece are wave-uniform: the copies' rows come in one load per
    // wavefront (one per lane), issued with the row chunk
    const int wv = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
    const int t = wv / nsplit;
    if (t >= T) return;
    const int sl = wv - t * nsplit;
    const int c = sl * kPermSlice + lane;
    const u32x4* src = x + (size_t)t * nch;
    const int32_t* rid = row_id + (size_t)t * K;
    for (int j0 = 0; j0 < K; j0 += 64) {
        const int rv = j0 + lane < K ? rid[j0 + lane] : -1;   // copy j0 + l's row in lane l
        u32x4 v = {0u, 0u, 0u, 0u};
        if (c < nch) v = src[c];
        const int nj = min(64, K - j0);
        for (int j = 0; j < nj; ++j) {
            const int r = __builtin_amdgcn_readlane(rv, j);
            if (r < 0 || r >= R) continue;
            if (c < nch) __builtin_nontemporal_store(v, out + (size_t)r * nch + c);
            // at most two stores in flight per wavefront: measured on MI355X,
            // bursts of k stores per wavefront write slower (0.219 against
            // 0.204 ms at 8192 x 7168, top-8), as for a plain fill
            asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
        }
        if (xs && sl == 0) {
            for (int i0 = 0; i0 < nsc; i0 += 64) {
                const int i = i0 + lane;
                const float sv = i < nsc ? xs[(size_t)t * nsc + i] : 0.f;
                for (int j = 0; j < nj; ++j) {
                    const int r = __builtin_amdgcn_readlane(rv, j);
                    if (r < 0 || r >= R) continue;
                    if (i < nsc) outs[(size_t)r * nsc + i] = sv;
                }
            }
        }
    }
}

__global__ __launch_bounds__(256) void k_permute_quant(const uint16_t* __restrict__ x, int H, int T, int K, int R,
                                                       const int32_t* __restrict__ row_id, uint8_t* __restrict__ out,
                                                       float* __restrict__ outs) {
    const int lane = threadIdx.x & 63;
    const int nb = H / 128;
    const int ngrp = (nb + kPQBlocks - 1) / kPQBlocks;
    const long long wv = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const long long t = wv / ngrp;
    if (t >= T) return;
    permute_quant_wave(x, H, K, R, row_id, out, outs, t, (int)(wv - t * ngrp) * kPQBlocks, lane);
}

}  // namespace

hipError_t launch_permute_quant(const moe_handle* h, const void* x, void* out, float* out_scales, hipStream_t s) {
    const moe_desc& d = h->desc;
    if (d.T == 0) return hipSuccess;
    const long long ngrp = (d.H / 128 + kPQBlocks - 1) / kPQBlocks;
    const long long waves = (long long)d.T * ngrp;
    hipLaunchKernelGGL(k_permute_quant, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, (const uint16_t*)x, d.H,
                       d.T, d.K, (int)d.out_rows, h->row_id, (uint8_t*)out, out_scales);
    return hipGetLastError();
}

hipError_t launch_permute(const moe_handle* h, const void* x, const float* x_scales, void* out,
                          float* out_scales, hipStream_t s) {
    const moe_desc& d = h->desc;
    if (d.T == 0) return hipSuccess;
    const bool fp8 = d.payload == MOE_FP8E4M3_B128;
    const int row_bytes = fp8 ? d.H : d.H * 2;
    const int nch = row_bytes / 16;
    const int nsc = fp8 ? d.H / 128 : 0;
    const int nsplit = (nch + kPermSlice - 1) / kPermSlice;
    const long long waves = (long long)d.T * nsplit;
    hipLaunchKernelGGL(k_permute, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, (const u32x4*)x, d.T, d.K, nch,
                       (int)d.out_rows, nsplit, h->row_id, (u32x4*)out, fp8 ? x_scales : nullptr,
                       fp8 ? out_scales : nullptr, nsc);
    return hipGetLastError();
}

}  // namespace moe
