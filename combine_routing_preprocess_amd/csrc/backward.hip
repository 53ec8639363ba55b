// Backward of dispatch and of combine (token, row and probability gradients).
//
// Operation: DeepEP PR #716 "perf: reuse HybridEP routing allgather buffer"
// (section "Full HybridEP reference validation": hidden-state and probability
// gradients of the backward-of-dispatch and backward-of-combine) and
// NeMo-Automodel PR #3931 "perf(moe): sync-free HybridEP dispatch" (section
// "What does this PR do ?": the combine's backward is a dispatch sized by the
// same host-known row count, so it needs no host sync either).
//
//  * Dispatch backward: a token's gradient is the sum of its kept copies'
//    row gradients, which is the combine with unit weights (the combine
//    kernel runs it); the probability gradient of copy (t, j) is its row's
//    gradient, gathered into the routing's shape.
//  * Combine backward: the token's gradient row is held in registers by one
//    to four wavefronts (column slices); for each kept copy they write
//    w * grad_y to the copy's row (w = the copy probability, or 1) and, when
//    probabilities were applied, reduce grad_y . Y[row] in fp32 for the
//    probability gradient (per lane in column order, a fixed butterfly
//    across the lanes, then the slices in order).
//  * Probability gradients in a Boolean-map routing live at [t, e]; the
//    expert of a row is found by binary search of the segment offsets, and
//    the [T, E] table is cleared by a fill kernel first (no memset node, so
//    the sequence stays safe to capture in a graph).
#include "moe_internal.h"

namespace moe {
namespace {

// Expert whose segment holds row r: the largest e in [0, E) with
// seg_off[e] <= r (empty segments share their offset with the next one).
__device__ __forceinline__ int expert_of(const int64_t* __restrict__ seg_off, int E, int r) {
    int lo = 0, hi = E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (seg_off[mid] <= (int64_t)r) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// bf16 of the exact product w * x (one rounding, nearest-even).  The fp32
// product p is the exact product rounded; the only case where rounding p to
// bf16 differs from rounding the exact product is p sitting exactly on a bf16
// midpoint (midpoints are fp32 values) while the exact product is not: the
// rounding error e = fma(w, x, -p) then says which side the product lies on.
__device__ __forceinline__ uint32_t bf16_mul_rn(float w, float x) {
    const float p = w * x;
    const uint32_t u = __float_as_uint(p);
    if ((u & 0xffffu) == 0x8000u) {
        const float e = fmaf(w, x, -p);
        if (e != 0.f) return (u >> 16) + (((e > 0.f) == (p > 0.f)) ? 1u : 0u);
    }
    return f32_to_bf16(p);
}

__global__ __launch_bounds__(256) void k_fill_zero(float* __restrict__ p, long long n) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0.f;
}

// Dispatch backward, probabilities: one thread per copy (t, j).
__global__ __launch_bounds__(256) void k_probs_gather(const int32_t* __restrict__ row_id,
                                                      const float* __restrict__ grad_row_probs,
                                                      const int64_t* __restrict__ seg_off, int T, int K, int E,
                                                      int R, int sparse, float* __restrict__ grad_probs) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= (long long)T * K) return;
    const int r = row_id[i];
    const bool kept = r >= 0 && r < R;
    if (!sparse) {
        grad_probs[i] = kept ? grad_row_probs[r] : 0.f;
    } else if (kept) {
        const long long t = i / K;
        grad_probs[t * E + expert_of(seg_off, E, r)] = grad_row_probs[r];
    }
}

// Combine backward: a token's row is cut into 1 KB pieces (64 16-byte
// chunks), one wavefront per piece, as many tokens per 16-wavefront
// workgroup as fit whole (one token of up to 16 pieces, 8192 bf16).  Each
// wavefront holds its chunk of grad_y in registers; per copy it issues the
// expert-output load, writes the row gradient, then reduces its partial dot
// product (butterfly) into LDS.  After a workgroup barrier the first
// wavefront of each token adds the pieces' partials in piece order.  Row ids
// and probabilities are loaded one copy ahead.  Measured on MI355X at 8192 x
// 7168, top-8, many short wavefronts beat fewer long ones here as in the
// permute: 0.404 ms against 0.415 ms with 4 KB slices of four wavefronts.
__global__ __launch_bounds__(1024) void k_combine_backward(const u32x4* __restrict__ gy, const u32x4* __restrict__ Y,
                                                           int T, int K, int E, int nch, int R, int nsl,
                                                           const int32_t* __restrict__ row_id,
                                                           const float* __restrict__ copy_prob, int apply,
                                                           const int64_t* __restrict__ seg_off, int sparse,
                                                           u32x4* __restrict__ gY, float* __restrict__ grad_probs) {
    extern __shared__ float part[];   // [16][K] per-wavefront partial dot of each copy
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int tpb = 16 / nsl;   // tokens per workgroup
    const int t = blockIdx.x * tpb + wave / nsl;
    const int c = (wave % nsl) * 64 + lane;
    const bool active = t < T && wave < tpb * nsl;
    const bool in_row = c < nch;
    const bool want_dot = grad_probs != nullptr && apply;
    if (active) {
        const u32x4 g = in_row ? gy[(size_t)t * nch + c] : u32x4{0u, 0u, 0u, 0u};
        const int32_t* rid = row_id + (size_t)t * K;
        const float* cp = copy_prob + (size_t)t * K;
        int r_next = rid[0];
        float w_next = apply ? cp[0] : 1.f;
        for (int j = 0; j < K; ++j) {
            const int r = r_next;
            const float w = w_next;
            if (j + 1 < K) {
                r_next = rid[j + 1];
                w_next = apply ? cp[j + 1] : 1.f;
            }
            if (r < 0 || r >= R) {
                if (want_dot && lane == 0) part[wave * K + j] = 0.f;
                continue;
            }
            u32x4 y = {0u, 0u, 0u, 0u};
            if (want_dot && in_row) y = __builtin_nontemporal_load(Y + (size_t)r * nch + c);
            if (in_row) {
                u32x4 o;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    o[q] = bf16_mul_rn(w, bf16_lo(g[q])) | (bf16_mul_rn(w, bf16_hi(g[q])) << 16);
                __builtin_nontemporal_store(o, gY + (size_t)r * nch + c);
            }
            if (want_dot) {
                float dot = 0.f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    dot = fmaf(bf16_lo(g[q]), bf16_lo(y[q]), dot);
                    dot = fmaf(bf16_hi(g[q]), bf16_hi(y[q]), dot);
                }
#pragma unroll
                for (int m = 32; m >= 1; m >>= 1) dot += __shfl_xor(dot, m, 64);
                if (lane == 0) part[wave * K + j] = dot;
            }
        }
    }
    if (grad_probs == nullptr) return;   // uniform over the workgroup
    __syncthreads();
    if (!active || wave % nsl != 0) return;
    for (int j = lane; j < K; j += 64) {
        const int r = row_id[(size_t)t * K + j];
        const bool kept = r >= 0 && r < R;
        float v = 0.f;
        if (want_dot && kept)
            for (int s2 = 0; s2 < nsl; ++s2) v += part[(wave + s2) * K + j];
        if (!sparse) grad_probs[(size_t)t * K + j] = v;
        else if (kept) grad_probs[(size_t)t * E + expert_of(seg_off, E, r)] = v;
    }
}

// One wavefront per token for rows longer than 16 pieces of 64 chunks: the
// gradient row is re-read from cache for every copy.
__global__ __launch_bounds__(256) void k_combine_backward_long(const u32x4* __restrict__ gy,
                                                               const u32x4* __restrict__ Y, int T, int K, int E,
                                                               int nch, int R, const int32_t* __restrict__ row_id,
                                                               const float* __restrict__ copy_prob, int apply,
                                                               const int64_t* __restrict__ seg_off, int sparse,
                                                               u32x4* __restrict__ gY, float* __restrict__ grad_probs) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const bool want_dot = grad_probs != nullptr && apply;
    const u32x4* src = gy + (size_t)t * nch;
    for (int j = 0; j < K; ++j) {
        const int r = row_id[(size_t)t * K + j];
        const bool kept = r >= 0 && r < R;
        if (!kept) {
            if (grad_probs && !sparse && lane == 0) grad_probs[(size_t)t * K + j] = 0.f;
            continue;
        }
        const float w = apply ? copy_prob[(size_t)t * K + j] : 1.f;
        u32x4* dst = gY + (size_t)r * nch;
        const u32x4* yr = want_dot ? Y + (size_t)r * nch : nullptr;
        float dot = 0.f;
        for (int c = lane; c < nch; c += 64) {
            const u32x4 gv = src[c];
            if (want_dot) {
                const u32x4 yv = __builtin_nontemporal_load(yr + c);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    dot = fmaf(bf16_lo(gv[q]), bf16_lo(yv[q]), dot);
                    dot = fmaf(bf16_hi(gv[q]), bf16_hi(yv[q]), dot);
                }
            }
            u32x4 o;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                o[q] = bf16_mul_rn(w, bf16_lo(gv[q])) | (bf16_mul_rn(w, bf16_hi(gv[q])) << 16);
            __builtin_nontemporal_store(o, dst + c);
        }
        if (grad_probs) {
            if (want_dot) {
#pragma unroll
                for (int m = 32; m >= 1; m >>= 1) dot += __shfl_xor(dot, m, 64);
            }
            if (lane == 0) {
                const size_t at = sparse ? (size_t)t * E + expert_of(seg_off, E, r) : (size_t)t * K + j;
                grad_probs[at] = want_dot ? dot : 0.f;
            }
        }
    }
}

constexpr int kMaxPieces = 16;   // 1 KB pieces per row in one workgroup (rows up to 8192 bf16)

hipError_t fill_zero(float* p, long long n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_probs_gather(const moe_handle* h, const float* grad_row_probs, float* grad_probs,
                               hipStream_t s) {
    const moe_desc& d = h->desc;
    if (d.T == 0) return hipSuccess;
    const int sparse = d.route_fmt == MOE_ROUTE_SPARSE_BOOL;
    if (sparse) {
        hipError_t e = fill_zero(grad_probs, (long long)d.T * d.E, s);
        if (e != hipSuccess) return e;
    }
    const long long n = (long long)d.T * d.K;
    hipLaunchKernelGGL(k_probs_gather, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, h->row_id,
                       grad_row_probs, h->seg_off, d.T, d.K, d.E, (int)d.out_rows, sparse, grad_probs);
    return hipGetLastError();
}

hipError_t launch_combine_backward(const moe_handle* h, const void* grad_y, const void* expert_out,
                                   int apply_probs, void* grad_expert_out, float* grad_probs, hipStream_t s) {
    const moe_desc& d = h->desc;
    if (d.T == 0) return hipSuccess;
    const int sparse = d.route_fmt == MOE_ROUTE_SPARSE_BOOL;
    if (sparse && grad_probs) {
        hipError_t e = fill_zero(grad_probs, (long long)d.T * d.E, s);
        if (e != hipSuccess) return e;
    }
    const int nch = d.H * 2 / 16;
    const int nsl = (nch + 63) / 64;
    if (nsl <= kMaxPieces) {
        const int tpb = kMaxPieces / nsl;
        const size_t lds = grad_probs ? (size_t)kMaxPieces * d.K * sizeof(float) : 0;
        hipLaunchKernelGGL(k_combine_backward, dim3((unsigned)((d.T + tpb - 1) / tpb)), dim3(64 * kMaxPieces), lds, s,
                           (const u32x4*)grad_y, (const u32x4*)expert_out, d.T, d.K, d.E, nch, (int)d.out_rows, nsl,
                           h->row_id, h->copy_prob, apply_probs, h->seg_off, sparse, (u32x4*)grad_expert_out,
                           grad_probs);
    } else {
        const dim3 grid((unsigned)((d.T + 3) / 4));
        hipLaunchKernelGGL(k_combine_backward_long, grid, dim3(256), 0, s, (const u32x4*)grad_y,
                           (const u32x4*)expert_out, d.T, d.K, d.E, nch, (int)d.out_rows, h->row_id, h->copy_prob,
                           apply_probs, h->seg_off, sparse, (u32x4*)grad_expert_out, grad_probs);
    }
    return hipGetLastError();
}

}  // namespace moe
