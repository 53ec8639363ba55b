// Grouped expert MLP with fp8 (OCP e4m3) weights and 128x128 fp32 weight
// block scales, W8A8: token rows are quantised per 1x128 block before FC1,
// the SwiGLU output is re-quantised per 1x128 block before FC2.
//
// Operation: Megatron-LM PR #6800 "Reuse caller-owned HybridEP dispatch and
// expert output buffers" (section "Configuration": FP8 expert GEMMs behind the
// dispatch) and TensorRT-LLM PR #16190 "Update CuTeDSL MegaMoE kernels" (first
// and streaming-load commit messages: low-precision expert weights with block
// scales for decode-sized batches).  Quantisation: scale = block amax / 448
// (1 for an all-zero block), code = e4m3(x / scale), round to nearest even,
// saturating at 448; dot products use code * scale.
//
// Design (decode: a few rows per expert, bound by streaming the weights):
//  * k_quant_rows quantises each row that holds a kept copy once per launch
//    (16 lanes per 128-column block, 8 values per lane), so the GEMMs only
//    move codes.  FC1 reads the permuted bf16 rows through it; FC2 reads the
//    fp32 SwiGLU output of FC1 through it.  Both land in the caller's scratch.
//  * GEMM work unit = (expert, 64 features) for FC1 and (expert, 128 output
//    rows) for FC2, one workgroup per unit (experts without rows exit at
//    once); four wavefronts, each owning two 16-row weight tiles: for FC1 the
//    16 gate rows and the matching 16 up rows of 16 features, for FC2 32
//    consecutive rows of W2.  A wavefront streams its weight rows straight from HBM
//    into registers, kU 128-wide K blocks per group so several KB per
//    wavefront are in flight; there is no LDS and no barrier, latency is
//    hidden by the in-flight loads and by occupancy.
//  * v_mfma_scale_f32_16x16x128_f8f6f4 (unit scales) computes one 128-wide K
//    block per instruction: weights are the A operand (16 rows), token codes
//    the B operand (16 columns).  Lane l supplies row/column l%16 and the
//    same 32 bytes of the block for both operands (two 16-byte pieces 64
//    bytes apart, so each load instruction reads 64 contiguous bytes per
//    row); the 16x16 block product is exact; it is multiplied by weight scale x token scale and
//    added into fp32 accumulators (lane l holds column l%16, rows
//    4*(l/16) + i).
//  * Up to 4 token blocks (64 rows) per pass; more rows take more passes.
#include "moe_internal.h"

namespace moe {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxTB = 4;         // token blocks (16 rows) per pass
constexpr int kFeat = 64;         // FC1: features per unit (16 per wavefront: gate + up tile)
constexpr int kFeat2 = 128;       // FC2: output rows per unit (32 per wavefront: two tiles)
constexpr int kU = 4;             // 128-wide K blocks per load group

// ---- row quantiser ------------------------------------------------------------
// Rows r with src_row[r] >= 0 (rows that hold a kept copy): src [R, ncols]
// (bf16 bit patterns or fp32) -> q [R, ncols] e4m3 codes, qs [R, ncols/128]
// scales.  One wavefront per (row, group of 8 column blocks of 128); 16
// lanes per block, 8 values per lane, 4 blocks per step, the loads of both
// steps issued together.
constexpr int kQBlocks = 8;                  // 128-column blocks per wavefront

template <typename SRC>
__global__ __launch_bounds__(256) void k_quant_rows(const SRC* __restrict__ src, int ncols, long long R,
                                                    const int32_t* __restrict__ src_row, uint8_t* __restrict__ q,
                                                    float* __restrict__ qs) {
    constexpr int NIT = kQBlocks / 4;
    const int lane = threadIdx.x & 63;
    const int nb = ncols / 128;
    const int ngrp = (nb + kQBlocks - 1) / kQBlocks;
    const long long wv = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const long long row = wv / ngrp;
    if (row >= R || src_row[row] < 0) return;
    const int b0 = (int)(wv - row * ngrp) * kQBlocks;
    const int g = lane >> 4, l16 = lane & 15;
    const SRC* s = src + (size_t)row * ncols;
    uint8_t* qr = q + (size_t)row * ncols;
    float v[NIT][8];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int b = b0 + 4 * it + g;
        const size_t c = (size_t)b * 128 + l16 * 8;
        if (b < nb) {
            if constexpr (sizeof(SRC) == 2) {
                const u32x4 w = *(const u32x4*)(s + c);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v[it][2 * i] = bf16_lo(w[i]);
                    v[it][2 * i + 1] = bf16_hi(w[i]);
                }
            } else {
                const float4 a = *(const float4*)(s + c), bb = *(const float4*)(s + c + 4);
                v[it][0] = a.x; v[it][1] = a.y; v[it][2] = a.z; v[it][3] = a.w;
                v[it][4] = bb.x; v[it][5] = bb.y; v[it][6] = bb.z; v[it][7] = bb.w;
            }
        }
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int b = b0 + 4 * it + g;
        if (b < nb) {                       // whole 16-lane groups are active or not
            const size_t c = (size_t)b * 128 + l16 * 8;
            float amax = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[it][i]));
            amax = fmaxf(amax, __shfl_xor(amax, 1));
            amax = fmaxf(amax, __shfl_xor(amax, 2));
            amax = fmaxf(amax, __shfl_xor(amax, 4));
            amax = fmaxf(amax, __shfl_xor(amax, 8));
            const float sc = e4m3_scale(amax);
            uint2 out;
            out.x = e4m3_pack4(v[it][0], v[it][1], v[it][2], v[it][3], sc);
            out.y = e4m3_pack4(v[it][4], v[it][5], v[it][6], v[it][7], sc);
            *(uint2*)(qr + c) = out;
            if (l16 == 0) qs[(size_t)row * nb + b] = sc;
        }
    }
}

// The 32 operand bytes of a lane in a 128-wide K block: bytes kq..kq+15 and
// kq+64..kq+79 with kq = 16*(lane/16).  Weights and tokens use the same K
// assignment, so each 128-byte block is covered exactly once, and one load
// instruction reads 64 contiguous bytes of each of its 16 rows.
__device__ __forceinline__ i32x8 load_fp8x32(const uint8_t* p) {
    const u32x4 a = *(const u32x4*)p, b = *(const u32x4*)(p + 64);
    return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

__device__ __forceinline__ f32x4 mfma_fp8(const i32x8& a, const i32x8& b) {
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 127, 0, 127);
}

// One pass over up to 16*NTB rows (m0 .. m0+mv-1 of the segment) for this
// wavefront's two 16-row weight tiles (FC1: gate and up rows of 16 features;
// FC2: 32 consecutive output rows); NTB token blocks of 16 rows.
template <int MODE, int NTB>
__device__ __forceinline__ void fp8_pass(const uint8_t* __restrict__ Xq, const float* __restrict__ Xs,
                                         const uint8_t* wg, const uint8_t* wu, const float* sg, const float* su,
                                         void* __restrict__ Outv, long long seg, int m0, int mv, int Kdim, int Nout,
                                         int f0, int lane) {
    constexpr int U = kU;
    const int kq = (lane >> 4) * 16;
    const int nkb = Kdim / 128;
    f32x4 acc_g[NTB], acc_u[NTB];
#pragma unroll
    for (int t = 0; t < NTB; ++t) {
        acc_g[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc_u[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // token row of this lane in block t: m0 + 16t + lane%16 (clamped)
    size_t xrow[NTB];
#pragma unroll
    for (int t = 0; t < NTB; ++t) xrow[t] = (size_t)(seg + m0 + min(16 * t + (lane & 15), mv - 1));

    // one group of UU K blocks: the weights of all of them are loaded first
    auto group = [&](int kb0, auto uc) {
        constexpr int UU = decltype(uc)::value;
        i32x8 a_g[UU], a_u[UU];
        float s_g[UU], s_u[UU];
#pragma unroll
        for (int u = 0; u < UU; ++u) {
            a_g[u] = load_fp8x32(wg + (size_t)(kb0 + u) * 128);
            a_u[u] = load_fp8x32(wu + (size_t)(kb0 + u) * 128);
            s_g[u] = sg[kb0 + u];
            s_u[u] = su[kb0 + u];
        }
#pragma unroll
        for (int t = 0; t < NTB; ++t) {
#pragma unroll
            for (int u = 0; u < UU; ++u) {
                const i32x8 bq = load_fp8x32(Xq + xrow[t] * Kdim + (size_t)(kb0 + u) * 128 + kq);
                const float sx = Xs[xrow[t] * nkb + kb0 + u];
                const f32x4 pg = mfma_fp8(a_g[u], bq);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc_g[t][i] = fmaf(pg[i], s_g[u] * sx, acc_g[t][i]);
                const f32x4 pu = mfma_fp8(a_u[u], bq);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc_u[t][i] = fmaf(pu[i], s_u[u] * sx, acc_u[t][i]);
            }
        }
    };
    int kb = 0;
    for (; kb + U <= nkb; kb += U) group(kb, std::integral_constant<int, U>{});
    for (; kb < nkb; ++kb) group(kb, std::integral_constant<int, 1>{});

    // ---- epilogue: lane holds token m0+16t+lane%16, features f0+4*(lane/16)+i
#pragma unroll
    for (int t = 0; t < NTB; ++t) {
        const int tok = 16 * t + (lane & 15);
        if (tok >= mv) continue;
        const size_t orow = (size_t)(seg + m0 + tok) * Nout + f0 + 4 * (lane >> 4);
        if (MODE == 0) {
            float4 o;
            float a[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float g = acc_g[t][i], u = acc_u[t][i];
                a[i] = g / (1.f + __expf(-g)) * u;
            }
            o.x = a[0]; o.y = a[1]; o.z = a[2]; o.w = a[3];
            *(float4*)((float*)Outv + orow) = o;
        } else {
            uint2 o;
            o.x = f32_to_bf16(acc_g[t][0]) | (f32_to_bf16(acc_g[t][1]) << 16);
            o.y = f32_to_bf16(acc_g[t][2]) | (f32_to_bf16(acc_g[t][3]) << 16);
            *(uint2*)((uint16_t*)Outv + orow) = o;
            o.x = f32_to_bf16(acc_u[t][0]) | (f32_to_bf16(acc_u[t][1]) << 16);
            o.y = f32_to_bf16(acc_u[t][2]) | (f32_to_bf16(acc_u[t][3]) << 16);
            *(uint2*)((uint16_t*)Outv + orow + 16) = o;
        }
    }
}

// MODE 0: FC1 + SwiGLU.  Xq/Xs = quantised permuted rows [R,H] / [R,H/128];
//         W = W1 [E,2F,H] e4m3, Ws = [E,2F/128,H/128]; Out = fp32 [R,F].
// MODE 1: FC2.  Xq/Xs = quantised activations [R,F] / [R,F/128]; W = W2
//         [E,H,F] e4m3, Ws = [E,H/128,F/128]; Out = bf16 expert output [R,H].
template <int MODE>
__global__ __launch_bounds__(256) void k_gemm_fp8(const uint8_t* __restrict__ Xq, const float* __restrict__ Xs,
                                                  const uint8_t* __restrict__ W, const float* __restrict__ Ws,
                                                  void* __restrict__ Outv, const int64_t* __restrict__ seg_off,
                                                  const int32_t* __restrict__ kept, long long R, int Kdim,
                                                  int Wrows, int Nout, int units_per_expert) {
    const int e = blockIdx.x / units_per_expert;
    const int unit = blockIdx.x - e * units_per_expert;
    const long long seg = seg_off[e];
    long long me_l = seg < R ? (long long)kept[e] : 0;
    if (seg + me_l > R) me_l = R - seg;
    const int me = (int)me_l;
    if (me <= 0) return;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kq = (lane >> 4) * 16;                  // this lane's 32 bytes inside a 128 block
    const int nkb = Kdim / 128;
    // first output feature (FC1) / output row (FC2) of this wavefront; its two
    // weight tiles start at rows r0 and r1 (FC1: gate and up rows of features
    // f0..f0+15; FC2: rows f0..f0+15 and f0+16..f0+31, one 128-row scale block)
    const int f0 = MODE == 0 ? unit * kFeat + wave * 16 : unit * kFeat2 + wave * 32;
    const int r0 = f0, r1 = MODE == 0 ? Nout + f0 : f0 + 16;
    const uint8_t* wg = W + ((size_t)e * Wrows + r0 + (lane & 15)) * Kdim + kq;
    const uint8_t* wu = W + ((size_t)e * Wrows + r1 + (lane & 15)) * Kdim + kq;
    const float* sg = Ws + ((size_t)e * (Wrows / 128) + r0 / 128) * nkb;
    const float* su = Ws + ((size_t)e * (Wrows / 128) + r1 / 128) * nkb;

    for (int m0 = 0; m0 < me; m0 += 16 * kMaxTB) {
        const int mv = min(16 * kMaxTB, me - m0);
        switch ((mv + 15) / 16) {
            case 1: fp8_pass<MODE, 1>(Xq, Xs, wg, wu, sg, su, Outv, seg, m0, mv, Kdim, Nout, f0, lane); break;
            case 2: fp8_pass<MODE, 2>(Xq, Xs, wg, wu, sg, su, Outv, seg, m0, mv, Kdim, Nout, f0, lane); break;
            case 3: fp8_pass<MODE, 3>(Xq, Xs, wg, wu, sg, su, Outv, seg, m0, mv, Kdim, Nout, f0, lane); break;
            default: fp8_pass<MODE, 4>(Xq, Xs, wg, wu, sg, su, Outv, seg, m0, mv, Kdim, Nout, f0, lane); break;
        }
    }
}

size_t up256(size_t n) { return (n + 255) & ~(size_t)255; }

}  // namespace

// Scratch of the fp8 path, in this order: fp32 SwiGLU activations [R,F],
// token codes [R,H] and scales [R,H/128], activation codes [R,F] and scales
// [R,F/128]; each region starts on a 256-byte boundary.
size_t fp8_mlp_scratch_bytes(long long R, int H, int F) {
    const size_t r = (size_t)R;
    return up256(r * F * 4) + up256(r * H) + up256(r * (H / 128) * 4) + up256(r * F) + up256(r * (F / 128) * 4);
}

hipError_t launch_gemm_fp8(const moe_handle* h, int stage, int F, const void* in, const float* in_scales,
                           const void* w, const float* ws, void* scratch, void* out, hipStream_t s) {
    const moe_desc& d = h->desc;
    const long long R = d.out_rows;
    if (R == 0) return hipSuccess;
    char* base = (char*)scratch;
    float* act = (float*)base;
    uint8_t* xq = (uint8_t*)(base + up256((size_t)R * F * 4));
    float* xs = (float*)((char*)xq + up256((size_t)R * d.H));
    uint8_t* aq = (uint8_t*)((char*)xs + up256((size_t)R * (d.H / 128) * 4));
    float* as = (float*)((char*)aq + up256((size_t)R * F));
    auto qgrid = [&](int ncols) {   // (row, block group) wavefronts, four per workgroup
        const long long ngrp = (ncols / 128 + kQBlocks - 1) / kQBlocks;
        return (unsigned)((R * ngrp + 3) / 4);
    };
    if (stage == 0) {
        const uint8_t* q = xq;
        const float* qs = xs;
        if (in_scales) {   // rows quantised on dispatch
            q = (const uint8_t*)in;
            qs = in_scales;
        } else {
            hipLaunchKernelGGL(k_quant_rows<uint16_t>, dim3(qgrid(d.H)), dim3(256), 0, s, (const uint16_t*)in, d.H,
                               R, h->src_row, xq, xs);
        }
        const int upe = F / kFeat;
        hipLaunchKernelGGL(k_gemm_fp8<0>, dim3(d.E * upe), dim3(256), 0, s, q, qs, (const uint8_t*)w, ws, act,
                           h->seg_off, h->kept, R, d.H, 2 * F, F, upe);
    } else {
        hipLaunchKernelGGL(k_quant_rows<float>, dim3(qgrid(F)), dim3(256), 0, s, act, F, R, h->src_row, aq, as);
        const int upe = d.H / kFeat2;
        hipLaunchKernelGGL(k_gemm_fp8<1>, dim3(d.E * upe), dim3(256), 0, s, aq, as, (const uint8_t*)w, ws, out,
                           h->seg_off, h->kept, R, F, d.H, d.H, upe);
    }
    return hipGetLastError();
}

}  // namespace moe
