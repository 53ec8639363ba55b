// Grouped expert MLP with fp8 (OCP e4m3) weights and 128x128 fp32 weight
// block scales, W8A8: token rows are quantised per 1x128 block on load, the
// SwiGLU output is re-quantised per 1x128 block on FC2's load.
//
// Operation: Megatron-LM PR #6800 "Reuse caller-owned HybridEP dispatch and
// expert output buffers" (section "Configuration": FP8 expert GEMMs behind the
// dispatch) and TensorRT-LLM PR #16190 "Update CuTeDSL MegaMoE kernels" (first
// and streaming-load commit messages: low-precision expert weights with block
// scales for decode-sized batches).  Quantisation: scale = block amax / 448
// (1 for an all-zero block), code = e4m3(x / scale), round to nearest even,
// saturating at 448; dot products use code * scale.
//
// Design (decode: few rows per expert, weight streaming bound):
//  * Work unit = (expert, 64 output features).  One workgroup per unit
//    (experts without rows exit at once); four wavefronts, each owning 16
//    features: for FC1 its 16 gate rows and the matching 16 up rows, for FC2
//    16 rows of W2.  A wavefront streams its weight rows straight from HBM to
//    registers; there is no LDS and no barrier, so latency is hidden by
//    occupancy (the kernel needs few registers).
//  * v_mfma_scale_f32_16x16x128_f8f6f4 (unit scales) computes one 128-wide K
//    block per instruction: weights are the A operand (16 rows), tokens the B
//    operand (16 columns).  Lane l supplies row/column l%16 and the 32 K
//    values (l/16)*32 .. +31 of the block for both operands, so the 16x16
//    block product is exact; its result is multiplied by weight scale x token
//    scale and added into fp32 accumulators (lane l holds column l%16, rows
//    4*(l/16) + i).
//  * Token quantisation on load: the four lanes holding a token's 128 values
//    of a block combine their maxima with two xor-shuffles, then each converts
//    its 32 values (fp32 divide, hardware e4m3 conversion after clamping).
//  * Up to 4 token blocks (64 rows) per pass; more rows take more passes.
#include "moe_internal.h"

namespace moe {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxTB = 4;         // token blocks (16 rows) per pass
constexpr int kFeat = 64;         // output features per unit

__device__ __forceinline__ float e4m3_prep(float v) {   // saturate to the e4m3 range
    return fminf(fmaxf(v, -448.f), 448.f);
}

// 32 values of one lane (fp32) -> 32 e4m3 codes for the MFMA operand, with
// the 128-wide block scale shared by the 4 lanes l, l^16, l^32, l^48.
__device__ __forceinline__ i32x8 quant32(const float (&v)[32], float& scale) {
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    const float s = amax > 0.f ? amax / 448.f : 1.f;
    scale = s;
    i32x8 q;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        int p = 0;
        p = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_prep(v[4 * w + 0] / s), e4m3_prep(v[4 * w + 1] / s), p, false);
        p = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_prep(v[4 * w + 2] / s), e4m3_prep(v[4 * w + 3] / s), p, true);
        q[w] = p;
    }
    return q;
}

__device__ __forceinline__ void load_bf16x32(const uint16_t* p, float (&v)[32]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const u32x4 w = *(const u32x4*)(p + 8 * c);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[8 * c + 2 * i] = bf16_lo(w[i]);
            v[8 * c + 2 * i + 1] = bf16_hi(w[i]);
        }
    }
}

__device__ __forceinline__ void load_f32x32(const float* p, float (&v)[32]) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const float4 w = *(const float4*)(p + 4 * c);
        v[4 * c] = w.x;
        v[4 * c + 1] = w.y;
        v[4 * c + 2] = w.z;
        v[4 * c + 3] = w.w;
    }
}

__device__ __forceinline__ i32x8 load_fp8x32(const uint8_t* p) {
    const u32x4 a = *(const u32x4*)p, b = *(const u32x4*)(p + 16);
    return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

__device__ __forceinline__ f32x4 mfma_fp8(const i32x8& a, const i32x8& b) {
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 127, 0, 127);
}

// MODE 0: FC1 + SwiGLU.  X = permuted bf16 rows [R,H]; W = W1 [E,2F,H] e4m3,
//         Ws = [E,2F/128,H/128]; Out = fp32 activations [R,F].
// MODE 1: FC2.  X = fp32 activations [R,F]; W = W2 [E,H,F] e4m3,
//         Ws = [E,H/128,F/128]; Out = bf16 expert output [R,H].
template <int MODE>
__global__ __launch_bounds__(256) void k_gemm_fp8(const void* __restrict__ Xv, const uint8_t* __restrict__ W,
                                                  const float* __restrict__ Ws, void* __restrict__ Outv,
                                                  const int64_t* __restrict__ seg_off,
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
    const int kq = (lane >> 4) * 32;                  // this lane's 32 K values inside a 128 block
    const int nkb = Kdim / 128;
    const int f0 = unit * kFeat + wave * 16;          // first output feature of this wavefront
    const int ksb = Kdim / 128;                        // scale blocks along K
    // weight rows of this lane: gate (and up) row f0 + lane%16
    const int r_g = f0 + (lane & 15);
    const uint8_t* wg = W + ((size_t)e * Wrows + r_g) * Kdim + kq;
    const uint8_t* wu = W + ((size_t)e * Wrows + (MODE == 0 ? Nout + r_g : r_g)) * Kdim + kq;
    const float* sg = Ws + ((size_t)e * (Wrows / 128) + f0 / 128) * ksb;
    const float* su = Ws + ((size_t)e * (Wrows / 128) + (MODE == 0 ? (Nout + f0) / 128 : f0 / 128)) * ksb;

    for (int m0 = 0; m0 < me; m0 += 16 * kMaxTB) {
        const int mv = min(16 * kMaxTB, me - m0);
        const int ntb = (mv + 15) / 16;
        f32x4 acc_g[kMaxTB], acc_u[kMaxTB];
#pragma unroll
        for (int t = 0; t < kMaxTB; ++t) {
            acc_g[t] = f32x4{0.f, 0.f, 0.f, 0.f};
            acc_u[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        // token row of this lane in block t: m0 + 16t + lane%16 (clamped)
        size_t xrow[kMaxTB];
#pragma unroll
        for (int t = 0; t < kMaxTB; ++t)
            xrow[t] = (size_t)(seg + m0 + min(16 * t + (lane & 15), mv - 1)) * Kdim + kq;

        for (int kb = 0; kb < nkb; ++kb) {
            const i32x8 a_g = load_fp8x32(wg + kb * 128);
            i32x8 a_u;
            if (MODE == 0) a_u = load_fp8x32(wu + kb * 128);
            const float s_g = sg[kb];
            const float s_u = MODE == 0 ? su[kb] : 0.f;
#pragma unroll
            for (int t = 0; t < kMaxTB; ++t) {
                if (t >= ntb) break;
                float v[32];
                if (MODE == 0) load_bf16x32((const uint16_t*)Xv + xrow[t] + kb * 128, v);
                else load_f32x32((const float*)Xv + xrow[t] + kb * 128, v);
                float sx;
                const i32x8 bq = quant32(v, sx);
                const f32x4 pg = mfma_fp8(a_g, bq);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc_g[t][i] = fmaf(pg[i], s_g * sx, acc_g[t][i]);
                if (MODE == 0) {
                    const f32x4 pu = mfma_fp8(a_u, bq);
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc_u[t][i] = fmaf(pu[i], s_u * sx, acc_u[t][i]);
                }
            }
        }
        // ---- epilogue: lane holds token m0+16t+lane%16, features f0+4*(lane/16)+i
#pragma unroll
        for (int t = 0; t < kMaxTB; ++t) {
            const int tok = 16 * t + (lane & 15);
            if (t >= ntb || tok >= mv) continue;
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
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm_fp8(const moe_handle* h, int stage, int F, const void* in, const void* w,
                           const float* ws, void* out, hipStream_t s) {
    const moe_desc& d = h->desc;
    const long long R = d.out_rows;
    if (R == 0) return hipSuccess;
    if (stage == 0) {
        const int upe = F / kFeat;
        hipLaunchKernelGGL(k_gemm_fp8<0>, dim3(d.E * upe), dim3(256), 0, s, in, (const uint8_t*)w, ws, out,
                           h->seg_off, h->kept, R, d.H, 2 * F, F, upe);
    } else {
        const int upe = d.H / kFeat;
        hipLaunchKernelGGL(k_gemm_fp8<1>, dim3(d.E * upe), dim3(256), 0, s, in, (const uint8_t*)w, ws, out,
                           h->seg_off, h->kept, R, F, d.H, d.H, upe);
    }
    return hipGetLastError();
}

}  // namespace moe
