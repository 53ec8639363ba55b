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
#include "device_ops.h"

namespace moe {
namespace {

using namespace ops;

template <typename SRC>
__global__ __launch_bounds__(256) void k_quant_rows(const SRC* __restrict__ src, int ncols, long long R,
                                                    const int32_t* __restrict__ src_row, uint8_t* __restrict__ q,
                                                    float* __restrict__ qs) {
    const int lane = threadIdx.x & 63;
    const int nb = ncols / 128;
    const int ngrp = (nb + kQBlocks - 1) / kQBlocks;
    const long long wv = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const long long row = wv / ngrp;
    if (row >= R || src_row[row] < 0) return;
    quant_row_wave(src, ncols, q, qs, row, (int)(wv - row * ngrp) * kQBlocks, lane);
}

template <int MODE>
__global__ __launch_bounds__(256) void k_gemm_fp8(const uint8_t* __restrict__ Xq, const float* __restrict__ Xs,
                                                  const uint8_t* __restrict__ W, const float* __restrict__ Ws,
                                                  void* __restrict__ Outv, const int64_t* __restrict__ seg_off,
                                                  const int32_t* __restrict__ kept, long long R, int Kdim,
                                                  int Wrows, int Nout, int units_per_expert) {
    __shared__ __attribute__((aligned(16))) unsigned char s_w[4 * kWaveLds];   // one weight buffer per wavefront
    const int e = blockIdx.x / units_per_expert;
    const int unit = blockIdx.x - e * units_per_expert;
    const int wave = threadIdx.x >> 6;
    fp8_unit<MODE>(Xq, Xs, W, Ws, Outv, seg_off, kept, R, Kdim, Wrows, Nout, e, unit, threadIdx.x & 63, wave,
                   s_w + wave * kWaveLds);
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
