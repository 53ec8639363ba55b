// Device-side building blocks shared by the expert-MLP, dispatch and combine
// kernels and by the persistent decode layer (one workgroup or one wavefront
// of work each; the kernels around them only pick the indices).
#pragma once
#include "moe_internal.h"

namespace moe {
namespace ops {

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

// One wavefront's share of the row quantiser: row `row`, 128-column blocks
// b0 .. b0+kQBlocks-1 (16 lanes per block, 8 values per lane, 4 blocks per
// step, the loads of both steps issued together).
template <typename SRC>
__device__ __forceinline__ void quant_row_wave(const SRC* __restrict__ src, int ncols, uint8_t* __restrict__ q,
                                               float* __restrict__ qs, long long row, int b0, int lane) {
    constexpr int NIT = kQBlocks / 4;
    const int nb = ncols / 128;
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

// SwiGLU of one feature: silu(gate) * up.
__device__ __forceinline__ float swiglu(float g, float u) { return g / (1.f + __expf(-g)) * u; }

// The 32 operand bytes of a lane in a 128-wide K block: bytes kq..kq+15 and
// kq+64..kq+79 with kq = 16*(lane/16).  Weights and tokens use the same K
// assignment, so each 128-byte block is covered exactly once.  Token operands
// are loaded this way (a few rows, from L2); weights go through wl_load.
__device__ __forceinline__ i32x8 load_fp8x32(const uint8_t* p) {
    const u32x4 a = *(const u32x4*)p, b = *(const u32x4*)(p + 64);
    return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

__device__ __forceinline__ f32x4 mfma_fp8(const i32x8& a, const i32x8& b) {
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 127, 0, 127);
}

// Weight tiles through a wavefront-private LDS buffer: the loads read whole
// 128-byte lines (load (u, i) covers rows 8*(i&1) + lane/8 of tile i/2 at K
// block u, 16 bytes per lane) with the non-temporal policy (weights are read
// once), the buffer holds them with a 16-byte chunk XOR swizzle, and the MFMA
// operands are read back from it (lane l: row l%16, chunks l/16 and l/16 + 4).
// Only this wavefront touches its buffer, and its LDS operations run in
// order, so no barrier is needed.  Measured on MI355X for the decode layer
// (7168 x 2048 experts, graph replay): 0.77 -> 0.67 ms at 16 tokens against
// operand-layout loads that read 64 bytes of each of 16 rows per instruction.
template <int UU>
__device__ __forceinline__ void wl_load(const uint8_t* t0, const uint8_t* t1, int Kdim, int kb0, int lane,
                                        u32x4 (&raw)[UU][4]) {
#pragma unroll
    for (int u = 0; u < UU; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            raw[u][i] = __builtin_nontemporal_load((const u32x4*)((i < 2 ? t0 : t1) +
                                                                  (size_t)(8 * (i & 1) + (lane >> 3)) * Kdim +
                                                                  (size_t)(kb0 + u) * 128 + 16 * (lane & 7)));
}

template <int UU>
__device__ __forceinline__ void wl_stash(unsigned char* lds, int lane, const u32x4 (&raw)[UU][4]) {
#pragma unroll
    for (int u = 0; u < UU; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 8 * i + (lane >> 3);
            *(u32x4*)(lds + u * 4096 + r * 128 + 16 * ((lane & 7) ^ (r & 7))) = raw[u][i];
        }
}

__device__ __forceinline__ i32x8 wl_operand(const unsigned char* tile, int r, int c1) {
    const u32x4 lo = *(const u32x4*)(tile + r * 128 + 16 * (c1 ^ (r & 7)));
    const u32x4 hi = *(const u32x4*)(tile + r * 128 + 16 * ((c1 + 4) ^ (r & 7)));
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

constexpr int kWaveLds = kU * 4096;   // bytes of a wavefront's weight buffer

// K loop of one pass over up to 16*NTB rows (m0 .. m0+mv-1 of the segment)
// for this wavefront's two 16-row weight tiles (FC1: gate and up rows of 16
// features; FC2: 32 consecutive output rows); NTB token blocks of 16 rows.
// t0 / t1 point at byte 0 of the first row of each tile; sg / su are the
// tiles' weight scales per K block; lds is this wavefront's kWaveLds-byte
// buffer.  Per group of kU K blocks the weights are loaded as whole lines,
// passed through the buffer into operand layout, then multiplied with the
// token codes (loaded per K block from the quantised rows).  On return lane
// l holds, for token m0 + 16t + l%16, the fp32 sums of tile rows 4*(l/16)+i
// in acc_g[t][i] / acc_u[t][i].
template <int NTB>
__device__ __forceinline__ void fp8_accumulate(const uint8_t* __restrict__ Xq, const float* __restrict__ Xs,
                                               const uint8_t* t0, const uint8_t* t1, const float* sg,
                                               const float* su, long long seg, int m0, int mv, int Kdim, int lane,
                                               unsigned char* lds, f32x4 (&acc_g)[NTB], f32x4 (&acc_u)[NTB]) {
    constexpr int U = kU;
    const int kq = (lane >> 4) * 16, c1 = lane >> 4, r16 = lane & 15;
    const int nkb = Kdim / 128;
#pragma unroll
    for (int t = 0; t < NTB; ++t) {
        acc_g[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc_u[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // token row of this lane in block t: m0 + 16t + lane%16 (clamped)
    size_t xrow[NTB];
#pragma unroll
    for (int t = 0; t < NTB; ++t) xrow[t] = (size_t)(seg + m0 + min(16 * t + r16, mv - 1));

    // one group of UU K blocks: the weights of all of them are loaded first
    auto group = [&](int kb0, auto uc) {
        constexpr int UU = decltype(uc)::value;
        u32x4 raw[UU][4];
        wl_load<UU>(t0, t1, Kdim, kb0, lane, raw);
        wl_stash<UU>(lds, lane, raw);
        i32x8 a_g[UU], a_u[UU];
        float s_g[UU], s_u[UU];
#pragma unroll
        for (int u = 0; u < UU; ++u) {
            a_g[u] = wl_operand(lds + u * 4096, r16, c1);
            a_u[u] = wl_operand(lds + u * 4096, 16 + r16, c1);
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

}

// One pass of a work unit: the K loop, then the epilogue.
// MODE 0: SwiGLU of (gate, up) stored as fp32 [rows, Nout] at features
// f0 + 4*(lane/16) + i; MODE 1: both tiles stored as bf16 at output rows f0..
template <int MODE, int NTB>
__device__ __forceinline__ void fp8_pass(const uint8_t* __restrict__ Xq, const float* __restrict__ Xs,
                                         const uint8_t* t0, const uint8_t* t1, const float* sg, const float* su,
                                         void* __restrict__ Outv, long long seg, int m0, int mv, int Kdim, int Nout,
                                         int f0, int lane, unsigned char* lds) {
    f32x4 acc_g[NTB], acc_u[NTB];
    fp8_accumulate<NTB>(Xq, Xs, t0, t1, sg, su, seg, m0, mv, Kdim, lane, lds, acc_g, acc_u);
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
                a[i] = swiglu(g, u);
            }
            o.x = a[0]; o.y = a[1]; o.z = a[2]; o.w = a[3];
            *(float4*)((float*)Outv + orow) = o;
        } else {
            uint2 o;
            o.x = bf16x2_rne(acc_g[t][0], acc_g[t][1]);
            o.y = bf16x2_rne(acc_g[t][2], acc_g[t][3]);
            *(uint2*)((uint16_t*)Outv + orow) = o;
            o.x = bf16x2_rne(acc_u[t][0], acc_u[t][1]);
            o.y = bf16x2_rne(acc_u[t][2], acc_u[t][3]);
            *(uint2*)((uint16_t*)Outv + orow + 16) = o;
        }
    }
}

// One work unit of the fp8 expert GEMM: expert e, unit `unit` (FC1: 64
// features, FC2: 128 output rows), four wavefronts of 16 features (FC1) /
// 32 output rows (FC2) each.  Experts without rows return at once.
// MODE 0: FC1 + SwiGLU.  Xq/Xs = quantised permuted rows [R,H] / [R,H/128];
//         W = W1 [E,2F,H] e4m3, Ws = [E,2F/128,H/128]; Out = fp32 [R,F].
// MODE 1: FC2.  Xq/Xs = quantised activations [R,F] / [R,F/128]; W = W2
//         [E,H,F] e4m3, Ws = [E,H/128,F/128]; Out = bf16 expert output [R,H].
template <int MODE>
__device__ __forceinline__ void fp8_unit(const uint8_t* __restrict__ Xq, const float* __restrict__ Xs,
                                         const uint8_t* __restrict__ W, const float* __restrict__ Ws,
                                         void* __restrict__ Outv, const int64_t* __restrict__ seg_off,
                                         const int32_t* __restrict__ kept, long long R, int Kdim, int Wrows,
                                         int Nout, int e, int unit, int lane, int wave, unsigned char* lds) {
    const long long seg = seg_off[e];
    long long me_l = seg < R ? (long long)kept[e] : 0;
    if (seg + me_l > R) me_l = R - seg;
    const int me = (int)me_l;
    if (me <= 0) return;

    const int nkb = Kdim / 128;
    // first output feature (FC1) / output row (FC2) of this wavefront; its two
    // weight tiles start at rows r0 and r1 (FC1: gate and up rows of features
    // f0..f0+15; FC2: rows f0..f0+15 and f0+16..f0+31, one 128-row scale block)
    const int f0 = MODE == 0 ? unit * kFeat + wave * 16 : unit * kFeat2 + wave * 32;
    const int r0 = f0, r1 = MODE == 0 ? Nout + f0 : f0 + 16;
    const uint8_t* t0 = W + ((size_t)e * Wrows + r0) * Kdim;
    const uint8_t* t1 = W + ((size_t)e * Wrows + r1) * Kdim;
    const float* sg = Ws + ((size_t)e * (Wrows / 128) + r0 / 128) * nkb;
    const float* su = Ws + ((size_t)e * (Wrows / 128) + r1 / 128) * nkb;

    for (int m0 = 0; m0 < me; m0 += 16 * kMaxTB) {
        const int mv = min(16 * kMaxTB, me - m0);
        switch ((mv + 15) / 16) {
            case 1: fp8_pass<MODE, 1>(Xq, Xs, t0, t1, sg, su, Outv, seg, m0, mv, Kdim, Nout, f0, lane, lds); break;
            case 2: fp8_pass<MODE, 2>(Xq, Xs, t0, t1, sg, su, Outv, seg, m0, mv, Kdim, Nout, f0, lane, lds); break;
            case 3: fp8_pass<MODE, 3>(Xq, Xs, t0, t1, sg, su, Outv, seg, m0, mv, Kdim, Nout, f0, lane, lds); break;
            default: fp8_pass<MODE, 4>(Xq, Xs, t0, t1, sg, su, Outv, seg, m0, mv, Kdim, Nout, f0, lane, lds); break;
        }
    }
}

// ---- quantise-on-dispatch --------------------------------------------------
constexpr int kPQBlocks = 8;

// Quantise-on-dispatch, one wavefront's share: bf16 token row t, 128-column
// blocks b0 .. b0+kPQBlocks-1 -> e4m3 codes + 1x128 fp32 scales, written to
// every kept copy's row.  16 lanes per block, 8 values per lane, 4 blocks per
// step.  The block scale and codes follow the same rule as the expert MLP's
// row quantiser (amax / 448, nearest-even codes saturating at 448), so rows
// quantised here feed the fp8 expert GEMMs unchanged.
__device__ __forceinline__ void permute_quant_wave(const uint16_t* __restrict__ x, int H, int K, int R,
                                                   const int32_t* __restrict__ row_id, uint8_t* __restrict__ out,
                                                   float* __restrict__ outs, long long t, int b0, int lane) {
    constexpr int NIT = kPQBlocks / 4;
    const int nb = H / 128;
    const int g = lane >> 4, l16 = lane & 15;
    const uint16_t* src = x + (size_t)t * H;
    float v[NIT][8];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int b = b0 + 4 * it + g;
        if (b < nb) {
            const u32x4 w = *(const u32x4*)(src + (size_t)b * 128 + l16 * 8);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[it][2 * i] = bf16_lo(w[i]);
                v[it][2 * i + 1] = bf16_hi(w[i]);
            }
        }
    }
    u32x2 code[NIT];
    float sc[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int b = b0 + 4 * it + g;
        if (b < nb) {                       // whole 16-lane groups are active or not
            float amax = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[it][i]));
            amax = fmaxf(amax, __shfl_xor(amax, 1));
            amax = fmaxf(amax, __shfl_xor(amax, 2));
            amax = fmaxf(amax, __shfl_xor(amax, 4));
            amax = fmaxf(amax, __shfl_xor(amax, 8));
            sc[it] = e4m3_scale(amax);
            code[it][0] = e4m3_pack4(v[it][0], v[it][1], v[it][2], v[it][3], sc[it]);
            code[it][1] = e4m3_pack4(v[it][4], v[it][5], v[it][6], v[it][7], sc[it]);
        }
    }
    const int32_t* rid = row_id + (size_t)t * K;
    for (int j = 0; j < K; ++j) {
        const int r = rid[j];
        if (r < 0 || r >= R) continue;
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int b = b0 + 4 * it + g;
            if (b < nb) {
                __builtin_nontemporal_store(code[it], (u32x2*)(out + (size_t)r * H + (size_t)b * 128 + l16 * 8));
                if (l16 == 0) outs[(size_t)r * nb + b] = sc[it];
            }
        }
    }
}

// ---- combine -----------------------------------------------------------------
constexpr int kCombU = 4;   // 16-byte chunks per lane per pass
constexpr int kCombJ = 4;   // copies loaded ahead of their multiply-adds

// Combine of token t by one workgroup: wavefront w owns the row's 1 KB
// pieces w, w+4, w+8, ... (64 16-byte chunks each); copies summed in slot
// order with fp32 fma, four copies' loads issued ahead, one bf16 rounding.
__device__ __forceinline__ void combine_token_wg(const u32x4* __restrict__ Y, int K, int nch, int R,
                                                 const int32_t* __restrict__ row_id,
                                                 const float* __restrict__ copy_prob, int apply,
                                                 u32x4* __restrict__ y, int t, int w, int lane) {
    const int32_t* rid = row_id + (size_t)t * K;
    const float* cp = copy_prob + (size_t)t * K;
    for (int p0 = 0; p0 * 256 < nch; p0 += kCombU) {
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
                    const int c = ((p0 + u) * 4 + w) * 64 + lane;
                    v[jj][u] = (ok[jj] && c < nch) ? __builtin_nontemporal_load(src + c) : u32x4{0u, 0u, 0u, 0u};
                }
            }
#pragma unroll
            for (int jj = 0; jj < kCombJ; ++jj) {
                if (!ok[jj]) continue;
#pragma unroll
                for (int u = 0; u < kCombU; ++u)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        acc[u][2 * q] = fmaf(pj[jj], bf16_lo(v[jj][u][q]), acc[u][2 * q]);
                        acc[u][2 * q + 1] = fmaf(pj[jj], bf16_hi(v[jj][u][q]), acc[u][2 * q + 1]);
                    }
            }
        }
#pragma unroll
        for (int u = 0; u < kCombU; ++u) {
            const int c = ((p0 + u) * 4 + w) * 64 + lane;
            if (c < nch) {
                u32x4 o;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    o[q] = bf16x2_rne(acc[u][2 * q], acc[u][2 * q + 1]);
                y[(size_t)t * nch + c] = o;
            }
        }
    }
}

// Combine of token t by one wavefront: the four quarters of the workgroup
// form above, one after the other (same arithmetic, same result).
__device__ __forceinline__ void combine_token_wave(const u32x4* __restrict__ Y, int K, int nch, int R,
                                                   const int32_t* __restrict__ row_id,
                                                   const float* __restrict__ copy_prob, int apply,
                                                   u32x4* __restrict__ y, int t, int lane) {
    for (int w = 0; w < 4; ++w) combine_token_wg(Y, K, nch, R, row_id, copy_prob, apply, y, t, w, lane);
}

}  // namespace ops
}  // namespace moe
