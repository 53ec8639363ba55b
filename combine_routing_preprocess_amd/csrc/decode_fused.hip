// Fused fp8 decode layer: after the routing metadata, two launches run the
// rest of the MoE layer for a decode batch.
//
// Operation: TensorRT-LLM PR #16190 "Update CuTeDSL MegaMoE kernels": the
// first commit message describes one persistent kernel that runs dispatch,
// FC1, FC2 and combine for decode-sized batches with low-precision block-
// scaled expert weights; the review-fix commit trims work to the live tokens
// and launches nothing for an empty batch.  The arithmetic is the fp8 W8A8
// expert MLP of this library (1x128 activation blocks, 128x128 weight blocks,
// scale = block amax / 448) followed by the probability-weighted combine.
//
// Design.  Decode puts one or two rows on most touched experts, so the layer
// is a stream of expert weights (W1 and W2 of every touched expert, once).
//  * k_fused_prep (one workgroup per token, plus one): quantise-on-dispatch
//    of every token row into each of its kept copies (codes + 1x128 scales),
//    zero output rows of tokens without a kept copy, clear the completion
//    counters, and list the touched experts with compact row offsets.
//  * k_decode_fused (persistent, one workgroup per CU): work unit = (touched
//    expert, 128-feature slice s of the FFN).  A unit computes FC1 + SwiGLU
//    for its 128 features, quantises them as one 1x128 activation block (the
//    block is whole inside the unit, so no other unit is needed), and
//    multiplies that block with the matching 128 columns of W2: the FC2 block
//    product of slice s for every output row.  Those fp32 block products
//    (before scaling) go to a partial buffer [S, rows, H].
//  * No workgroup ever waits for another.  A unit publishes its partials
//    with a release increment of its expert's counter; the unit that brings
//    it to S (the last of the expert's slices) reduces the expert's rows over
//    s = 0..S-1 in ascending order (fp32 fma with weight scale x activation
//    scale, as the FC2 GEMM accumulates its K blocks) into the bf16 expert
//    output, then increments each row's token counter; the workgroup that
//    brings a token's counter to its number of kept copies combines that
//    token.  Every counter is read only by the workgroup whose increment
//    returned the final value, after an acquire fence.
//  * Weights stream into a 4-stage LDS ring by global_load_lds_dwordx4: one
//    instruction moves 8 whole 128-byte rows (one K block of 8 weight rows),
//    stored with a 16-byte chunk XOR swizzle so the MFMA operand reads are
//    conflict-free.  A stage is 256 weight rows x one 128-wide K block
//    (32 KB): FC1 stages hold the unit's 128 gate and 128 up rows at K block
//    kb plus the token codes of that block, FC2 stages 256 rows of W2 at the
//    slice's 128 columns.  Three stages are in flight while one is consumed.
//  * v_mfma_scale_f32_16x16x128_f8f6f4 with unit scales: one 128-wide K block
//    per instruction, weights as A (16 rows) and token or activation codes
//    as B (16 columns), the same K assignment per lane as the separate fp8
//    GEMMs, so every block product, every scale and every rounding matches
//    the separate launches bit for bit.
#include "device_ops.h"

namespace moe {
namespace {

using namespace ops;

constexpr int kSlice = 128;                  // FFN features per unit
constexpr int kStRows = 256;                 // weight rows per stage
constexpr int kTBMax = 2;                    // token blocks (16 rows) per pass
constexpr int kRing = 4;                     // stages in the LDS ring
constexpr int kWBytes = kStRows * 128;       // weight bytes of a stage (32 KB)
constexpr int kTBytes = kTBMax * 16 * 128;   // token code bytes of a stage
constexpr int kSlotBytes = kWBytes + kTBytes;
constexpr int kMaxKB = 64;                   // H / 128 limit (H <= 8192)
constexpr int kRingBytes = kRing * kSlotBytes;
constexpr int kXsStride = kMaxKB + 1;                // floats per token row (odd: no bank conflicts)
constexpr int kXsBytes = kTBMax * 16 * kXsStride * 4; // token scales of a pass
constexpr int kAqBytes = kTBMax * 16 * 128;           // activation codes of a pass
constexpr int kWsBytes = 2 * kMaxKB * 4;                // gate and up weight scales of a pass
constexpr int kLdsBytes = kRingBytes + kXsBytes + kAqBytes + kWsBytes;

struct FusedArgs {
    const uint16_t* x;          // [T,H] bf16 tokens
    const int32_t* row_id;      // [T,K]
    const float* copy_prob;     // [T,K]
    const int32_t* src_row;     // [R]
    const int64_t* seg_off;     // [E+1]
    const int32_t* kept;        // [E]
    const uint8_t* w1;          // [E,2F,H] e4m3
    const float* w1s;           // [E,2F/128,H/128]
    const uint8_t* w2;          // [E,H,F] e4m3
    const float* w2s;           // [E,H/128,F/128]
    uint8_t* xq;                // [R,H] token codes per copy row
    float* xs;                  // [R,H/128]
    float* part;                // [S,TK,H] FC2 block products, compact rows
    float* asc;                 // [TK,S] activation scales, compact rows
    int32_t* act_list;          // [E] touched experts, ascending
    int32_t* coff;              // [E] compact row offset of each touched expert
    int32_t* n_act;             // [1]
    int32_t* cnt_e;             // [E] finished slices per touched expert
    int32_t* cnt_t;             // [T] reduced copies per token
    uint16_t* eo;               // [R,H] bf16 expert output
    uint16_t* y;                // [T,H] bf16 layer output
    long long R;
    int T, H, F, K, E, TK, apply;
};

__device__ __forceinline__ long long rows_of(const FusedArgs& a, int e, long long* seg) {
    const long long so = a.seg_off[e];
    long long me = so < a.R ? (long long)a.kept[e] : 0;
    if (so + me > a.R) me = a.R - so;
    *seg = so;
    return me > 0 ? me : 0;
}

// Copies of token t that hold a row (the K slots read together).
__device__ __forceinline__ int count_copies(const int32_t* __restrict__ row_id, int K, long long R, int t) {
    int n = 0;
    for (int j0 = 0; j0 < K; j0 += 8) {
        int r[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) r[u] = j0 + u < K ? row_id[(size_t)t * K + j0 + u] : -1;
#pragma unroll
        for (int u = 0; u < 8; ++u) n += (r[u] >= 0 && r[u] < R) ? 1 : 0;
    }
    return n;
}

__global__ __launch_bounds__(256) void k_fused_prep(FusedArgs a) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if ((int)blockIdx.x == a.T) {
        // touched experts (rows kept), ascending, with compact row offsets
        for (int i = threadIdx.x; i < a.E; i += blockDim.x) a.cnt_e[i] = 0;
        if (wave == 0) {
            int run = 0, rows = 0;
            for (int c = 0; c < a.E; c += 64) {
                const int e = c + lane;
                long long seg;
                const int me = e < a.E ? (int)rows_of(a, e, &seg) : 0;
                const unsigned long long has = __ballot(me > 0);
                int incl = me;                       // inclusive scan of rows over the chunk
                for (int d = 1; d < 64; d <<= 1) {
                    const int v = __shfl_up(incl, d);
                    if (lane >= d) incl += v;
                }
                if (me > 0) {
                    const int at = run + __popcll(has & ((1ull << lane) - 1ull));
                    a.act_list[at] = e;
                    a.coff[at] = rows + incl - me;
                }
                run += __popcll(has);
                rows += __shfl(incl, 63);
            }
            if (lane == 0) a.n_act[0] = run;
        }
        return;
    }
    const int t = blockIdx.x;
    const int nb = a.H / 128, ng = (nb + kPQBlocks - 1) / kPQBlocks;
    for (int g = wave; g < ng; g += 4)
        permute_quant_wave(a.x, a.H, a.K, (int)a.R, a.row_id, a.xq, a.xs, t, g * kPQBlocks, lane);
    if (count_copies(a.row_id, a.K, a.R, t) == 0) {
        u32x4* yr = (u32x4*)(a.y + (size_t)t * a.H);
        for (int c = threadIdx.x; c < a.H / 8; c += blockDim.x) yr[c] = u32x4{0u, 0u, 0u, 0u};
    }
    if (threadIdx.x == 0) a.cnt_t[t] = 0;
}

// ---- LDS DMA ----------------------------------------------------------------
// One 16-byte-per-lane global -> LDS transfer from a per-lane address; lane
// l's bytes land at LDS byte address lds + 16*l.  Inline asm, so the compiler
// does not order later LDS reads after it: completion is awaited explicitly
// with s_waitcnt vmcnt, counting only these transfers (loads return in issue
// order, and other memory operations only lengthen a wait).  m0 is written
// only by these asm statements in this translation unit.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(gptr), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void dma16_nt(const void* gptr, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" : : "v"(gptr), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier that waits for this wavefront's LDS operations only (a
// __syncthreads fence would also wait for the ring transfers in flight).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p);
}

// 32 operand bytes of row `r` of a swizzled 128-byte-row tile: logical chunks
// c1 = lane/16 and c1 + 4 (chunk c of row r sits at position c ^ (r & 7)).
__device__ __forceinline__ i32x8 read_op(const unsigned char* tile, int r, int c1) {
    const unsigned char* row = tile + r * 128;
    const u32x4 lo = *(const u32x4*)(row + 16 * (c1 ^ (r & 7)));
    const u32x4 hi = *(const u32x4*)(row + 16 * ((c1 + 4) ^ (r & 7)));
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// One pass of a unit over up to 16*NTB rows of expert e (segment rows m0 ..
// m0+mv-1), slice s: the FC1 K blocks, the activation block, the FC2 stages.
template <int NTB>
__device__ __forceinline__ void fused_pass(const FusedArgs& a, unsigned char* smem, int e, int s, long long seg,
                                           int m0, int mv, int crow, int lane, int wave) {
    constexpr int NI = 8 + NTB;                 // ring transfers per wavefront per stage
    const int nkb = a.H / 128;
    const int nh2 = (a.H + kStRows - 1) / kStRows;
    const int nst = nkb + nh2;
    const int S = a.F / kSlice;
    const int c1 = lane >> 4, l16 = lane & 15;
    unsigned char* ring = smem;
    float* s_xs = (float*)(smem + kRingBytes);
    unsigned char* s_aq = smem + kRingBytes + kXsBytes;
    float* s_ws = (float*)(smem + kRingBytes + kXsBytes + kAqBytes);   // [2][kMaxKB]
    float* s_amax = (float*)(smem + kLdsBytes);   // [4][16*kTBMax], after the main regions

    lds_barrier();   // the previous pass is done with the ring, token scales and codes

    // token scales of the pass: row i (clamped to the last live row) x K block
    for (int q = threadIdx.x; q < 16 * NTB * nkb; q += 256) {
        const int i = q / nkb, kb = q - i * nkb;
        s_xs[i * kXsStride + kb] = a.xs[(size_t)(seg + m0 + min(i, mv - 1)) * nkb + kb];
    }

    // FC1 weight scales of the slice (gate row block s, up row block F/128 + s),
    // read here so that no load other than the ring transfers runs in the K loop
    {
        const float* sg = a.w1s + ((size_t)e * (2 * (size_t)a.F / 128) + s) * nkb;
        const float* su = a.w1s + ((size_t)e * (2 * (size_t)a.F / 128) + a.F / 128 + s) * nkb;
        for (int q = threadIdx.x; q < 2 * nkb; q += 256)
            s_ws[(q / nkb) * kMaxKB + q % nkb] = q < nkb ? sg[q] : su[q - nkb];
    }

    // per-lane ring sources.  Weight transfer jj of this wavefront covers
    // stage rows 64*wave + 8*jj + lane/8, chunk position lane%8 holds chunk
    // (lane%8) ^ (lane/8) of that row.
    const int rr = lane >> 3, wc = (lane & 7) ^ rr;
    const size_t F2 = 2 * (size_t)a.F;
    const int w1row = (wave < 2 ? s * kSlice + 64 * wave : a.F + s * kSlice + 64 * (wave - 2)) + rr;
    const uint8_t* p1 = a.w1 + ((size_t)e * F2 + w1row) * a.H + 16 * wc;
    const uint8_t* p2 = a.w2 + (size_t)e * a.H * a.F + (size_t)s * kSlice + 16 * wc;
    // token transfer q of this wavefront (lanes 0..31): token rows 16q + 4*wave + lane/8
    const uint8_t* pt[NTB];
#pragma unroll
    for (int q = 0; q < NTB; ++q) {
        const int i = 16 * q + 4 * wave + (rr & 3);
        pt[q] = a.xq + (size_t)(seg + m0 + min(i, mv - 1)) * a.H + 16 * ((lane & 7) ^ (i & 7));
    }

    auto issue = [&](int k) {
        unsigned char* slot = ring + (k % kRing) * kSlotBytes;
        const uint32_t wl = lds_addr(slot + 64 * wave * 128);
        if (k < nkb) {
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) dma16_nt(p1 + (size_t)8 * jj * a.H + (size_t)k * 128, wl + jj * 1024);
        } else {
            const int h0 = (k - nkb) * kStRows + 64 * wave + rr;
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                // rows past H (a final half stage) repeat row H-1; their products are not stored
                const int h = min(h0 + 8 * jj, a.H - 1);
                dma16_nt(p2 + (size_t)h * a.F, wl + jj * 1024);
            }
        }
        // token codes of K block k (FC2 stages reload block 0: equal transfer counts)
        const int kt = k < nkb ? k : 0;
        const uint32_t tl = lds_addr(slot + kWBytes + 4 * wave * 128);
#pragma unroll
        for (int q = 0; q < NTB; ++q)
            if (lane < 32) dma16(pt[q] + (size_t)kt * 128, tl + q * 16 * 128);
    };

    f32x4 acc[4][NTB];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int t = 0; t < NTB; ++t) acc[j][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    i32x8 bq[NTB];

    for (int k = 0; k < kRing - 1 && k < nst; ++k) issue(k);
    for (int k = 0; k < nst; ++k) {
        const int ahead = min(kRing - 2, nst - 1 - k);
        if (ahead >= 2) wait_vm<2 * NI>();
        else if (ahead == 1) wait_vm<NI>();
        else wait_vm<0>();
        lds_barrier();
        if (k + kRing - 1 < nst) issue(k + kRing - 1);
        const unsigned char* slot = ring + (k % kRing) * kSlotBytes;
        if (k < nkb) {
            // FC1: gate tiles at stage rows 32w, 32w+16; up tiles at 128+32w, 128+32w+16
            const float wg = s_ws[k], wu = s_ws[kMaxKB + k];
            i32x8 xb[NTB];
            float sx[NTB];
#pragma unroll
            for (int t = 0; t < NTB; ++t) {
                xb[t] = read_op(slot + kWBytes, 16 * t + l16, c1);
                sx[t] = s_xs[(16 * t + l16) * kXsStride + k];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const i32x8 w = read_op(slot, (j < 2 ? 32 * wave + 16 * j : 128 + 32 * wave + 16 * (j - 2)) + l16, c1);
                const float ws = j < 2 ? wg : wu;
#pragma unroll
                for (int t = 0; t < NTB; ++t) {
                    const f32x4 p = mfma_fp8(w, xb[t]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[j][t][i] = fmaf(p[i], ws * sx[t], acc[j][t][i]);
                }
            }
            if (k == nkb - 1) {
                // SwiGLU of the slice; lane: token 16t + l16, features 32w + 16jj + 4*c1 + i
                float act[2][NTB][4];
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                    for (int t = 0; t < NTB; ++t)
#pragma unroll
                        for (int i = 0; i < 4; ++i) act[jj][t][i] = swiglu(acc[jj][t][i], acc[jj + 2][t][i]);
                // one 1x128 block per token: amax over lanes, then over wavefronts
#pragma unroll
                for (int t = 0; t < NTB; ++t) {
                    float m = 0.f;
#pragma unroll
                    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                        for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(act[jj][t][i]));
                    m = fmaxf(m, __shfl_xor(m, 16));
                    m = fmaxf(m, __shfl_xor(m, 32));
                    if (c1 == 0) s_amax[wave * 16 * kTBMax + 16 * t + l16] = m;
                }
                lds_barrier();
#pragma unroll
                for (int t = 0; t < NTB; ++t) {
                    const int tok = 16 * t + l16;
                    float m = s_amax[tok];
#pragma unroll
                    for (int w = 1; w < 4; ++w) m = fmaxf(m, s_amax[w * 16 * kTBMax + tok]);
                    const float sc = e4m3_scale(m);
#pragma unroll
                    for (int jj = 0; jj < 2; ++jj) {
                        const int chunk = 2 * wave + jj;
                        *(uint32_t*)(s_aq + tok * 128 + 16 * (chunk ^ (tok & 7)) + 4 * c1) =
                            e4m3_pack4(act[jj][t][0], act[jj][t][1], act[jj][t][2], act[jj][t][3], sc);
                    }
                    if (wave == 0 && c1 == 0 && tok < mv) a.asc[(size_t)(crow + tok) * S + s] = sc;
                }
                lds_barrier();
#pragma unroll
                for (int t = 0; t < NTB; ++t) bq[t] = read_op(s_aq, 16 * t + l16, c1);
            }
        } else {
            // FC2: stage rows 64w + 16jt, raw block products to the partial buffer
            const int h0 = (k - nkb) * kStRows + 64 * wave;
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) {
                const int hb = h0 + 16 * jt;
                const i32x8 w = read_op(slot, 64 * wave + 16 * jt + l16, c1);
#pragma unroll
                for (int t = 0; t < NTB; ++t) {
                    const f32x4 p = mfma_fp8(w, bq[t]);
                    const int tok = 16 * t + l16;
                    if (hb < a.H && tok < mv)
                        *(f32x4*)(a.part + ((size_t)s * a.TK + crow + tok) * a.H + hb + 4 * c1) = p;
                }
            }
        }
    }
}

// Rows of a touched expert: bf16 expert output = sum over slices s (in
// ascending order) of fma(block product, weight scale x activation scale),
// eight slices' loads issued together.
__device__ void reduce_expert(const FusedArgs& a, const float* __restrict__ w2s, int e, long long seg, int me,
                              int crow0) {
    const int S = a.F / kSlice, nbh = a.H / 128;
    const int n4 = a.H / 4;
    for (long long q = threadIdx.x; q < (long long)me * n4; q += blockDim.x) {
        const int i = (int)(q / n4), h = (int)(q - (long long)i * n4) * 4;
        const float* ws = w2s + ((size_t)e * nbh + h / 128) * S;
        const float* as = a.asc + (size_t)(crow0 + i) * S;
        const float* pp = a.part + (size_t)(crow0 + i) * a.H + h;
        const size_t sstride = (size_t)a.TK * a.H;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int s0 = 0; s0 < S; s0 += 8) {
            f32x4 p[8];
            float sc[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {   // past S: an in-bounds slice, not accumulated
                const int su = min(s0 + u, S - 1);
                p[u] = *(const f32x4*)(pp + (size_t)su * sstride);
                sc[u] = ws[su] * as[su];
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (s0 + u < S) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[r] = fmaf(p[u][r], sc[u], acc[r]);
                }
            }
        }
        u32x2 o;
        o[0] = f32_to_bf16(acc[0]) | (f32_to_bf16(acc[1]) << 16);
        o[1] = f32_to_bf16(acc[2]) | (f32_to_bf16(acc[3]) << 16);
        *(u32x2*)(a.eo + (size_t)(seg + i) * a.H + h) = o;
    }
}

// The routing arrays and W2 scales come in again as restrict parameters: the
// kernel never writes them, so uniform reads of them can use scalar loads.
__global__ __launch_bounds__(256, 1) void k_decode_fused(FusedArgs a, const int32_t* __restrict__ row_id,
                                                         const float* __restrict__ copy_prob,
                                                         const int32_t* __restrict__ src_row,
                                                         const int32_t* __restrict__ act_list,
                                                         const int32_t* __restrict__ coff,
                                                         const float* __restrict__ w2s) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[kLdsBytes + 4 * 16 * kTBMax * 4];
    __shared__ int s_last, s_ntok;
    __shared__ int s_tok[64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int S = a.F / kSlice;
    const int n_units = a.n_act[0] * S;
    for (int u = blockIdx.x; u < n_units; u += gridDim.x) {
        const int ai = u / S, s = u - ai * S;
        const int e = act_list[ai];
        long long seg;
        const int me = (int)rows_of(a, e, &seg);
        const int crow0 = coff[ai];
        for (int m0 = 0; m0 < me; m0 += 16 * kTBMax) {
            const int mv = min(16 * kTBMax, me - m0);
            if (mv <= 16) fused_pass<1>(a, smem, e, s, seg, m0, mv, crow0 + m0, lane, wave);
            else fused_pass<2>(a, smem, e, s, seg, m0, mv, crow0 + m0, lane, wave);
        }
        // publish this slice; the last of the expert's S slices reduces it
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __syncthreads();
        if (threadIdx.x == 0)
            s_last = __hip_atomic_fetch_add(a.cnt_e + ai, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT) == S - 1;
        __syncthreads();
        if (!s_last) continue;
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        reduce_expert(a, w2s, e, seg, me, crow0);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        // publish the expert rows; a token whose copies are all reduced is combined here
        for (int i0 = 0; i0 < me; i0 += 64) {
            __syncthreads();
            if (threadIdx.x == 0) s_ntok = 0;
            __syncthreads();
            if (wave == 0 && i0 + lane < me) {
                const int t = src_row[seg + i0 + lane];
                const int nv = count_copies(row_id, a.K, a.R, t);
                if (__hip_atomic_fetch_add(a.cnt_t + t, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT) == nv - 1)
                    s_tok[atomicAdd(&s_ntok, 1)] = t;
            }
            __syncthreads();
            const int ntok = s_ntok;
            if (ntok > 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            for (int q = 0; q < ntok; ++q)
                combine_token_wg((const u32x4*)a.eo, a.K, a.H / 8, (int)a.R, row_id, copy_prob, a.apply,
                                 (u32x4*)a.y, s_tok[q], wave, lane);
        }
        __syncthreads();
    }
}

size_t up256(size_t n) { return (n + 255) & ~(size_t)255; }

struct FusedLayout {
    size_t xq, xs, part, asc, act_list, coff, n_act, cnt_e, cnt_t, total;
};

FusedLayout fused_layout(long long R, int T, int K, int H, int F, int E) {
    FusedLayout L;
    const size_t r = (size_t)R, tk = (size_t)T * K, S = (size_t)F / kSlice;
    size_t o = 0;
    L.xq = o;       o += up256(r * H);
    L.xs = o;       o += up256(r * (H / 128) * 4);
    L.part = o;     o += up256(S * tk * H * 4);
    L.asc = o;      o += up256(tk * S * 4);
    L.act_list = o; o += up256((size_t)E * 4);
    L.coff = o;     o += up256((size_t)E * 4);
    L.n_act = o;    o += 256;
    L.cnt_e = o;    o += up256((size_t)E * 4);
    L.cnt_t = o;    o += up256((size_t)T * 4);
    L.total = o;
    return L;
}

}  // namespace

size_t decode_fused_scratch_bytes(long long R, int T, int K, int H, int F, int E) {
    return fused_layout(R, T, K, H, F, E).total;
}

bool decode_fused_shape_ok(int H, int F) { return H % 128 == 0 && H / 128 <= kMaxKB && F % kSlice == 0; }

hipError_t launch_decode_fused(const moe_handle* h, int F, const void* x, const void* w1, const float* w1s,
                               const void* w2, const float* w2s, void* scratch, void* expert_out, int apply_probs,
                               void* y, int num_cu, hipStream_t s) {
    const moe_desc& d = h->desc;
    if (d.T == 0) return hipSuccess;   // an empty batch launches nothing
    const long long R = d.out_rows;
    const FusedLayout L = fused_layout(R, d.T, d.K, d.H, F, d.E);
    char* base = (char*)scratch;
    FusedArgs a;
    a.x = (const uint16_t*)x;
    a.row_id = h->row_id;
    a.copy_prob = h->copy_prob;
    a.src_row = h->src_row;
    a.seg_off = h->seg_off;
    a.kept = h->kept;
    a.w1 = (const uint8_t*)w1;
    a.w1s = w1s;
    a.w2 = (const uint8_t*)w2;
    a.w2s = w2s;
    a.xq = (uint8_t*)(base + L.xq);
    a.xs = (float*)(base + L.xs);
    a.part = (float*)(base + L.part);
    a.asc = (float*)(base + L.asc);
    a.act_list = (int32_t*)(base + L.act_list);
    a.coff = (int32_t*)(base + L.coff);
    a.n_act = (int32_t*)(base + L.n_act);
    a.cnt_e = (int32_t*)(base + L.cnt_e);
    a.cnt_t = (int32_t*)(base + L.cnt_t);
    a.eo = (uint16_t*)expert_out;
    a.y = (uint16_t*)y;
    a.R = R;
    a.T = d.T;
    a.H = d.H;
    a.F = F;
    a.K = d.K;
    a.E = d.E;
    a.TK = d.T * d.K;
    a.apply = apply_probs;
    hipLaunchKernelGGL(k_fused_prep, dim3(d.T + 1), dim3(256), 0, s, a);
    hipLaunchKernelGGL(k_decode_fused, dim3(num_cu), dim3(256), 0, s, a, a.row_id, a.copy_prob, a.src_row,
                       (const int32_t*)a.act_list, (const int32_t*)a.coff, a.w2s);
    return hipGetLastError();
}

}  // namespace moe
