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
//  * k_decode_fused (persistent, two workgroups per CU): work unit = (touched
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
//  * Four wavefronts per workgroup, two workgroups per CU (while one
//    synchronises or reduces, the other keeps weights streaming).  FC1:
//    wavefront w streams the gate and up rows of features 32w..32w+15, then
//    32w+16..32w+31 of the slice over all K blocks, exactly as the separate
//    FC1 GEMM does (whole 128-byte lines, non-temporal, through its own LDS
//    buffer into operand layout).  FC2: wavefront w streams a quarter of the
//    W2 rows at the slice's 128 columns, eight 16-row tiles (one 128-byte
//    line per row) per load group.  No barrier runs while weights stream;
//    the activation block is exchanged through LDS between the two phases.
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
constexpr int kWaves = 4;                    // wavefronts per workgroup
constexpr int kTBMax = 2;                    // token blocks (16 rows) per pass
constexpr int kMaxKB = 64;                   // H / 128 and F / 128 limit
constexpr int kWaveBytes = kWaves * kWaveLds;            // weight buffers of all wavefronts
constexpr int kAmaxBytes = kWaves * 16 * kTBMax * 4;     // per-wavefront block maxima
constexpr int kAqBytes = kTBMax * 16 * 128;              // activation codes of a pass
constexpr int kLdsBytes = kWaveBytes + kAmaxBytes + kAqBytes;
static_assert(2 * kMaxKB * kMaxKB * 4 <= kWaveBytes, "reduce scales fit the weight buffers");

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

// Workgroup barrier that waits for this wavefront's LDS operations only
// (weight loads of other wavefronts may still be in flight).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// All vector memory operations of this wavefront (its stores) have completed.
__device__ __forceinline__ void wait_stores() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// One pass of a unit over up to 16*NTB rows of expert e (segment rows m0 ..
// m0+mv-1), slice s: FC1 + SwiGLU of the slice, its activation block, and the
// FC2 block products of the slice for every output row.
template <int NTB>
__device__ __forceinline__ void fused_pass(const FusedArgs& a, const float* __restrict__ w1s, unsigned char* smem,
                                           int e, int s, long long seg, int m0, int mv, int crow, int lane,
                                           int wave) {
    const int nkb = a.H / 128;
    const int S = a.F / kSlice;
    const int c1 = lane >> 4, r16 = lane & 15;
    unsigned char* wl = smem + wave * kWaveLds;
    float* s_amax = (float*)(smem + kWaveBytes);
    unsigned char* s_aq = smem + kWaveBytes + kAmaxBytes;

    lds_barrier();   // the previous pass is done with the activation exchange

    // ---- FC1: features 32w + 16hf .. +15 of the slice (hf = 0, 1), gate and up tiles
    const size_t F2 = 2 * (size_t)a.F;
    const float* sg = w1s + ((size_t)e * (F2 / 128) + s) * nkb;
    const float* su = w1s + ((size_t)e * (F2 / 128) + a.F / 128 + s) * nkb;
    float act[2][NTB][4];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        const int f0 = s * kSlice + 32 * wave + 16 * hf;
        const uint8_t* t0 = a.w1 + ((size_t)e * F2 + f0) * a.H;
        const uint8_t* t1 = a.w1 + ((size_t)e * F2 + a.F + f0) * a.H;
        f32x4 acc_g[NTB], acc_u[NTB];
        fp8_accumulate<NTB>(a.xq, a.xs, t0, t1, sg, su, seg, m0, mv, a.H, lane, wl, acc_g, acc_u);
#pragma unroll
        for (int t = 0; t < NTB; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) act[hf][t][i] = swiglu(acc_g[t][i], acc_u[t][i]);
    }

    // ---- the slice's 1x128 activation block per token: lane holds token
    // 16t + l%16, features 32w + 16hf + 4*(l/16) + i of the slice
#pragma unroll
    for (int t = 0; t < NTB; ++t) {
        float m = 0.f;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(act[hf][t][i]));
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        if (c1 == 0) s_amax[wave * 16 * kTBMax + 16 * t + r16] = m;
    }
    lds_barrier();
#pragma unroll
    for (int t = 0; t < NTB; ++t) {
        const int tok = 16 * t + r16;
        float m = s_amax[tok];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) m = fmaxf(m, s_amax[w * 16 * kTBMax + tok]);
        const float sc = e4m3_scale(m);
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
            *(uint32_t*)(s_aq + tok * 128 + 16 * ((2 * wave + hf) ^ (tok & 7)) + 4 * c1) =
                e4m3_pack4(act[hf][t][0], act[hf][t][1], act[hf][t][2], act[hf][t][3], sc);
        if (wave == 0 && c1 == 0 && tok < mv) a.asc[(size_t)(crow + tok) * S + s] = sc;
    }
    lds_barrier();
    i32x8 bq[NTB];
#pragma unroll
    for (int t = 0; t < NTB; ++t) bq[t] = wl_operand(s_aq, 16 * t + r16, c1);

    // ---- FC2: this wavefront's W2 tiles at the slice's 128 columns, eight
    // 16-row tiles per load group (tile j of a group at buffer offset 2048j)
    const int ntiles = a.H / 16;
    const int per_w = (ntiles + kWaves - 1) / kWaves;
    const int tb0 = wave * per_w, tb1 = min(ntiles, tb0 + per_w);
    const uint8_t* w2e = a.w2 + (size_t)e * a.H * a.F + (size_t)s * kSlice + 16 * (lane & 7);
    for (int g0 = tb0; g0 < tb1; g0 += 8) {
        u32x4 raw[8][2];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int tj = min(g0 + j, tb1 - 1);      // past the range: a repeat, not stored
#pragma unroll
            for (int h = 0; h < 2; ++h)
                raw[j][h] = __builtin_nontemporal_load(
                    (const u32x4*)(w2e + (size_t)(16 * tj + 8 * h + (lane >> 3)) * a.F));
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int r = 8 * h + (lane >> 3);
                *(u32x4*)(wl + j * 2048 + r * 128 + 16 * ((lane & 7) ^ (r & 7))) = raw[j][h];
            }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const i32x8 w = wl_operand(wl + j * 2048, r16, c1);
            const bool live = g0 + j < tb1;
#pragma unroll
            for (int t = 0; t < NTB; ++t) {
                const f32x4 p = mfma_fp8(w, bq[t]);
                const int tok = 16 * t + r16;
                if (live && tok < mv)
                    *(f32x4*)(a.part + ((size_t)s * a.TK + crow + tok) * a.H + 16 * (g0 + j) + 4 * c1) = p;
            }
        }
    }
}

// Rows of a touched expert: bf16 expert output = sum over slices s (in
// ascending order) of fma(block product, weight scale x activation scale).
// The scales are staged in LDS; each item's partials (up to 16 slices) are
// loaded together.
__device__ void reduce_expert(const FusedArgs& a, const float* __restrict__ w2s, unsigned char* smem, int e,
                              long long seg, int me, int crow0) {
    const int S = a.F / kSlice, nbh = a.H / 128;
    const int n4 = a.H / 4;
    float* s_ws = (float*)smem;                          // [nbh][S]
    float* s_as = (float*)(smem + kMaxKB * kMaxKB * 4);  // [64][S]
    const size_t sstride = (size_t)a.TK * a.H;
    for (int q = threadIdx.x; q < nbh * S; q += blockDim.x) s_ws[q] = w2s[(size_t)e * nbh * S + q];
    for (int i0 = 0; i0 < me; i0 += 64) {
        const int nrow = min(64, me - i0);
        __syncthreads();
        for (int q = threadIdx.x; q < nrow * S; q += blockDim.x) s_as[q] = a.asc[(size_t)(crow0 + i0) * S + q];
        __syncthreads();
        for (int q = threadIdx.x; q < nrow * n4; q += blockDim.x) {
            const int i = q / n4, h = (q - i * n4) * 4;
            const float* pp = a.part + (size_t)(crow0 + i0 + i) * a.H + h;
            const float* ws = s_ws + (h / 128) * S;
            const float* as = s_as + i * S;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int s0 = 0; s0 < S; s0 += 16) {
                f32x4 p[16];
#pragma unroll
                for (int u = 0; u < 16; ++u)   // past S: an in-bounds slice, not accumulated
                    p[u] = *(const f32x4*)(pp + (size_t)min(s0 + u, S - 1) * sstride);
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    if (s0 + u < S) {
                        const float sc = ws[s0 + u] * as[s0 + u];
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[r] = fmaf(p[u][r], sc, acc[r]);
                    }
                }
            }
            u32x2 o;
            o[0] = bf16x2_rne(acc[0], acc[1]);
            o[1] = bf16x2_rne(acc[2], acc[3]);
            *(u32x2*)(a.eo + (size_t)(seg + i0 + i) * a.H + h) = o;
        }
    }
}

// The routing arrays and weight scales come in again as restrict parameters:
// the kernel never writes them, so uniform reads of them can use scalar loads.
__global__ __launch_bounds__(kWaves * 64, 2) void k_decode_fused(FusedArgs a, const int32_t* __restrict__ row_id,
                                                                 const float* __restrict__ copy_prob,
                                                                 const int32_t* __restrict__ src_row,
                                                                 const int32_t* __restrict__ act_list,
                                                                 const int32_t* __restrict__ coff,
                                                                 const float* __restrict__ w1s,
                                                                 const float* __restrict__ w2s) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[kLdsBytes];
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
            if (mv <= 16) fused_pass<1>(a, w1s, smem, e, s, seg, m0, mv, crow0 + m0, lane, wave);
            else fused_pass<2>(a, w1s, smem, e, s, seg, m0, mv, crow0 + m0, lane, wave);
        }
        // publish this slice: every wavefront's stores are complete at the
        // barrier, then one release increment (it writes back this XCD's L2);
        // the last of the expert's S slices acquires and reduces the expert
        wait_stores();
        __syncthreads();
        if (threadIdx.x == 0) {
            const int last =
                __hip_atomic_fetch_add(a.cnt_e + ai, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT) == S - 1;
            if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            s_last = last;
        }
        __syncthreads();
        if (!s_last) continue;
        reduce_expert(a, w2s, smem, e, seg, me, crow0);
        // publish the expert rows; a token whose copies are all reduced is combined here
        for (int i0 = 0; i0 < me; i0 += 64) {
            wait_stores();
            __syncthreads();
            if (threadIdx.x == 0) s_ntok = 0;
            __syncthreads();
            if (wave == 0) {
                bool done = false;
                int t = 0;
                if (i0 + lane < me) {
                    t = src_row[seg + i0 + lane];
                    const int nv = count_copies(row_id, a.K, a.R, t);
                    done = __hip_atomic_fetch_add(a.cnt_t + t, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT) ==
                           nv - 1;
                }
                if (__ballot(done) != 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                if (done) s_tok[atomicAdd(&s_ntok, 1)] = t;
            }
            __syncthreads();
            const int ntok = s_ntok;
            for (int q = wave; q < ntok; q += kWaves)
                combine_token_wave((const u32x4*)a.eo, a.K, a.H / 8, (int)a.R, row_id, copy_prob, a.apply,
                                   (u32x4*)a.y, s_tok[q], lane);
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

bool decode_fused_shape_ok(int H, int F) {
    return H % 128 == 0 && H / 128 <= kMaxKB && F % kSlice == 0 && F / kSlice <= kMaxKB;
}

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
    hipLaunchKernelGGL(k_decode_fused, dim3(2 * num_cu), dim3(kWaves * 64), 0, s, a, a.row_id, a.copy_prob, a.src_row,
                       (const int32_t*)a.act_list, (const int32_t*)a.coff, a.w1s, a.w2s);
    return hipGetLastError();
}

}  // namespace moe
