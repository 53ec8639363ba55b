// Grouped expert MLP, bf16 weights (K3 = FC1 + SwiGLU, K4 = FC2).
//
// Operation: Megatron-LM PR #6800 "Reuse caller-owned HybridEP dispatch and
// expert output buffers" (sections "Summary", "Configuration": a grouped
// FC1 -> activation -> FC2 MLP whose FC2 lands in a caller-provided buffer)
// and TensorRT-LLM PR #16190 "Update CuTeDSL MegaMoE kernels" (streaming-load
// commit: FC1's weight is one concatenated gate/up matrix).  W1[e] is
// [2F, H] (rows [0,F) gate, [F,2F) up), W2[e] is [H, F]; for each kept row x
// of expert e's segment: a = silu(W1g x) * (W1u x) stored bf16, then
// y = W2 a stored bf16.
//
// Design (CDNA4): v_mfma_f32_32x32x16_bf16 on 64-wide wavefronts.  A tile is
// 128 token rows x 256 weight rows, reduced over K in 64-wide slices staged
// through XOR-swizzled LDS (double buffered, register prefetch of the next
// slice while the MFMAs run).  Four wavefronts each own a 64 x 128 block:
// 2 x 4 MFMA accumulators of 32 x 32.  For FC1 the 256 weight rows are 128
// gate rows and the 128 matching up rows, and each wavefront holds a gate and
// an up accumulator for the same output columns, so SwiGLU is applied in
// registers before the single bf16 store.
//
// Scheduling: group sizes live on the device (segment offsets and kept
// counts from the routing kernels), so each workgroup derives the tile list
// itself: a prefix over experts of ceil(rows/128) in LDS, then a persistent
// loop over (expert, N tile, M tile) with the M tiles of one weight tile
// adjacent.  Workgroup ids are renumbered so a contiguous tile range runs on
// one XCD (hardware deals workgroups round-robin over the 8 XCDs), keeping a
// weight tile's re-reads by its M tiles inside one L2.
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128;                        // token rows per tile
constexpr int BNW = 256;                       // weight rows per tile
constexpr int BK = 64;                         // K slice per stage
constexpr int kAChunks = BM * BK / 8;          // 16-byte chunks in an A slice (1024)
constexpr int kBChunks = BNW * BK / 8;         // 2048
constexpr int kStageChunks = kAChunks + kBChunks;

// Chunk position of (row, 16-byte column chunk) inside a 64-column slice:
// the chunk index is XORed with the row's low bits so the 32 rows read by
// one MFMA operand fetch spread over all banks.
__device__ __forceinline__ int swz(int row, int ch) { return row * 8 + (ch ^ (row & 7)); }

template <int MODE>  // 0: FC1 + SwiGLU (out = act [R,F]); 1: FC2 (out = expert_out [R,H])
__global__ __launch_bounds__(256, 1) void k_gemm_bf16(const uint16_t* __restrict__ X,
                                                      const uint16_t* __restrict__ W,
                                                      uint16_t* __restrict__ Out,
                                                      const int64_t* __restrict__ seg_off,
                                                      const int32_t* __restrict__ kept, int E,
                                                      long long R, int Kdim, int Wrows, int Nout,
                                                      int n_ntiles) {
    __shared__ u32x4 smem[2 * kStageChunks];   // 96 KiB
    __shared__ int s_mt[kMaxE + 1];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // ---- device-side tile list: prefix over experts of M-tile counts ------
    for (int i = tid; i <= kMaxE; i += 256) s_mt[i] = 0;
    __syncthreads();
    for (int e = tid; e < E; e += 256) {
        const long long so = seg_off[e];
        long long m = so < R ? (long long)kept[e] : 0;
        if (so + m > R) m = R - so;
        s_mt[e + 1] = (int)((m + BM - 1) / BM);
    }
    __syncthreads();
    for (int off = 1; off <= kMaxE; off <<= 1) {   // inclusive scan of s_mt[1..kMaxE]
        int v[5];
#pragma unroll
        for (int q = 0; q < 5; ++q) {
            const int i = 1 + tid + q * 256;
            v[q] = (i <= kMaxE && i - off >= 1) ? s_mt[i - off] : 0;
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 5; ++q) {
            const int i = 1 + tid + q * 256;
            if (i <= kMaxE) s_mt[i] += v[q];
        }
        __syncthreads();
    }
    const int total = s_mt[E] * n_ntiles;

    const int G = gridDim.x, b = blockIdx.x;
    const int vid = (G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;

    for (int tile = vid; tile < total; tile += G) {
        // ---- decode (expert, N tile, M tile) ------------------------------
        int lo = 0, hi = E - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_mt[mid] * n_ntiles <= tile) lo = mid; else hi = mid - 1;
        }
        const int e = lo;
        const int ce = s_mt[e + 1] - s_mt[e];
        const int local = tile - s_mt[e] * n_ntiles;
        const int nt = local / ce, mt = local - nt * ce;
        const long long seg = seg_off[e];
        long long me_l = kept[e];
        if (seg + me_l > R) me_l = R - seg;
        const int me = (int)me_l;
        const int m0 = mt * BM;
        const int mv = min(BM, me - m0);
        const uint16_t* Xb = X + (size_t)(seg + m0) * Kdim;
        const uint16_t* Wb = W + (size_t)e * Wrows * Kdim;
        const int n0 = (MODE == 0) ? nt * 128 : nt * 256;

        // ---- per-thread global / LDS addresses of its 12 chunks -----------
        const uint16_t* ap[4];
        bool aok[4];
        int al[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int i = tid + q * 256, row = i >> 3, ch = i & 7;
            aok[q] = row < mv;
            ap[q] = Xb + (size_t)(aok[q] ? row : 0) * Kdim + ch * 8;
            al[q] = swz(row, ch);
        }
        const uint16_t* bp[8];
        int bl[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int i = tid + q * 256, row = i >> 3, ch = i & 7;
            int wr;
            if (MODE == 0) wr = row < 128 ? n0 + row : Nout + n0 + (row - 128);
            else wr = n0 + row;
            bp[q] = Wb + (size_t)wr * Kdim + ch * 8;
            bl[q] = kAChunks + swz(row, ch);
        }

        f32x16 acc[2][4];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[mi][ni][i] = 0.f;

        // rows of this wavefront's operand fetches (LDS)
        int arow[2], brow[4];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) arow[mi] = wm * 64 + mi * 32 + (lane & 31);
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
            if (MODE == 0) brow[ni] = (ni < 2 ? 0 : 128) + wn * 64 + (ni & 1) * 32 + (lane & 31);
            else brow[ni] = wn * 128 + ni * 32 + (lane & 31);
        }

        u32x4 ra[4], rb[8];
        const u32x4 zero = {0u, 0u, 0u, 0u};
        const int nk = Kdim / BK;

#define GLOAD(kt)                                                                        \
    do {                                                                                 \
        const int k0_ = (kt) * BK;                                                       \
        _Pragma("unroll") for (int q = 0; q < 4; ++q) ra[q] =                            \
            aok[q] ? *(const u32x4*)(ap[q] + k0_) : zero;                                \
        _Pragma("unroll") for (int q = 0; q < 8; ++q) rb[q] = *(const u32x4*)(bp[q] + k0_); \
    } while (0)
#define SSTORE(st)                                                                       \
    do {                                                                                 \
        u32x4* base_ = smem + (st) * kStageChunks;                                       \
        _Pragma("unroll") for (int q = 0; q < 4; ++q) base_[al[q]] = ra[q];              \
        _Pragma("unroll") for (int q = 0; q < 8; ++q) base_[bl[q]] = rb[q];              \
    } while (0)

        GLOAD(0);
        SSTORE(0);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const int st = kt & 1;
            if (kt + 1 < nk) GLOAD(kt + 1);
            const u32x4* base = smem + st * kStageChunks;
#pragma unroll
            for (int s = 0; s < BK / 16; ++s) {
                const int ch = s * 2 + (lane >> 5);
                bf16x8 a[2], bb[4];
#pragma unroll
                for (int mi = 0; mi < 2; ++mi) a[mi] = __builtin_bit_cast(bf16x8, base[swz(arow[mi], ch)]);
#pragma unroll
                for (int ni = 0; ni < 4; ++ni)
                    bb[ni] = __builtin_bit_cast(bf16x8, base[kAChunks + swz(brow[ni], ch)]);
#pragma unroll
                for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni)
                        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], bb[ni], acc[mi][ni], 0, 0, 0);
            }
            if (kt + 1 < nk) SSTORE(st ^ 1);
            __syncthreads();
        }
#undef GLOAD
#undef SSTORE

        // ---- epilogue ------------------------------------------------------
        // 32x32 accumulator layout: lane l holds column l%32 and rows
        // 8*(i/4) + 4*(l/32) + i%4 for its 16 values i.
        uint16_t* Ob = Out + (size_t)(seg + m0) * Nout;
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = wm * 64 + mi * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
                if (r >= mv) continue;
                uint16_t* orow = Ob + (size_t)r * Nout;
                if (MODE == 0) {
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        const float g = acc[mi][c][i], u = acc[mi][2 + c][i];
                        const float av = g / (1.f + __expf(-g)) * u;
                        orow[n0 + wn * 64 + c * 32 + (lane & 31)] = (uint16_t)f32_to_bf16(av);
                    }
                } else {
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni)
                        orow[n0 + wn * 128 + ni * 32 + (lane & 31)] = (uint16_t)f32_to_bf16(acc[mi][ni][i]);
                }
            }
        }
    }
}

int grid_for(long long upper, int num_cu) {
    long long g = upper < num_cu ? upper : num_cu;
    if (g >= 8) g -= g % 8;
    return (int)(g < 1 ? 1 : g);
}

}  // namespace

hipError_t launch_mlp_bf16(const moe_handle* h, int F, const void* perm, const void* w1,
                           const void* w2, void* act, void* expert_out, int num_cu, hipStream_t s) {
    const moe_desc& d = h->desc;
    const long long R = d.out_rows;
    if (R == 0) return hipSuccess;
    const long long mt_upper = (R + BM - 1) / BM + d.E;
    const int nt1 = F / 128, nt2 = d.H / 256;
    hipLaunchKernelGGL(k_gemm_bf16<0>, dim3(grid_for(mt_upper * nt1, num_cu)), dim3(256), 0, s,
                       (const uint16_t*)perm, (const uint16_t*)w1, (uint16_t*)act, h->seg_off, h->kept, d.E, R,
                       d.H, 2 * F, F, nt1);
    hipLaunchKernelGGL(k_gemm_bf16<1>, dim3(grid_for(mt_upper * nt2, num_cu)), dim3(256), 0, s,
                       (const uint16_t*)act, (const uint16_t*)w2, (uint16_t*)expert_out, h->seg_off, h->kept, d.E,
                       R, F, d.H, d.H, nt2);
    return hipGetLastError();
}

}  // namespace moe
