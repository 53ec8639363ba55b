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
// Design (CDNA4, 256 CUs in 8 XCDs, 4 MB L2 per XCD):
//  * Work unit = (expert, 128 weight rows).  For FC1 the 128 rows are 64 gate
//    rows and the 64 matching up rows; for FC2 they are 128 output columns.
//    A unit takes ALL of the expert's rows (in chunks of up to 320 tokens), so
//    a weight row is streamed from HBM once per layer in the common case.
//  * Experts are dealt to XCDs (expert e -> XCD e mod 8; hardware deals
//    workgroups round-robin over XCDs, so workgroup b runs on XCD b mod 8).
//    The 32 workgroups of an XCD walk that XCD's units in order, so at any
//    time they share one expert: its token rows are read from L2, not HBM.
//  * MFMA v_mfma_f32_32x32x16_bf16 with the weights as the A operand (rows of
//    the 32x32 result = weight rows) and tokens as B (columns), so each lane
//    ends up with 4 consecutive output features of one token: the epilogue
//    stores 8 bytes per lane, and the FC1 gate/up values of a feature sit in
//    the same lane for the SwiGLU.
//  * Global -> LDS through global_load_lds_dwordx4 (no VGPR staging): token
//    slices in a 2-deep ring (they come from L2), weight slices in a 4-deep
//    ring (from HBM: ~48 KB in flight per CU).  The 16-byte chunk swizzle is
//    applied on the global side so MFMA operand reads from LDS are bank
//    conflict free (64 banks).  DMA instructions are interleaved one per MFMA.
//  * 4 wavefronts; wave w owns token blocks w, w+4, w+8 (32 rows each) and
//    all 4 weight blocks of the unit: per 16-wide K step 4 weight + up to 3
//    token fragment reads feed up to 12 MFMAs; the next step's fragments load
//    while the current step's MFMAs run, and the last step of a stage is
//    deferred past the next barrier.  Token blocks past the expert's row
//    count are neither loaded nor multiplied.
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int NTOKB = 10;                        // token blocks (32 rows) per chunk
constexpr int MCH = NTOKB * 32;                  // token rows per chunk (320)
constexpr int TBW = (NTOKB + 3) / 4;             // most token blocks one wavefront owns (3)
constexpr int NW = 128;                          // weight rows per unit
constexpr int BK = 64;                           // K slice per stage
constexpr int KS = BK / 16;                      // MFMA K steps per stage
constexpr int CPR = BK / 8;                      // 16-byte chunks per row of a slice
constexpr int X_CH = MCH * CPR;                  // chunks of a token stage
constexpr int W_CH = NW * CPR;                   // chunks of a weight stage
constexpr int X_LD = X_CH / 256;                 // token DMA instructions per wavefront per stage (10)
constexpr int W_LD = W_CH / 256;                 // weight DMA instructions per wavefront per stage (4)
constexpr int WAHEAD = 3;                        // weight stages in flight ahead of the computed one
constexpr int NWSET = WAHEAD + 1;                // weight ring depth
constexpr int kNxcd = 8;
static_assert(X_CH % 256 == 0 && W_CH % 256 == 0, "whole DMA instructions");
static_assert((2 * X_CH + NWSET * W_CH) * 16 + 8 * (kMaxE + 8) <= 160 * 1024, "LDS budget");

// Physical 16-byte slot of logical chunk `ch` of row `row` in a slice: the
// XOR makes the 16 rows that one 16-lane group of an operand fetch touches
// land on 16 distinct 16-byte bank groups of a 256-byte LDS line.
__device__ __forceinline__ int swz(int row, int ch) { return row * 8 + (ch ^ ((row >> 1) & 7)); }

// One 16-byte-per-lane global -> LDS transfer (global_load_lds_dwordx4): lane
// l's 16 bytes land at LDS address lds + 16*l.  Issued as inline asm so the
// compiler does not treat every later LDS read as dependent on it (it would
// otherwise drain all loads in flight before the first ds_read); completion
// is awaited explicitly.  m0 is written only by these asm statements in this
// translation unit, so the clobber of a reserved register is safe here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(gptr), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

// LDS byte address of a __shared__ object (wave-uniform).
__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr_t)p);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier without the memory fence of __syncthreads (which would
// also drain the loads still in flight for later stages).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// K loop of one token chunk.
//  * Token slices go through a 2-deep LDS ring (stage kt+1 is loaded while kt
//    is computed; they come from L2), weight slices through a (WAHEAD+1)-deep
//    ring (they come from HBM and need more bytes in flight).
//  * Per iteration the token DMAs of stage kt+1 are issued before the weight
//    DMAs of stage kt+WAHEAD.  Loads complete in issue order, so "at most the
//    newest W_LD operations in flight" at the top of iteration kt+1 means
//    token stage kt+1 and weight stage kt+1 (issued earlier) have landed
//    while the weight stages further ahead stay in flight.
//  * DMA instructions are interleaved one per MFMA (inline asm is a
//    scheduling boundary, so the source order is the issue order), token DMAs
//    only for blocks that hold rows.
//  * NTB = token blocks of this wavefront holding rows (blocks wave, wave+4,
//    wave+8); MFMAs of the others are skipped.
template <int NTB>
__device__ __forceinline__ void mainloop(u32x4* xring, u32x4* wring, const uint16_t* xbase,
                                         const int (&xofs)[X_LD], int nblk, const uint16_t* wbase,
                                         const int (&wofs)[W_LD], int Kdim, int nk, int wave, int lane,
                                         f32x16 (&acc)[4][TBW]) {
    const uint32_t xl0 = lds_addr_of(xring) + wave * 64 * 16;
    const uint32_t wl0 = lds_addr_of(wring) + wave * 64 * 16;
    auto dma_x = [&](int kt, int q) {   // token DMA q of stage kt (rows of block q)
        if (q < nblk) dma16(xbase + xofs[q] + kt * BK, xl0 + ((kt & 1) * X_CH + q * 256) * 16);
    };
    auto dma_w = [&](int kt, int q) {
        dma16(wbase + wofs[q] + kt * BK, wl0 + ((kt % NWSET) * W_CH + q * 256) * 16);
    };
    int woff[KS][4], xoff[KS][TBW];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const int ch = s * 2 + (lane >> 5);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) woff[s][nb] = swz(nb * 32 + (lane & 31), ch);
#pragma unroll
        for (int i = 0; i < TBW; ++i) xoff[s][i] = swz((wave + 4 * i) * 32 + (lane & 31), ch);
    }

    // prologue: token stage 0, weight stages 0..WAHEAD-1
#pragma unroll
    for (int q = 0; q < X_LD; ++q) dma_x(0, q);
#pragma unroll
    for (int st = 0; st < WAHEAD; ++st)
        if (st < nk)
#pragma unroll
            for (int q = 0; q < W_LD; ++q) dma_w(st, q);

    // Fragment registers: step s of a stage uses set s&1.  The last step of
    // stage kt is deferred past the barrier of iteration kt+1, so its MFMAs
    // keep the matrix pipe busy while stage kt+1's first fragments load.
    bf16x8 wf[2][4], xf[2][TBW];
    for (int kt = 0; kt < nk; ++kt) {
        // ---- wait for token stage kt and weight stage kt ------------------
        if (kt == 0) {
            const int later = min(WAHEAD - 1, nk - 1);   // weight stages issued after stage 0
            if (later >= 2) wait_vm<2 * W_LD>();
            else if (later == 1) wait_vm<W_LD>();
            else wait_vm<0>();
        } else if (kt - 1 + WAHEAD < nk) {
            wait_vm<W_LD>();
        } else {
            wait_vm<0>();
        }
        lds_barrier();

        const bool more_x = kt + 1 < nk, more_w = kt + WAHEAD < nk;
        const u32x4* xb = xring + (kt & 1) * X_CH;
        const u32x4* wb = wring + (kt % NWSET) * W_CH;
        auto frags = [&](int s, int buf) {
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) wf[buf][nb] = __builtin_bit_cast(bf16x8, wb[woff[s][nb]]);
#pragma unroll
            for (int i = 0; i < NTB; ++i) xf[buf][i] = __builtin_bit_cast(bf16x8, xb[xoff[s][i]]);
        };
        // DMA slots in issue order: token q = 0..X_LD-1, then weight q = 0..W_LD-1
        int slot = 0;
        auto next_dma = [&]() {
            if (slot < X_LD) {
                if (more_x) dma_x(kt + 1, slot);
            } else if (slot < X_LD + W_LD) {
                if (more_w) dma_w(kt + WAHEAD, slot - X_LD);
            }
            ++slot;
        };
        auto mfmas = [&](int buf, bool with_dma) {
#pragma unroll
            for (int i = 0; i < NTB; ++i)
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) {
                    acc[nb][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[buf][nb], xf[buf][i], acc[nb][i], 0, 0, 0);
                    if (with_dma) next_dma();
                }
        };
        if (NTB == 0) {
#pragma unroll
            for (int d = 0; d < X_LD + W_LD; ++d) next_dma();
        } else {
            frags(0, 0);
            if (kt > 0) mfmas((KS - 1) & 1, true);     // deferred last step of stage kt-1
#pragma unroll
            for (int s = 0; s < KS - 1; ++s) {
                frags(s + 1, (s + 1) & 1);
                mfmas(s & 1, true);
            }
#pragma unroll
            for (int d = 0; d < X_LD + W_LD; ++d) next_dma();   // slots not yet used (no-op when exhausted)
        }
    }
    if (NTB > 0 && nk > 0)
    {
#pragma unroll
        for (int i = 0; i < NTB; ++i)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
                acc[nb][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[(KS - 1) & 1][nb], xf[(KS - 1) & 1][i],
                                                                    acc[nb][i], 0, 0, 0);
    }
    lds_barrier();   // the rings are free before the next chunk / unit refills them
}

template <int MODE>  // 0: FC1 + SwiGLU (out = act [R,F]); 1: FC2 (out = expert_out [R,H])
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_bf16(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, uint16_t* __restrict__ Out,
    const int64_t* __restrict__ seg_off, const int32_t* __restrict__ kept, int E, long long R, int Kdim,
    int Wrows, int Nout, int n_units) {
    __shared__ u32x4 xring[2 * X_CH];
    __shared__ u32x4 wring[NWSET * W_CH];
    __shared__ int s_list[kMaxE];      // active experts of this XCD, ascending
    __shared__ int s_rows[kMaxE];      // their row counts (clipped to R)
    __shared__ int s_cnt;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = gridDim.x, b = blockIdx.x;
    const int nx = (G % kNxcd == 0) ? kNxcd : 1;
    const int xcd = b % nx, P = G / nx, j = b / nx;

    // ---- this XCD's experts that have rows (wavefront 0, ballot compaction) --
    if (wave == 0) {
        int run = 0;
        for (int c = 0; c * nx < E; c += 64) {
            const int e = xcd + nx * (c + lane);
            int m = 0;
            if (e < E) {
                const long long so = seg_off[e];
                long long mm = so < R ? (long long)kept[e] : 0;
                if (so + mm > R) mm = R - so;
                m = (int)mm;
            }
            const unsigned long long act = __ballot(m > 0);
            if (m > 0) {
                const int pos = run + __popcll(act & ((1ull << lane) - 1ull));
                s_list[pos] = e;
                s_rows[pos] = m;
            }
            run += __popcll(act);
        }
        if (lane == 0) s_cnt = run;
    }
    __syncthreads();
    const int total = s_cnt * n_units;

    for (int t = j; t < total; t += P) {
        const int slot = t / n_units, nt = t - slot * n_units;
        const int e = s_list[slot];
        const int me = s_rows[slot];
        const long long seg = seg_off[e];
        const uint16_t* Wb = W + (size_t)e * Wrows * Kdim;
        const int n0 = (MODE == 0) ? nt * 64 : nt * 128;

        // weight DMA q of wavefront w fills slots (q*4+w)*64.. of a stage:
        // rows 8*(q*4+w)..+7, each lane the logical chunk of its slot
        int wofs[W_LD];
#pragma unroll
        for (int q = 0; q < W_LD; ++q) {
            const int p = (q * 4 + wave) * 64 + lane;
            const int row = p / CPR;
            const int ch = swz(row, p % CPR) - row * CPR;   // XOR is its own inverse
            const int wr = (MODE == 0) ? (row < 64 ? n0 + row : Nout + n0 + row - 64) : n0 + row;
            wofs[q] = wr * Kdim + ch * 8;
        }

        for (int m0 = 0; m0 < me; m0 += MCH) {
            const int mv = min(MCH, me - m0);
            const int nblk = (mv + 31) / 32;                // token blocks holding rows
            const uint16_t* Xb = X + (size_t)(seg + m0) * Kdim;
            // token DMA q covers rows 32q + 8*wave .. +7 (block q)
            int xofs[X_LD];
#pragma unroll
            for (int q = 0; q < X_LD; ++q) {
                const int p = (q * 4 + wave) * 64 + lane;
                const int row = p / CPR;
                const int ch = swz(row, p % CPR) - row * CPR;
                xofs[q] = min(row, mv - 1) * Kdim + ch * 8;   // rows past the group re-read a valid row
            }
            // token blocks of this wavefront that hold rows (wave-uniform)
            const int ntb = min(TBW, max(0, (nblk - wave + 3) / 4));

            f32x16 acc[4][TBW];
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                for (int i = 0; i < TBW; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[nb][i][r] = 0.f;

            const int nk = Kdim / BK;
            switch (ntb) {
                case 3: mainloop<3>(xring, wring, Xb, xofs, nblk, Wb, wofs, Kdim, nk, wave, lane, acc); break;
                case 2: mainloop<2>(xring, wring, Xb, xofs, nblk, Wb, wofs, Kdim, nk, wave, lane, acc); break;
                case 1: mainloop<1>(xring, wring, Xb, xofs, nblk, Wb, wofs, Kdim, nk, wave, lane, acc); break;
                default: mainloop<0>(xring, wring, Xb, xofs, nblk, Wb, wofs, Kdim, nk, wave, lane, acc); break;
            }

            // ---- epilogue: lane holds token (lane&31) of each token block and
            // weight rows 8*(r/4) + 4*(lane/32) + r%4 of each weight block.
#pragma unroll
            for (int i = 0; i < TBW; ++i) {
                const int tok = (wave + 4 * i) * 32 + (lane & 31);
                if (i >= ntb || tok >= mv) continue;
                uint16_t* orow = Out + (size_t)(seg + m0 + tok) * Nout + n0;
                if (MODE == 0) {
#pragma unroll
                    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                        for (int g4 = 0; g4 < 4; ++g4) {
                            float a[4];
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                const float g = acc[nb][i][g4 * 4 + q], u = acc[nb + 2][i][g4 * 4 + q];
                                a[q] = g / (1.f + __expf(-g)) * u;
                            }
                            uint2 v;
                            v.x = pack_bf16x2(a[0], a[1]);
                            v.y = pack_bf16x2(a[2], a[3]);
                            *(uint2*)(orow + nb * 32 + g4 * 8 + (lane >> 5) * 4) = v;
                        }
                } else {
#pragma unroll
                    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                        for (int g4 = 0; g4 < 4; ++g4) {
                            uint2 v;
                            v.x = pack_bf16x2(acc[nb][i][g4 * 4 + 0], acc[nb][i][g4 * 4 + 1]);
                            v.y = pack_bf16x2(acc[nb][i][g4 * 4 + 2], acc[nb][i][g4 * 4 + 3]);
                            *(uint2*)(orow + nb * 32 + g4 * 8 + (lane >> 5) * 4) = v;
                        }
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm_bf16(const moe_handle* h, int stage, int F, const void* in, const void* w,
                            void* out, int num_cu, hipStream_t s) {
    const moe_desc& d = h->desc;
    const long long R = d.out_rows;
    if (R == 0) return hipSuccess;
    int grid = num_cu - num_cu % kNxcd;
    if (grid < kNxcd) grid = num_cu;
    if (stage == 0) {
        hipLaunchKernelGGL(k_gemm_bf16<0>, dim3(grid), dim3(256), 0, s, (const uint16_t*)in, (const uint16_t*)w,
                           (uint16_t*)out, h->seg_off, h->kept, d.E, R, d.H, 2 * F, F, F / 64);
    } else {
        hipLaunchKernelGGL(k_gemm_bf16<1>, dim3(grid), dim3(256), 0, s, (const uint16_t*)in, (const uint16_t*)w,
                           (uint16_t*)out, h->seg_off, h->kept, d.E, R, F, d.H, d.H, d.H / 128);
    }
    return hipGetLastError();
}

}  // namespace moe
