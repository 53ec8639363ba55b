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
// Design (CDNA4: 256 CUs in 8 XCDs, 4 MB L2 per XCD, 160 KB LDS per CU):
//  * Work unit = (expert, 256 weight rows): for FC1 the gate and up rows of
//    128 features, for FC2 256 output columns.  A unit takes all of the
//    expert's token rows at once, so each weight row is streamed from HBM
//    once per layer.  Segments of up to 256 rows take one 256-row pass.
//    Segments of 257..320 rows take one pass over units of 192 weight rows
//    (FC1: 96 features, FC2: 192 columns; 96 weight rows x up to 160 tokens
//    per wavefront = 240 accumulation registers); FC1's blocks then hold 16
//    features each, gate rows then up rows, so accumulators r and r+8 of a
//    lane are the gate and up values of one feature.  Longer segments, and
//    FC2 into the fp8 format, cut them into chunks of 320 rows taken by two
//    128-row passes (the token chunk is then read twice, from L2).
//  * The units of all experts, listed by residue class e mod 8, are cut into
//    8 contiguous runs of equal weight, one per XCD (workgroup b runs on XCD
//    b mod 8).  A unit's time is set by its weight stream, nearly whatever its
//    rows, so every unit of a segment of up to 320 rows weighs 1 (longer
//    segments: their number of 320-row chunks).  The 32 workgroups of an XCD walk its run in order and
//    move through K at the same pace, so a token slice comes from HBM once
//    per XCD that holds units of its expert and is then served by that XCD's
//    L2.
//  * 256-row pass: the four wavefronts form a 2x2 grid of 128 weight rows x
//    up to 128 tokens each (256 accumulation registers).  Weight slices (HBM)
//    are loaded with plain 16-byte loads into registers two 64-wide K stages
//    ahead and copied into a 2-slot LDS ring; token slices (L2) go straight
//    to LDS (global_load_lds_dwordx4) one stage ahead.  Measured on MI355X,
//    this keeps more weight bandwidth next to the token stream than loading
//    both through LDS-direct loads.  Each K step interleaves its MFMAs one by
//    one with the next step's fragment reads and with one kind of side work
//    (the copy into LDS, the token loads or the weight loads).
//  * 128-row pass: four wavefronts each own all 4 weight blocks and token
//    blocks w, w+4, w+8; both operands go global -> LDS directly (token ring
//    2 deep, weight ring 4 deep), in the same LDS as the 256-row pass.
//  * A 16-byte chunk swizzle keeps the LDS operand reads free of bank
//    conflicts (64 banks).  MFMA v_mfma_f32_32x32x16_bf16 with weights as the
//    A operand (rows of the 32x32 result = weight rows) and tokens as B
//    (columns): each lane holds 4 consecutive features of one token, so the
//    epilogue stores 8 bytes per lane and FC1's gate and up values of a
//    feature sit in the same lane.  Every output element accumulates its K
//    steps in ascending order in both passes.
#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BK = 64;                 // K per stage
constexpr int KS = BK / 16;            // MFMA K steps per stage
constexpr int CPR = BK / 8;            // 16-byte chunks per row of a stage
constexpr int WROWS = 256;             // weight rows per unit
constexpr int XROWS_A = 256;           // token rows of a 256-row pass
constexpr int XROWS_B = 320;           // token rows of a chunk of 128-row passes
constexpr int W_SLOT = WROWS * CPR;    // 16-byte chunks of a weight stage
constexpr int X_SLOT = XROWS_B * CPR;  // 16-byte chunks of a token stage
constexpr int kNxcd = 8;
constexpr int BIG_BLOCKS = 6;           // 32-row weight blocks of a unit for 257..320-row segments
static_assert((2 * W_SLOT + 2 * X_SLOT) * 16 + 14 * kMaxE + 64 <= 160 * 1024, "LDS budget");

// Physical 16-byte slot of logical chunk `ch` of row `row` in a stage (8
// chunks per row, 2 rows per 256-byte LDS line): the XOR spreads the 16 rows
// one 16-lane group of an operand fetch touches over 16 distinct bank groups.
__device__ __forceinline__ int swz(int row, int ch) { return row * CPR + (ch ^ ((row >> 1) & 7)); }

// Read one accumulator element where it lives (an accumulation register).
// The explicit read keeps the compiler from copying every accumulator into
// vector registers at once when the K loop ends.
__device__ __forceinline__ float acc_read(float a) {
    float v;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
    return v;
}

typedef __attribute__((address_space(1))) const char gchar;   // global memory
typedef __attribute__((address_space(1))) const u32x4 gu32x4;

// A global pointer value made explicitly wave-uniform (it is uniform by
// construction); both halves stay unsigned, and the result keeps the global
// address space so loads through it are global (not flat) loads.
__device__ __forceinline__ gchar* uniform_ptr(const char* p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (gchar*)(((uint64_t)hi << 32) | lo);
}

// One 16-byte-per-lane global -> LDS transfer (global_load_lds_dwordx4):
// address = sbase (wave-uniform) + voff (per lane), lane l's 16 bytes land at
// LDS byte address lds + 16*l.  Inline asm, so the compiler does not treat
// later LDS reads as dependent on it; completion is awaited explicitly.  m0
// is written only by these asm statements in this translation unit.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(gchar* sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "s"(lds)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p);
}

// Workgroup barrier without the memory fence of __syncthreads (a fence would
// also wait for the loads of later stages still in flight).  This wavefront's
// LDS writes are complete before it arrives.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Two floats -> two bf16 (lo in the low half), round to nearest even: one
// v_cvt_pk_bf16_f32 (replacing the software rounding measured the epilogue
// 1-2 % of the layer step faster).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) { return bf16x2_rne(lo, hi); }

// FC2 output in the fp8 combine format: e4m3 codes [rows, Nout] and one fp32
// scale per (row, 128 columns); q and s point at the chunk's first row.
struct QOut {
    uint8_t* q;
    float* s;
};

// Quantise and store one token's 128 output columns held by a lane pair
// (lanes l and l^32, 64 values each: blocks j = 0..3, 4 groups of 4
// consecutive columns): block amax over both lanes, scale = amax / 448,
// nearest-even e4m3 codes.  `cols` is the first of the 128 columns.
__device__ __forceinline__ void store_q128(const float (&v)[4][16], bool ok, int lane, QOut o, size_t row,
                                           int Nout, int cols) {
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) amax = fmaxf(amax, fabsf(v[j][r]));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    if (!ok) return;
    const float sc = e4m3_scale(amax);
    uint8_t* qrow = o.q + row * Nout + cols + (lane >> 5) * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
            *(uint32_t*)(qrow + j * 32 + g4 * 8) =
                e4m3_pack4(v[j][g4 * 4], v[j][g4 * 4 + 1], v[j][g4 * 4 + 2], v[j][g4 * 4 + 3], sc);
    if (lane < 32) o.s[row * (Nout / 128) + cols / 128] = sc;
}

// One pass: NWB weight blocks (32 rows) per wavefront over the workgroup's
// 2*NWB weight blocks, NXB token blocks in the chunk, NTB of them (blocks
// q, q+2, ...) owned by this wavefront.  All threads load; the MFMAs and the
// epilogue belong to the wavefront.
//   Weights: thread t loads row 32*b + t/8, 16-byte chunk t%8, of every
//   weight block b into registers (per-lane offset `voff` plus a wave-uniform
//   block base, wrow[b] = first row of block b) and writes it to LDS.
//   Tokens: DMA instruction b of wavefront w fills LDS chunk slots
//   256*b + 64*w + lane, i.e. row 32*b + 8*w + lane/8; `xoff`/`xoff_last`
//   are the per-lane offsets (the last block's rows clamped to the chunk).
template <int MODE, bool OUTQ, int NWB, int NXB, int NTB>
__device__ __forceinline__ void pass(u32x4* wlds, u32x4* xlds, gchar* wbase, const int (&wrow)[2 * NWB],
                                     gchar* xbase, uint32_t voff, uint32_t xoff, uint32_t xoff_last, int pitch,
                                     int nk, int lane, int wave, int p, int q, int mv, uint16_t* obase, int Nout,
                                     int ocol0, QOut qo, int vb) {
    constexpr int NWL = 2 * NWB;   // weight loads per thread per stage (one per block of 32 rows)
    // LDS write slot of this thread's chunk within a block (same for every block)
    const int tid = threadIdx.x;
    const int wsl = (tid >> 3) * CPR + ((tid & 7) ^ (((tid >> 3) >> 1) & 7));
    // operand fetch base of step s for rows (block*32 + lane%32)
    int fb[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const int r = lane & 31, ch = 2 * s + (lane >> 5);
        fb[s] = r * CPR + (ch ^ ((r >> 1) & 7));
    }

    f32x16 acc[NWB][NTB > 0 ? NTB : 1];
#pragma unroll
    for (int j = 0; j < NWB; ++j)
#pragma unroll
        for (int i = 0; i < (NTB > 0 ? NTB : 1); ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.f;

    u32x4 sw0[NWL], sw1[NWL];
    auto gload = [&](u32x4 (&sw)[NWL], int kt) {
        // stages past the end re-read the last one (valid memory); keeps the
        // number of loads in flight the same on every path.  Weights are read
        // once per layer: non-temporal loads (here and in the refill below),
        // so they do not displace the token slices the XCD's units re-read
        // from L2, nor the freshly written outputs the next kernel reads
        // (measured on MI355X: layer step 1.5 % faster than with plain refill
        // loads, the combine after FC2 7 %).
        const int k = min(kt, nk - 1) * (BK * 2);
#pragma unroll
        for (int b = 0; b < NWL; ++b)
            sw[b] = __builtin_nontemporal_load((const gu32x4*)(wbase + ((size_t)wrow[b] * pitch + k) + voff));
    };
    auto swrite = [&](const u32x4 (&sw)[NWL], int slot) {
        u32x4* wl = wlds + slot * W_SLOT + wsl;
#pragma unroll
        for (int b = 0; b < NWL; ++b) wl[b * 32 * CPR] = sw[b];
    };
    const uint32_t xl0 = lds_addr_of(xlds) + wave * 64 * 16;
    auto xdma = [&](int kt, int slot) {   // token stage kt -> LDS slot (NXB instructions per wavefront)
        const int k = min(kt, nk - 1) * (BK * 2);
        // a stage past the end is never read: every lane takes the same 16
        // bytes (one line per instruction, the count in flight unchanged)
        const bool live = kt < nk;
        const uint32_t xo = live ? xoff : 0u, xol = live ? xoff_last : 0u;
#pragma unroll
        for (int b = 0; b < NXB; ++b)
            dma16(xbase + ((size_t)(b * 32) * pitch + k), b == NXB - 1 ? xol : xo,
                  xl0 + (slot * X_SLOT + b * 256) * 16);
    };
    bf16x8 wf[2][NWB], xf[2][NTB > 0 ? NTB : 1];
    auto frags = [&](int slot, int s, int buf) {
        const u32x4* wl = wlds + slot * W_SLOT + fb[s] + p * NWB * 32 * CPR;
        const u32x4* xl = xlds + slot * X_SLOT + fb[s] + q * 32 * CPR;
#pragma unroll
        for (int j = 0; j < NWB; ++j) wf[buf][j] = __builtin_bit_cast(bf16x8, wl[j * 32 * CPR]);
#pragma unroll
        for (int i = 0; i < NTB; ++i) xf[buf][i] = __builtin_bit_cast(bf16x8, xl[i * 64 * CPR]);
    };
    auto mfmas = [&](int buf) {
#pragma unroll
        for (int i = 0; i < NTB; ++i)
#pragma unroll
            for (int j = 0; j < NWB; ++j)
                acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[buf][j], xf[buf][i], acc[j][i], 0, 0, 0);
    };
    constexpr int NMF = NWB * (NTB > 0 ? NTB : 1);      // MFMAs per step
    constexpr bool DMA_FIRST = NXB > 8 || MODE == 0;
    auto gload_h = [&](u32x4 (&sw)[NWL], int kt, int hh) {   // half hh of the refill loads
        const int k = min(kt, nk - 1) * (BK * 2);
        const uint32_t vo = kt < nk ? voff : 0u;   // past the end: one line per load, as in xdma
#pragma unroll
        for (int b = 0; b < NWL; ++b)
            if (b % 2 == hh)
                sw[b] = __builtin_nontemporal_load((const gu32x4*)(wbase + ((size_t)wrow[b] * pitch + k) + vo));
    };
    // One stage: 4 K steps of LDS slot `slot`; step s issues the fragment
    // reads of step s+1 and one kind of side work, interleaved one by one with
    // its MFMAs: step 0 the register -> LDS copy of weight stage kt+1, step 1
    // the token DMA of stage kt+1 (step 0 after the copy, for DMA_FIRST
    // passes; the DMA is inline asm, a scheduling boundary, so it issues after
    // its step's MFMAs), steps 2-3 the refill of the weight registers with
    // stage kt+3.  Loads complete in issue order: the
    // compiler's wait before the copy (it counts only its own loads, weight
    // stage kt+2 after kt+1) finds stage kt+1 already landed and leaves stage
    // kt+2 in flight; before the closing barrier token stage kt+1 must have
    // landed, with only the NWL weight loads issued after it still in flight.
    auto stage = [&](int slot, u32x4 (&sw)[NWL], int kt_x, int kt_load) {
        if (NTB > 0) frags(slot, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        auto step = [&](auto stc) {
            constexpr int st = decltype(stc)::value;
            if (NTB > 0 && st + 1 < KS) frags(slot, st + 1, (st + 1) & 1);
            if (NTB > 0) mfmas(st & 1);
            // FC1, and a pass of more than 8 token blocks, issue the DMA in
            // step 0, right after the copy (whose wait for the weight
            // registers, placed by the compiler, does not see the DMA), so
            // that it has one more step to land before the stage's closing
            // wait (measured on MI355X: FC1 1.2 % faster; FC2's 256-row pass
            // was 1.1 % slower with it).
            if (st == 0) {
                swrite(sw, slot ^ 1);
                if (DMA_FIRST) xdma(kt_x, slot ^ 1);
            } else if (st == 1) {
                if (!DMA_FIRST) xdma(kt_x, slot ^ 1);
            } else {
                gload_h(sw, kt_load, st - 2);
            }
            if (NTB > 0) {
                constexpr int nside = st == 0 ? NWL : st == 1 ? 0 : NWL / 2;
#pragma unroll
                for (int i = 0; i < NMF; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, st);
                    if (st + 1 < KS && i < NTB + NWB) __builtin_amdgcn_sched_group_barrier(0x100, 1, st);
                    if (i < nside) __builtin_amdgcn_sched_group_barrier(st == 0 ? 0x200 : 0x020, 1, st);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        };
        step(std::integral_constant<int, 0>{});
        step(std::integral_constant<int, 1>{});
        step(std::integral_constant<int, 2>{});
        step(std::integral_constant<int, 3>{});
        static_assert(KS == 4, "four K steps per stage");
        wait_vm<NWL>();
        lds_barrier();
    };

    // prologue: token stage 0, weight stages 0 and 1 in flight; weight stage 0
    // to slot 0; weight stage 2 in flight; token stage 0 and weight stage 0
    // landed before the barrier (weight stages 1 and 2 may still fly).
    xdma(0, 0);
    gload(sw0, 0);
    gload(sw1, 1);
    swrite(sw0, 0);
    gload(sw0, 2);
    wait_vm<2 * NWL>();
    lds_barrier();
    // nk is even: each trip computes two stages from slots 0 and 1.
    for (int kt = 0; kt < nk; kt += 2) {
        stage(0, sw1, kt + 1, kt + 3);
        stage(1, sw0, kt + 2, kt + 4);
    }
    wait_vm<0>();

    // epilogue: lane holds token (lane&31) of each token block and weight rows
    // 8*(r/4) + 4*(lane/32) + r%4 of each weight block
    auto store_block = [&](auto ic) {
        constexpr int i = decltype(ic)::value;
        if constexpr (i < NTB && OUTQ) {
            static_assert(MODE == 1 && NWB == 4, "fp8 output: FC2, 128 columns per wavefront");
            __builtin_amdgcn_sched_barrier(0);
            const int tok = (q + 2 * i) * 32 + (lane & 31);
            float v[4][16];
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) v[j][r] = acc_read(acc[j][i][r]);
            store_q128(v, tok < mv, lane, qo, (size_t)tok, Nout, ocol0);
        } else if constexpr (i < NTB && NWB == 4 && (MODE == 0 || MODE == 1)) {
            // Whole-line stores: the wavefront's outputs for this token block
            // (FC1: 64 features = 128 B per token, FC2: 128 columns = 256 B)
            // go through its own part of token slot 1, then leave as whole row
            // segments, 16 bytes per lane.  Token slot 1 is free after the K
            // loop (its last reads end at the final barrier) and is written
            // next only after the following unit's prologue barrier.  Only
            // this wavefront touches its part, and its LDS operations run in
            // order, so no barrier is needed here.  Rows are padded by 16 bytes
            // (consecutive rows start 4 banks apart), so every access is one
            // base address plus a constant offset.
            __builtin_amdgcn_sched_barrier(0);
            constexpr int RB = MODE == 0 ? 128 : 256;              // bytes of a token row
            constexpr int RS = RB + 16;                             // row stride in LDS
            constexpr int NC = RB / 16;                             // 16-byte chunks per row
            constexpr int RPI = 64 / NC;                            // token rows per store instruction
            static_assert(4 * 32 * RS <= X_SLOT * 16, "epilogue staging fits token slot 1");
            int ln;                                                 // the lane, kept from being hoisted
            asm volatile("v_mov_b32 %0, %1" : "=v"(ln) : "v"(lane));
            char* st = (char*)(xlds + X_SLOT) + wave * (32 * RS);
            char* wr = st + (ln & 31) * RS + (ln >> 5) * 8;        // this lane's token row, its 8-byte half
            if constexpr (MODE == 0) {
#pragma unroll
                for (int j = 0; j < NWB / 2; ++j)
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        float a[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float g = acc_read(acc[j][i][g4 * 4 + r]);
                            const float u = acc_read(acc[j + NWB / 2][i][g4 * 4 + r]);
                            a[r] = g / (1.f + __expf(-g)) * u;
                        }
                        uint2 v;
                        v.x = pack_bf16x2(a[0], a[1]);
                        v.y = pack_bf16x2(a[2], a[3]);
                        *(uint2*)(wr + (j * 4 + g4) * 16) = v;
                    }
            } else {
#pragma unroll
                for (int j = 0; j < NWB; ++j)
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        uint2 v;
                        v.x = pack_bf16x2(acc_read(acc[j][i][g4 * 4 + 0]), acc_read(acc[j][i][g4 * 4 + 1]));
                        v.y = pack_bf16x2(acc_read(acc[j][i][g4 * 4 + 2]), acc_read(acc[j][i][g4 * 4 + 3]));
                        *(uint2*)(wr + (j * 4 + g4) * 16) = v;
                    }
            }
            const int tok0 = (q + 2 * i) * 32, rl = ln / NC, ch = ln % NC;
            const char* rd = st + rl * RS + ch * 16;
            uint16_t* od = obase + (size_t)(tok0 + rl) * Nout + ocol0 + ch * 8;
#pragma unroll
            for (int k = 0; k < 32 / RPI; ++k) {
                const u32x4 v = *(const u32x4*)(rd + k * RPI * RS);
                if (tok0 + k * RPI + rl < mv) *(u32x4*)(od + (size_t)(k * RPI) * Nout) = v;
            }
        } else if constexpr (i < NTB && NWB <= 3 && !OUTQ) {
            // The same whole-line path for the three-block pass (segments of
            // 257..320 rows): FC2 96 columns = 192 B per token, FC1's
            // interleaved blocks 48 features = 96 B; a unit's last blocks may
            // not exist (vb), so the row width is counted at run time.
            __builtin_amdgcn_sched_barrier(0);
            constexpr int BB = MODE == 2 ? 32 : 64;                 // bytes per weight block and token
            constexpr int RS = NWB * BB + 16;                       // padded row stride in LDS
            constexpr int LPR = MODE == 2 ? 8 : 16;                 // lanes per row when storing
            constexpr int RPI = 64 / LPR;                           // token rows per store instruction
            static_assert(4 * 32 * RS <= X_SLOT * 16, "epilogue staging fits token slot 1");
            const int nvb = min(NWB, max(0, vb - p * NWB));         // this wavefront's blocks that exist (uniform)
            int ln;                                                 // the lane, kept from being hoisted
            asm volatile("v_mov_b32 %0, %1" : "=v"(ln) : "v"(lane));
            char* st = (char*)(xlds + X_SLOT) + wave * (32 * RS);
            char* wr = st + (ln & 31) * RS + (ln >> 5) * 8;
#pragma unroll
            for (int j = 0; j < NWB; ++j) {
                if (j >= nvb) continue;
                if constexpr (MODE == 2) {
                    // rows 0..15 of the block gate, 16..31 up: accumulators r and r + 8
#pragma unroll
                    for (int g = 0; g < 2; ++g) {
                        float a[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float gt = acc_read(acc[j][i][4 * g + r]);
                            const float u = acc_read(acc[j][i][8 + 4 * g + r]);
                            a[r] = gt / (1.f + __expf(-gt)) * u;
                        }
                        uint2 v;
                        v.x = pack_bf16x2(a[0], a[1]);
                        v.y = pack_bf16x2(a[2], a[3]);
                        *(uint2*)(wr + j * BB + g * 16) = v;
                    }
                } else {
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        uint2 v;
                        v.x = pack_bf16x2(acc_read(acc[j][i][g4 * 4 + 0]), acc_read(acc[j][i][g4 * 4 + 1]));
                        v.y = pack_bf16x2(acc_read(acc[j][i][g4 * 4 + 2]), acc_read(acc[j][i][g4 * 4 + 3]));
                        *(uint2*)(wr + j * BB + g4 * 16) = v;
                    }
                }
            }
            const int tok0 = (q + 2 * i) * 32, rl = ln / LPR, ch = ln % LPR;
            const bool cv = ch < nvb * (BB / 16);                   // this lane's 16 bytes exist
            const char* rd = st + rl * RS + ch * 16;
            uint16_t* od = obase + (size_t)(tok0 + rl) * Nout + ocol0 + ch * 8;
#pragma unroll
            for (int k = 0; k < 32 / RPI; ++k) {
                if (cv && tok0 + k * RPI + rl < mv) {
                    const u32x4 v = *(const u32x4*)(rd + k * RPI * RS);
                    *(u32x4*)(od + (size_t)(k * RPI) * Nout) = v;
                }
            }
        } else if constexpr (i < NTB) {
            static_assert(NWB == 0, "every pass shape has a staged epilogue above");
        }
    };
    store_block(std::integral_constant<int, 0>{});
    store_block(std::integral_constant<int, 1>{});
    store_block(std::integral_constant<int, 2>{});
    store_block(std::integral_constant<int, 3>{});
    store_block(std::integral_constant<int, 4>{});
    static_assert(NTB <= 5, "one store_block call per token block");
}

// Weight-row offsets of the pass over features/columns [f0, f0 + 32*2*NWB/(MODE==0 ? 2 : 1))
// and token-row offsets of the chunk, then the pass itself for this
// wavefront's token-block count.
// MODE 2 (FC1, units of segments of 257..320 rows): each 32-row block holds
// 16 features, rows 0..15 their gate rows and 16..31 their up rows; `vb` is
// the number of blocks of the unit that exist (the rest re-read the last one
// and are not stored).
template <int MODE, bool OUTQ, int NWB, int NXB>
__device__ __forceinline__ void run_pass(u32x4* wlds, u32x4* xlds, const char* We, const char* Xc, int Kdim,
                                         int Nout, int f0, int mv, uint16_t* ochunk, QOut qo, int lane, int p,
                                         int q, int vb = 2 * NWB) {
    const int tid = threadIdx.x;
    const int r8 = tid >> 3, c8 = (tid & 7) * 16;   // row within a 32-row block, byte offset of the chunk
    // first weight row of each 32-row block of the pass (blocks never straddle
    // the gate/up boundary, so rows inside a block are consecutive)
    int wrow[2 * NWB];
#pragma unroll
    for (int b = 0; b < 2 * NWB; ++b) {
        const int r = b * 32;
        const int bv = b < vb ? b : vb - 1;
        if (MODE == 0) {
            // wavefront p: NWB/2 gate blocks then NWB/2 up blocks of features
            // f0 + p*16*NWB .. +16*NWB-1
            const int pp = r / (32 * NWB), rr = r % (32 * NWB), half = 16 * NWB;
            wrow[b] = rr < half ? f0 + pp * half + rr : Nout + f0 + pp * half + rr - half;
        } else if (MODE == 2) {
            wrow[b] = f0 + 16 * bv;          // first feature of the block (gate row; up rows via voff)
        } else {
            wrow[b] = f0 + 32 * bv;
        }
    }
    const int pitch = Kdim * 2;
    // MODE 2: rows 16..31 of a block are the up rows, Nout rows further on
    const uint32_t vrow = MODE == 2 && r8 >= 16 ? (uint32_t)(r8 + Nout - 16) : (uint32_t)r8;
    const uint32_t voff = vrow * (uint32_t)pitch + (uint32_t)c8;
    // token DMA lane: row 8*wave + lane/8 of a block, logical chunk of its swizzled slot
    const int wave = tid >> 6, lane8 = (tid & 63) >> 3;
    const int xr = 8 * wave + lane8;
    const int xch = (tid & 7) ^ ((xr >> 1) & 7);
    const uint32_t xoff = (uint32_t)xr * (uint32_t)pitch + (uint32_t)xch * 16u;
    const uint32_t xoff_last = (uint32_t)min(xr, mv - 1 - (NXB - 1) * 32) * (uint32_t)pitch + (uint32_t)xch * 16u;
    const int nk = Kdim / BK;
    const int ocol0 = MODE != 1 ? f0 + p * 16 * NWB : f0 + p * 32 * NWB;
    // a unit's last blocks may not exist (vb): wavefronts with none of its
    // blocks only load and keep the barriers, with no MFMAs (the three-block
    // pass, whose experts' last unit holds 2 of 6 blocks)
    if constexpr (NWB == 3) {
        if (p * NWB >= vb) {
            pass<MODE, OUTQ, NWB, NXB, 0>(wlds, xlds, uniform_ptr(We), wrow, uniform_ptr(Xc), voff, xoff, xoff_last,
                                          pitch, nk, lane, __builtin_amdgcn_readfirstlane(wave), p, q, mv, ochunk,
                                          Nout, ocol0, qo, vb);
            return;
        }
    }
    if (q == 0)
        pass<MODE, OUTQ, NWB, NXB, (NXB + 1) / 2>(wlds, xlds, uniform_ptr(We), wrow, uniform_ptr(Xc), voff, xoff,
                                                  xoff_last, pitch, nk, lane, __builtin_amdgcn_readfirstlane(wave), p,
                                                  q, mv, ochunk, Nout, ocol0, qo, vb);
    else
        pass<MODE, OUTQ, NWB, NXB, NXB / 2>(wlds, xlds, uniform_ptr(We), wrow, uniform_ptr(Xc), voff, xoff,
                                            xoff_last, pitch, nk, lane, __builtin_amdgcn_readfirstlane(wave), p, q,
                                            mv, ochunk, Nout, ocol0, qo, vb);
}

// ---- 128-row passes (segments of 257..320 rows) ------------------------------
// Work unit = (expert, 128 weight rows): FC1 64 gate + 64 up rows, FC2 128
// output columns.  Four wavefronts, each owning all 4 weight blocks and token
// blocks w, w+4, w+8 of a chunk of up to 320 rows.  Token slices come from L2
// through a 2-deep LDS ring and weight slices from HBM through a 4-deep ring,
// both by LDS-direct loads; the rings alias the LDS of the 256-row passes.
constexpr int H_NTOKB = 10;                      // token blocks (32 rows) per chunk
constexpr int H_MCH = H_NTOKB * 32;              // token rows per chunk (320)
constexpr int TBW = (H_NTOKB + 3) / 4;           // most token blocks one wavefront owns (3)
constexpr int H_NW = 128;                        // weight rows per pass
constexpr int X_CH = H_MCH * CPR;                // chunks of a token stage
constexpr int W_CH = H_NW * CPR;                 // chunks of a weight stage
constexpr int X_LD = X_CH / 256;                 // token DMA instructions per wavefront per stage (10)
constexpr int W_LD = W_CH / 256;                 // weight DMA instructions per wavefront per stage (4)
constexpr int WAHEAD = 3;                        // weight stages in flight ahead of the computed one
constexpr int NWSET = WAHEAD + 1;                // weight ring depth
static_assert(2 * X_CH == 2 * X_SLOT && NWSET * W_CH == 2 * W_SLOT, "128-row rings alias the 256-row slots");

// One 16-byte-per-lane global -> LDS transfer from a per-lane 64-bit address.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16v(const void* gptr, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(gptr), "s"(lds) : "memory", "m0");
}
// The same with the non-temporal cache policy, for data read once (weights).
__device__ __forceinline__ void dma16v_nt(const void* gptr, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" : : "v"(gptr), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

typedef __bf16 bf16x8h __attribute__((ext_vector_type(8)));

// K loop of a 128-row pass over one token chunk.
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
        if (q < nblk) dma16v(xbase + xofs[q] + kt * BK, xl0 + ((kt & 1) * X_CH + q * 256) * 16);
    };
    auto dma_w = [&](int kt, int q) {
        dma16v_nt(wbase + wofs[q] + kt * BK, wl0 + ((kt % NWSET) * W_CH + q * 256) * 16);
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

// One 128-row pass of unit rows: weights from We (expert base), features
// (FC1) / columns (FC2) starting at n0, over a chunk of me_c rows starting at
// token row X (segment row m0 = 0 of the chunk), output rows Out.
template <int MODE, bool OUTQ>
__device__ __forceinline__ void half_pass(u32x4* xring, u32x4* wring, const uint16_t* X, const uint16_t* Wb,
                                          uint16_t* Out, QOut qo, long long seg, int me, int Kdim, int Nout, int n0,
                                          int wave, int lane) {
    // the rings span both 256-row weight slots: every wavefront has finished
    // the previous unit's whole-line epilogue (weight slot 1) before any DMA
    lds_barrier();
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

        for (int m0 = 0; m0 < me; m0 += H_MCH) {
            const int mv = min(H_MCH, me - m0);
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
                __builtin_amdgcn_sched_barrier(0);
                const int tok = (wave + 4 * i) * 32 + (lane & 31);
                if constexpr (OUTQ) {
                    if (i >= ntb) continue;          // wave-uniform
                    float v[4][16];
#pragma unroll
                    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) v[nb][r] = acc_read(acc[nb][i][r]);
                    store_q128(v, tok < mv, lane, qo, (size_t)(seg + m0 + tok), Nout, n0);
                    continue;
                }
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
                                const float g = acc_read(acc[nb][i][g4 * 4 + q]), u = acc_read(acc[nb + 2][i][g4 * 4 + q]);
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
                            v.x = pack_bf16x2(acc_read(acc[nb][i][g4 * 4 + 0]), acc_read(acc[nb][i][g4 * 4 + 1]));
                            v.y = pack_bf16x2(acc_read(acc[nb][i][g4 * 4 + 2]), acc_read(acc[nb][i][g4 * 4 + 3]));
                            *(uint2*)(orow + nb * 32 + g4 * 8 + (lane >> 5) * 4) = v;
                        }
                }
            }
        }
}

// MODE 0: FC1 + SwiGLU (out = act [R,F]); 1: FC2 (out = expert_out [R,H]);
// OUTQ (FC2 only): the output goes to Oq / Os in the fp8 combine format.
template <int MODE, bool OUTQ>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_bf16(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, uint16_t* __restrict__ Out,
    uint8_t* __restrict__ Oq, float* __restrict__ Os, const int64_t* __restrict__ seg_off,
    const int32_t* __restrict__ kept, int E, long long R, int Kdim, int Wrows, int Nout, int n_units) {
    // units of segments of 257..320 rows: BIG_BLOCKS blocks of 16 features (FC1) / 32 columns (FC2)
    const int n_big = MODE == 0 ? (Nout / 16 + BIG_BLOCKS - 1) / BIG_BLOCKS : (Nout / 32 + BIG_BLOCKS - 1) / BIG_BLOCKS;
    __shared__ u32x4 wlds[2 * W_SLOT];
    __shared__ u32x4 xlds[2 * X_SLOT];
    __shared__ short s_list[kMaxE];    // active experts, by residue class mod nxcd, then ascending
    __shared__ int s_rows[kMaxE];      // their row counts (clipped to R)
    __shared__ int s_pref[kMaxE + 1];  // first unit of each of them
    __shared__ int s_wpref[kMaxE + 1]; // weighted position of that unit
    __shared__ int s_cnt;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int p = wave >> 1, q = wave & 1;
    const int G = gridDim.x, b = blockIdx.x;
    const int nxcd = (G % kNxcd == 0) ? kNxcd : 1;
    const int xcd = b % nxcd, P = G / nxcd, j = b / nxcd;

    // ---- every expert with rows, its units and their weight (wavefront 0:
    // ballot compaction and wavefront prefix sums), listed by residue class
    // e mod nxcd.  A unit weighs the number of token chunks it takes (1 up to
    // 320 rows): units stream the same weight bytes, so their time depends
    // little on the rows below that. ----
    if (wave == 0) {
        int run = 0, run_u = 0, run_w = 0;
        const int nc = (E + 64 * nxcd - 1) / (64 * nxcd) * 64;         // list positions per residue class
        for (int c = 0; c < nxcd * nc; c += 64) {
            const int e = c / nc + nxcd * (c % nc + lane);
            int m = 0;
            if (e < E) {
                const long long so = seg_off[e];
                long long mm = so < R ? (long long)kept[e] : 0;
                if (so + mm > R) mm = R - so;
                m = (int)mm;
            }
            // segments of 257..320 rows take BIG_BLOCKS-block units (one pass)
            const int nu = m == 0 ? 0 : (!OUTQ && m > XROWS_A && m <= XROWS_B) ? n_big : n_units;
            const int wu = m > XROWS_B ? min((m + XROWS_B - 1) / XROWS_B, 1024) : 1;
            int iu = nu, iw = nu * wu;           // inclusive prefix sums over the lanes
            for (int d = 1; d < 64; d <<= 1) {
                const int su = __shfl_up(iu, d), sw = __shfl_up(iw, d);
                if (lane >= d) { iu += su; iw += sw; }
            }
            const unsigned long long act = __ballot(m > 0);
            if (m > 0) {
                const int pos = run + __popcll(act & ((1ull << lane) - 1ull));
                s_list[pos] = (short)e;
                s_rows[pos] = m;
                s_pref[pos] = run_u + iu - nu;
                s_wpref[pos] = run_w + iw - nu * wu;
            }
            run += __popcll(act);
            run_u += __shfl(iu, 63);
            run_w += __shfl(iw, 63);
        }
        if (lane == 0) {
            s_pref[run] = run_u;
            s_wpref[run] = run_w;
            s_cnt = run;
        }
    }
    __syncthreads();
    // XCD x takes the units whose weighted start lies in [x W / n, (x+1) W / n):
    // one contiguous run of the list, mostly residue class x, with at most a
    // few experts' units moved across class boundaries.  Its workgroups walk
    // the run in order, so an expert's token slices are read from HBM once
    // per XCD that holds units of it.
    const int cnt = s_cnt, wtot = s_wpref[cnt];
    auto unit_at = [&](int pos) {              // first unit whose weighted start is >= pos
        if (pos >= wtot) return s_pref[cnt];
        int lo = 0, hi = cnt - 1;              // last slot whose start is <= pos
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_wpref[mid] <= pos) lo = mid; else hi = mid - 1;
        }
        const int nu = s_pref[lo + 1] - s_pref[lo];
        const int wu = (s_wpref[lo + 1] - s_wpref[lo]) / nu;
        return s_pref[lo] + (pos - s_wpref[lo] + wu - 1) / wu;
    };
    const int t_lo = unit_at((int)((long long)wtot * xcd / nxcd));
    const int t_hi = unit_at((int)((long long)wtot * (xcd + 1) / nxcd));

    for (int t = t_lo + j; t < t_hi; t += P) {
        int lo = 0, hi = cnt - 1;            // last slot whose first unit is <= t
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_pref[mid] <= t) lo = mid; else hi = mid - 1;
        }
        const int slot = lo, nt = t - s_pref[slot];
        const int e = s_list[slot];
        const int me = s_rows[slot];
        if (!OUTQ && me > XROWS_A && me <= XROWS_B) {
            // one pass over all rows: 96 features (FC1) / 192 columns (FC2) per unit
            const char* We = (const char*)(W + (size_t)e * Wrows * Kdim);
            const char* Xc = (const char*)(X + (size_t)seg_off[e] * Kdim);
            uint16_t* oc = Out + (size_t)seg_off[e] * Nout;
            const int bsz = MODE == 0 ? 16 : 32;                  // features (FC1) / columns (FC2) per block
            const int f0 = nt * BIG_BLOCKS * bsz;
            const int vb = min(BIG_BLOCKS, Nout / bsz - nt * BIG_BLOCKS);
            const QOut qn = {nullptr, nullptr};
            // FC2: a unit of at most 2 blocks (an expert's last) takes one block
            // per wavefront pair.  (FC1 keeps the three-block pass: there the
            // faster unit ran ahead of its expert's others and re-read their
            // token slice from HBM, for no gain in time.)
            if (MODE == 1 && vb <= 2) {
                if ((me + 31) / 32 == 9)
                    run_pass<MODE == 0 ? 2 : 1, false, 1, 9>(wlds, xlds, We, Xc, Kdim, Nout, f0, me, oc, qn, lane, p, q, vb);
                else
                    run_pass<MODE == 0 ? 2 : 1, false, 1, 10>(wlds, xlds, We, Xc, Kdim, Nout, f0, me, oc, qn, lane, p, q, vb);
            } else if ((me + 31) / 32 == 9) {
                run_pass<MODE == 0 ? 2 : 1, false, 3, 9>(wlds, xlds, We, Xc, Kdim, Nout, f0, me, oc, qn, lane, p, q, vb);
            } else {
                run_pass<MODE == 0 ? 2 : 1, false, 3, 10>(wlds, xlds, We, Xc, Kdim, Nout, f0, me, oc, qn, lane, p, q, vb);
            }
            continue;
        }
        const long long seg = seg_off[e];
        const char* We = (const char*)(W + (size_t)e * Wrows * Kdim);
        const int u0 = nt * (MODE == 0 ? 128 : 256);    // first feature (FC1) / output column (FC2) of the unit

        for (int m0 = 0; m0 < me; ) {
            const int left = me - m0;
            const char* Xc = (const char*)(X + (size_t)(seg + m0) * Kdim);
            uint16_t* oc = OUTQ ? nullptr : Out + (size_t)(seg + m0) * Nout;
            const QOut qc = {OUTQ ? Oq + (size_t)(seg + m0) * Nout : nullptr,
                             OUTQ ? Os + (size_t)(seg + m0) * (Nout / 128) : nullptr};
            if (left <= XROWS_A) {
                const int mv = left, nblk = (mv + 31) / 32;
                switch (nblk) {
#define MOE_A(NB) case NB: run_pass<MODE, OUTQ, 4, NB>(wlds, xlds, We, Xc, Kdim, Nout, u0, mv, oc, qc, lane, p, q); break;
                    MOE_A(1) MOE_A(2) MOE_A(3) MOE_A(4) MOE_A(5) MOE_A(6) MOE_A(7) default: MOE_A(8)
#undef MOE_A
                }
                m0 += mv;
            } else {
                // 257..320 rows: two 128-row passes with the token chunk in L2
                const int mv = min(left, XROWS_B);
                const uint16_t* Wb = W + (size_t)e * Wrows * Kdim;
                const QOut qall = {Oq, Os};
                for (int h = 0; h < 2; ++h)
                    half_pass<MODE, OUTQ>(xlds, wlds, X, Wb, Out, qall, seg + m0, mv, Kdim, Nout,
                                          u0 + h * (MODE == 0 ? 64 : 128), wave, lane);
                m0 += mv;
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm_bf16(const moe_handle* h, int stage, int F, const void* in, const void* w,
                            void* out, float* out_scales, int num_cu, hipStream_t s) {
    const moe_desc& d = h->desc;
    const long long R = d.out_rows;
    if (R == 0) return hipSuccess;
    int grid = num_cu - num_cu % kNxcd;
    if (grid < kNxcd) grid = num_cu;
    if (stage == 0) {
        hipLaunchKernelGGL((k_gemm_bf16<0, false>), dim3(grid), dim3(256), 0, s, (const uint16_t*)in,
                           (const uint16_t*)w, (uint16_t*)out, nullptr, nullptr, h->seg_off, h->kept, d.E, R, d.H,
                           2 * F, F, F / 128);
    } else if (!out_scales) {
        hipLaunchKernelGGL((k_gemm_bf16<1, false>), dim3(grid), dim3(256), 0, s, (const uint16_t*)in,
                           (const uint16_t*)w, (uint16_t*)out, nullptr, nullptr, h->seg_off, h->kept, d.E, R, F, d.H,
                           d.H, d.H / 256);
    } else {   // FC2 into the fp8 combine format: out = e4m3 codes [R,H], out_scales [R,H/128]
        hipLaunchKernelGGL((k_gemm_bf16<1, true>), dim3(grid), dim3(256), 0, s, (const uint16_t*)in,
                           (const uint16_t*)w, nullptr, (uint8_t*)out, out_scales, h->seg_off, h->kept, d.E, R, F,
                           d.H, d.H, d.H / 256);
    }
    return hipGetLastError();
}

}  // namespace moe
