// Persistent decode layer: quantise-on-dispatch -> FC1 + SwiGLU -> activation
// quantiser -> FC2 -> combine in one launch, fed by device-side ticket queues
// (fp8 e4m3 expert weights with 128x128 block scales; decode-sized batches).
//
// Operation: TensorRT-LLM PR #16190 "Update CuTeDSL MegaMoE kernels" (first
// commit message: dispatch, FC1, FC2 and combine fused in one kernel for
// decode, with loads that wait on flags written by the producing stage;
// review-fix commit: the live-token trim and a launch that does nothing for
// an empty batch) on top of the routing metadata of Megatron-LM PR #6800 /
// DeepEP PR #716 (the same handle as the separate kernels).  The arithmetic
// is that of the separate launches, unit for unit: quantise-on-dispatch,
// the fp8 GEMM units, the row quantiser and the per-token combine are the
// same device functions, so the layer output is bit-identical to theirs.
//
// Work items, in their global order (every dependency points to an earlier
// item):
//   D(t,h)   quantise column groups 4h..4h+3 of token row t into each
//            kept copy's row (one group of 1024 columns per wavefront)
//   F1(a,u)  FC1 + SwiGLU units of the a-th expert holding rows     needs all D
//   Q(a)     quantise that expert's activation rows                 needs its F1
//   F2(a,u)  FC2 units of the expert                                needs its Q
//   C(t)     combine of token t                                     needs all F2
// Items are spread over 8 queues, one per XCD (tokens t % 8, experts a % 8);
// a workgroup takes tickets from the queue of the XCD it runs on (hardware
// register XCC_ID), so every F1 -> Q -> F2 dependency stays inside one XCD
// and its L2.  A workgroup only ever waits on items of lower global order.
// The lowest unfinished item is therefore always claimable: everything its
// queue's workgroups hold is lower, hence finished, so they take it next;
// its owner is running (a ticket is taken by a running workgroup) and its own
// dependencies are finished.  Progress does not depend on how many
// workgroups are resident at once, only on every XCD running at least one.
//
// Visibility.  Each XCD has its own L2; an acquire or release at agent scope
// invalidates or writes back the whole L2 of the XCD, which made the first
// form of this kernel (every dependency at agent scope) 1.7x slower.  Here a
// finished item's stores have completed in its XCD's L2 before the barrier
// that ends it (s_waitcnt vmcnt(0) in every wavefront).  Then:
//   * F1 and Q items (read only on their own XCD) are counted with relaxed
//     increments, and their readers, after seeing the count, invalidate only
//     the CU's L1 (buffer_inv sc0): the data are in the shared L2;
//   * D items (token rows read on every XCD) are counted per queue with
//     relaxed increments; the increment that completes a queue writes back
//     the XCD's L2 (release at agent scope) and counts the queue.  Before its
//     first F1 item a workgroup waits for every queue with D items; then the
//     first workgroup of each XCD to get there invalidates the XCD's L2
//     (acquire at agent scope) and marks it done, and the others wait for
//     that mark (its owner waits on nothing) and invalidate their CU's L1;
//   * F2 items are counted per queue with relaxed increments; the increment
//     that completes a queue writes back the XCD's L2 (release at agent scope,
//     covering every F2 item of the queue) and counts the queue; C items wait
//     for every queue, then acquire at agent scope.
// Counters are polled with agent-scope relaxed loads.  Every wait is bounded
// by the 100 MHz real-time counter (0.25 s unless the caller sets another
// bound): past the bound it sets bit 0 of the caller's status word and
// proceeds, and once any status bit is set every wait returns at once, so the
// kernel always runs to its end.  Bit 2 is the caller's abort request: set
// before the call or while the kernel runs, it ends every wait (the reset
// keeps it).  A workgroup whose XCC_ID is 8 or more sets bit 1 and does
// nothing (the queues assume eight XCDs numbered 0-7).
#include "device_ops.h"

namespace moe {
namespace {

using namespace ops;

constexpr int kQueues = 8;                            // one per XCD
constexpr int kCtlStride = 32;                        // ints between shared counters (128 bytes)
constexpr int kCtlDispatch = kQueues * kCtlStride;    // D items done
constexpr int kCtlFc2 = kCtlDispatch + kCtlStride;    // queues whose F2 items are all done
constexpr int kCtlFc1 = kCtlFc2 + kCtlStride;         // F1 items done, per active expert
constexpr int kCtlQuant = kCtlFc1 + kMaxE;            // Q item done, per active expert
constexpr int kCtlFc2Q = kCtlQuant + kMaxE;           // F2 items done, per queue
constexpr int kCtlDispQ = kCtlFc2Q + kQueues * kCtlStride;   // D items done, per queue
constexpr int kCtlDinv = kCtlDispQ + kQueues * kCtlStride;   // per queue: 1 = its XCD's L2 being invalidated, 2 = done
constexpr int kCtlInts = kCtlDinv + kQueues * kCtlStride;
// fp8 GEMM units per F1 / F2 item: fewer, larger items spend fewer claims,
// polls and publications per byte of weights streamed
#ifndef MOE_DECODE_UNITS_PER_ITEM
#define MOE_DECODE_UNITS_PER_ITEM 2
#endif
constexpr int kUnitsPerItem = MOE_DECODE_UNITS_PER_ITEM;
// how a finished item is published (see the claim loop)
constexpr int kPubLocal = 2, kPubFc2 = 3, kPubDisp = 4;
// status bits: a wait ran past its bound; a workgroup ran on an XCD numbered
// 8 or more; the caller's abort request (kept by the reset)
constexpr int kStatusTimeout = 1, kStatusPlacement = 2, kStatusAbort = 4;

struct DecodeArgs {
    const uint16_t* x;          // [T,H] bf16 tokens
    const int32_t* row_id;      // [T,K]
    const float* copy_prob;     // [T,K]
    const int64_t* seg_off;     // [E+1]
    const int32_t* kept;        // [E]
    const uint8_t* w1;          // [E,2F,H] e4m3
    const float* w1s;           // [E,2F/128,H/128]
    const uint8_t* w2;          // [E,H,F] e4m3
    const float* w2s;           // [E,H/128,F/128]
    uint8_t* xq;                // [R,H] token codes
    float* xs;                  // [R,H/128]
    float* act;                 // [R,F] fp32 SwiGLU output
    uint8_t* aq;                // [R,F] activation codes
    float* as;                  // [R,F/128]
    uint16_t* eo;               // [R,H] bf16 expert output
    uint16_t* y;                // [T,H] bf16 layer output
    int* ctl;                   // kCtlInts control ints, zero at launch
    int* status;                // kStatus* bits
    long long wait_ticks;       // bound of every wait, in ticks of the 100 MHz real-time counter
    long long R;
    int T, H, F, K, E, apply;
};

__global__ __launch_bounds__(256) void k_decode_reset(int* __restrict__ ctl, int n, int* __restrict__ status) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) ctl[i] = 0;
    if (threadIdx.x == 0) status[0] &= kStatusAbort;
}

// Thread 0: wait until *c >= target (bounded).  (The branch is taken per
// wavefront, then per lane inside wavefront 0.)  The caller then acquires:
// acquire_agent for data written on another XCD, acquire_local for data
// written on this one.
__device__ __forceinline__ void wait_count(const DecodeArgs& a, int* c, int target, int wave, int lane) {
    if (wave == 0 && lane == 0) {
        // any status bit (a time-out elsewhere, or the caller's abort) ends every wait at once
        const long long t0 = (long long)__builtin_amdgcn_s_memrealtime();
        while (__hip_atomic_load(a.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0 &&
               __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
            if ((long long)__builtin_amdgcn_s_memrealtime() - t0 > a.wait_ticks) {
                __hip_atomic_fetch_or(a.status, kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
    __syncthreads();
}

// Data written on any XCD: invalidate this CU's L1 and this XCD's L2.
__device__ __forceinline__ void acquire_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

// Data written by a workgroup on this XCD: it sits in this XCD's L2 (the
// producer's stores completed there before its counter increment), so only
// this CU's L1 can hold an older copy; invalidate the L1 alone.
__device__ __forceinline__ void acquire_local() { asm volatile("buffer_inv sc0" ::: "memory"); }

// End of an item: this wavefront's stores have completed, then the barrier.
__device__ __forceinline__ void finish_item() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
}

// Publishing a finished item: every thread's stores have completed in this
// XCD's L2 at the barrier that ends the item (finish_item); at the top of the
// next turn of the claim loop, lane 0 of wavefront 0 increments the item's
// counter, then claims the next ticket.  D items are read on every XCD: their
// increment is a release at agent scope (this XCD's L2 is written back first).
// F1 and Q items are read only on their own XCD: a relaxed increment (no
// write-back).  F2 items count per queue; the increment that completes a
// queue writes back this XCD's L2 (every F2 item of the queue has completed
// its stores in it) and counts the queue done, with a release at agent scope;
// C items wait for every queue.
//
// The claim loop keeps its control flow uniform across each wavefront: the
// claim is made inside a branch on the wavefront index and read back from
// LDS with readfirstlane.  A thread-0-only increment at the end of an item
// followed by a thread-0-only claim at the loop top lets the compiler send
// the other lanes of wavefront 0 (and every lane of the other wavefronts)
// straight back to the loop's barrier, where they re-read the old ticket and
// repeat the same item without end; no such pair is left in the loop.

__global__ __launch_bounds__(256, 2) void k_decode_layer(DecodeArgs a) {
    __shared__ int s_list[kMaxE];    // experts holding rows, ascending
    __shared__ __attribute__((aligned(16))) unsigned char s_w[4 * kWaveLds];   // weight buffer per wavefront
    __shared__ int s_cnt;
    __shared__ int s_ticket;
    __shared__ int s_flag;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // The queue is this workgroup's XCD (hardware register XCC_ID), so the
    // producer and consumer of every F1 -> Q -> F2 dependency share an L2.
    const int q = __builtin_amdgcn_readfirstlane(__builtin_amdgcn_s_getreg(20 | (15 << 11)));   // XCC_ID[15:0]
    if (q >= kQueues) {
        if (tid == 0) __hip_atomic_fetch_or(a.status, kStatusPlacement, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }

    // ---- experts holding rows (every workgroup builds the same list) ----------
    if (wave == 0) {
        int run = 0;
        for (int c = 0; c < a.E; c += 64) {
            const int e = c + lane;
            bool has = false;
            if (e < a.E) {
                const long long so = a.seg_off[e];
                long long mm = so < a.R ? (long long)a.kept[e] : 0;
                if (so + mm > a.R) mm = a.R - so;
                has = mm > 0;
            }
            const unsigned long long act = __ballot(has);
            if (has) s_list[run + __popcll(act & ((1ull << lane) - 1ull))] = e;
            run += __popcll(act);
        }
        if (lane == 0) s_cnt = run;
    }
    __syncthreads();
    const int n_act = s_cnt;
    const int upe1 = a.F / kFeat, upe2 = a.H / kFeat2;
    const int nbH = a.H / 128, ngH = (nbH + kPQBlocks - 1) / kPQBlocks;
    // this queue's items: tokens q, q+8, ...; active experts q, q+8, ...
    const int nTq = a.T > q ? (a.T - q + kQueues - 1) / kQueues : 0;
    const int dpt = (ngH + 3) / 4;       // D items per token: four column groups each, one per wavefront
    const int nD = nTq * dpt;
    const int nA = n_act > q ? (n_act - q + kQueues - 1) / kQueues : 0;
    // items per expert: runs of kUnitsPerItem consecutive units (the last may be shorter)
    const int ipe1 = (upe1 + kUnitsPerItem - 1) / kUnitsPerItem, ipe2 = (upe2 + kUnitsPerItem - 1) / kUnitsPerItem;
    const int eF1 = nD + nA * ipe1, eQ = eF1 + nA, eF2 = eQ + nA * ipe2, eC = eF2 + nTq;
    const int nbF = a.F / 128, ngF = (nbF + kQBlocks - 1) / kQBlocks;
    int* ctl = a.ctl;

    const int nF2q = eF2 - eQ;           // F2 items of this queue
    int* done = nullptr;                 // counter of the item finished last turn
    int pub = 0;                         // and how it is published
    bool have_d = false;                 // this workgroup has acquired the D items' rows
    for (;;) {
        if (wave == 0) {
            int tk = 0;
            if (lane == 0) {
                if (pub == kPubDisp) {
                    if (__hip_atomic_fetch_add(done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nD - 1)
                        __hip_atomic_fetch_add(ctl + kCtlDispatch, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
                } else if (pub == kPubLocal) {
                    __hip_atomic_fetch_add(done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                } else if (pub == kPubFc2) {
                    if (__hip_atomic_fetch_add(done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nF2q - 1)
                        __hip_atomic_fetch_add(ctl + kCtlFc2, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
                }
                tk = __hip_atomic_fetch_add(ctl + q * kCtlStride, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            s_ticket = __builtin_amdgcn_readfirstlane(tk);
        }
        done = nullptr;
        pub = 0;
        __syncthreads();
        const int i = __builtin_amdgcn_readfirstlane(s_ticket);
        __syncthreads();                 // s_ticket is rewritten by the next claim
        if (i >= eC) break;
        if (i < nD) {
            // D(t, h): quantise-on-dispatch of token t, column groups 4h .. 4h+3 (one per wavefront)
            const long long t = q + (long long)kQueues * (i / dpt);
            const int g = 4 * (i % dpt) + wave;
            if (g < ngH) permute_quant_wave(a.x, a.H, a.K, (int)a.R, a.row_id, a.xq, a.xs, t, g * kPQBlocks, lane);
            finish_item();
            done = ctl + kCtlDispQ + q * kCtlStride;
            pub = kPubDisp;
        } else if (i < eF1) {
            const int k = i - nD, ai = q + kQueues * (k / ipe1), u0 = (k % ipe1) * kUnitsPerItem;
            if (!__builtin_amdgcn_readfirstlane(have_d)) {   // token rows never change after the D items: acquire once
                // every queue with D items has written them back; then one
                // workgroup per XCD invalidates the XCD's L2, and the others
                // wait for it (it waits on nothing) and invalidate their L1
                wait_count(a, ctl + kCtlDispatch, min(a.T, kQueues), wave, lane);
                int* dinv = ctl + kCtlDinv + q * kCtlStride;
                if (wave == 0) {
                    int first = 0;
                    if (lane == 0) {
                        int expect = 0;
                        first = __hip_atomic_compare_exchange_strong(dinv, &expect, 1, __ATOMIC_RELAXED,
                                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                    s_flag = __builtin_amdgcn_readfirstlane(first);
                }
                __syncthreads();
                const int first = __builtin_amdgcn_readfirstlane(s_flag);
                __syncthreads();
                if (first) {
                    acquire_agent();
                    __syncthreads();
                    if (wave == 0 && lane == 0)
                        __hip_atomic_store(dinv, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                } else {
                    wait_count(a, dinv, 2, wave, lane);
                    acquire_local();
                }
                have_d = true;
            }
            for (int u = u0; u < min(upe1, u0 + kUnitsPerItem); ++u)
                fp8_unit<0>(a.xq, a.xs, a.w1, a.w1s, a.act, a.seg_off, a.kept, a.R, a.H, 2 * a.F, a.F, s_list[ai], u,
                            lane, wave, s_w + wave * kWaveLds);
            finish_item();
            done = ctl + kCtlFc1 + ai;
            pub = kPubLocal;
        } else if (i < eQ) {
            // Q(a): the expert's activation rows, (row, 8-block group) per wavefront
            const int ai = q + kQueues * (i - eF1), e = s_list[ai];
            wait_count(a, ctl + kCtlFc1 + ai, ipe1, wave, lane);
            acquire_local();
            const long long seg = a.seg_off[e];
            long long me = a.kept[e];
            if (seg + me > a.R) me = a.R - seg;
            for (long long w = wave; w < me * ngF; w += 4)
                quant_row_wave<float>(a.act, a.F, a.aq, a.as, seg + w / ngF, (int)(w % ngF) * kQBlocks, lane);
            finish_item();
            done = ctl + kCtlQuant + ai;
            pub = kPubLocal;
        } else if (i < eF2) {
            const int k = i - eQ, ai = q + kQueues * (k / ipe2), u0 = (k % ipe2) * kUnitsPerItem;
            wait_count(a, ctl + kCtlQuant + ai, 1, wave, lane);
            acquire_local();
            for (int u = u0; u < min(upe2, u0 + kUnitsPerItem); ++u)
                fp8_unit<1>(a.aq, a.as, a.w2, a.w2s, a.eo, a.seg_off, a.kept, a.R, a.F, a.H, a.H, s_list[ai], u, lane,
                            wave, s_w + wave * kWaveLds);
            finish_item();
            done = ctl + kCtlFc2Q + q * kCtlStride;
            pub = kPubFc2;
        } else {
            // C(t): combine of token t once every FC2 unit is done
            const int t = q + kQueues * (i - eF2);
            wait_count(a, ctl + kCtlFc2, min(n_act, kQueues), wave, lane);
            acquire_agent();
            combine_token_wg((const u32x4*)a.eo, a.K, a.H / 8, (int)a.R, a.row_id, a.copy_prob, a.apply,
                             (u32x4*)a.y, t, wave, lane);
            __syncthreads();
        }
    }
}

size_t up256(size_t n) { return (n + 255) & ~(size_t)255; }

}  // namespace

size_t decode_layer_scratch_bytes(long long R, int H, int F) {
    return up256(fp8_mlp_scratch_bytes(R, H, F)) + up256((size_t)kCtlInts * 4);
}

hipError_t launch_decode_layer(const moe_handle* h, int F, const void* x, const void* w1, const float* w1s,
                               const void* w2, const float* w2s, void* scratch, void* expert_out, int apply_probs,
                               void* y, int32_t* status, long long wait_ticks, int num_cu, hipStream_t s) {
    const moe_desc& d = h->desc;
    const long long R = d.out_rows;
    // the scratch regions of the fp8 expert MLP, then the control ints
    char* base = (char*)scratch;
    DecodeArgs a;
    a.act = (float*)base;
    a.xq = (uint8_t*)(base + up256((size_t)R * F * 4));
    a.xs = (float*)((char*)a.xq + up256((size_t)R * d.H));
    a.aq = (uint8_t*)((char*)a.xs + up256((size_t)R * (d.H / 128) * 4));
    a.as = (float*)((char*)a.aq + up256((size_t)R * F));
    a.ctl = (int*)(base + up256(fp8_mlp_scratch_bytes(R, d.H, F)));
    a.x = (const uint16_t*)x;
    a.row_id = h->row_id;
    a.copy_prob = h->copy_prob;
    a.seg_off = h->seg_off;
    a.kept = h->kept;
    a.w1 = (const uint8_t*)w1;
    a.w1s = w1s;
    a.w2 = (const uint8_t*)w2;
    a.w2s = w2s;
    a.eo = (uint16_t*)expert_out;
    a.y = (uint16_t*)y;
    a.status = status;
    a.wait_ticks = wait_ticks;
    a.R = R;
    a.T = d.T;
    a.H = d.H;
    a.F = F;
    a.K = d.K;
    a.E = d.E;
    a.apply = apply_probs;
    hipLaunchKernelGGL(k_decode_reset, dim3(1), dim3(256), 0, s, a.ctl, kCtlInts, status);
    if (d.T == 0) return hipGetLastError();   // nothing to compute: no launch of the layer
    // two workgroups per CU (the fp8 units hold about 190 registers), a whole
    // number of workgroups per queue
    int grid = 2 * num_cu;
    grid = (grid + kQueues - 1) / kQueues * kQueues;
    hipLaunchKernelGGL(k_decode_layer, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
