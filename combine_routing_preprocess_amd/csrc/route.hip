// Routing metadata preprocessing (K1): per-expert counts, capacity, padding,
// segment offsets, the destination row of every copy and the overflow flag,
// entirely on the device so the host never waits for the counts.
//
// Operation: DeepEP PR #716 "perf: reuse HybridEP routing allgather buffer"
// (sections "Summary", "Memory impact", "Output and gradient regression",
// "Full HybridEP reference validation") and NeMo-Automodel PR #3931
// "perf(moe): sync-free HybridEP dispatch" (sections "What does this PR do ?",
// "Validation").
//
// Three launches, all graph-capturable and free of memsets (batches of up to
// 256 tokens with dense routing take one, k_route_small, below):
//  1. k_route_tiles  -- one wavefront per 64-token tile.  Every tile builds a
//     64-bit membership mask per expert in LDS (bit l = token l of the tile
//     routes to the expert).  popcount(mask) is the tile's count for that
//     expert and popcount(mask & lanes_below) is a token's stable rank inside
//     the tile, so ranks are deterministic without ordered atomics.  It also
//     writes each slot's expert id (or -1) and probability, and tile flags.
//     Boolean maps take k_route_tiles_sparse: four wavefronts per tile, each
//     over a quarter of the experts, joined by a scan of per-token counts.
//  2. k_route_scan   -- one 1024-thread workgroup: per-expert exclusive scan
//     of tile counts, raw counts, capacity, padding, exclusive scan over
//     experts, rows needed, flag word.
//  3. k_route_assign -- final destination row of every slot (or -1), source
//     token of every row (or -1 for pad/unused rows), permuted probabilities.
#include "moe_internal.h"

namespace moe {
namespace {

template <int FMT>
__global__ __launch_bounds__(64) void k_route_tiles(const void* __restrict__ routing,
                                                    const float* __restrict__ probs,
                                                    const int32_t* __restrict__ T_live_ptr, int T,
                                                    int E, int K, uint64_t* __restrict__ tile_mask,
                                                    int32_t* __restrict__ tile_err,
                                                    int32_t* __restrict__ row_id,
                                                    float* __restrict__ copy_prob) {
    __shared__ unsigned long long msk[kMaxE];
    const int lane = threadIdx.x;
    const int tile = blockIdx.x;
    const int t = tile * kTileTok + lane;
    int T_live = T;
    if (T_live_ptr) T_live = min(max(*T_live_ptr, 0), T);
    for (int e = lane; e < E; e += 64) msk[e] = 0ull;
    __syncthreads();
    int err = 0;
    const bool in = t < T;
    const bool live = t < T_live;
    static_assert(FMT != MOE_ROUTE_SPARSE_BOOL, "Boolean maps take k_route_tiles_sparse");
    {
        if (in) {
            const unsigned long long bit = 1ull << lane;
            for (int j = 0; j < K; ++j) {
                const size_t at = (size_t)t * K + j;
                const int e = (FMT == MOE_ROUTE_DENSE_I16) ? (int)((const int16_t*)routing)[at]
                                                           : ((const int32_t*)routing)[at];
                int oute = -1;
                float p = 0.f;
                if (live && e != -1) {
                    if (e < -1 || e >= E) {
                        err |= MOE_FLAG_BAD_EXPERT;
                    } else {
                        // Only this lane touches bit `lane`, and it walks its
                        // slots in order: the old value says whether the
                        // expert already occurred earlier in the row.
                        const unsigned long long old = atomicOr(&msk[e], bit);
                        if (old & bit) {
                            err |= MOE_FLAG_DUPLICATE;
                        } else {
                            oute = e;
                            p = probs ? probs[at] : 1.f;
                        }
                    }
                }
                row_id[at] = oute;
                copy_prob[at] = p;
            }
        }
    }
    __syncthreads();
    for (int e = lane; e < E; e += 64) tile_mask[(size_t)tile * E + e] = msk[e];
    const unsigned long long bad = __ballot((err & MOE_FLAG_BAD_EXPERT) != 0);
    const unsigned long long dup = __ballot((err & MOE_FLAG_DUPLICATE) != 0);
    if (lane == 0) tile_err[tile] = (bad ? MOE_FLAG_BAD_EXPERT : 0) | (dup ? MOE_FLAG_DUPLICATE : 0);
}

// Boolean map [T,E]: one workgroup of four wavefronts per 64-token tile.
// Wavefront w walks experts [w*Eq, (w+1)*Eq) (Eq = E/4 rounded up to 16) in
// ascending order.  A token's routed experts fill its slots in ascending
// expert order, so wavefront w's first slot for a token is the number of that
// token's routed experts below its range: a scan over the four wavefronts'
// per-token counts.  Slots past K are not written (duplicate bit); the
// wavefront owning the top of the range clears the token's unused slots.
__global__ __launch_bounds__(256) void k_route_tiles_sparse(const uint8_t* __restrict__ routing,
                                                            const float* __restrict__ probs,
                                                            const int32_t* __restrict__ T_live_ptr, int T, int E,
                                                            int K, uint64_t* __restrict__ tile_mask,
                                                            int32_t* __restrict__ tile_err,
                                                            int32_t* __restrict__ row_id,
                                                            float* __restrict__ copy_prob) {
    __shared__ unsigned long long msk[kMaxE];
    __shared__ int cnt[4][kTileTok];
    __shared__ int serr;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int tile = blockIdx.x;
    const int t = tile * kTileTok + lane;
    int T_live = T;
    if (T_live_ptr) T_live = min(max(*T_live_ptr, 0), T);
    const bool in = t < T;
    const bool live = t < T_live;
    const int Eq = ((E + 3) / 4 + 15) / 16 * 16;
    const int eb = min(E, w * Eq), ee = min(E, eb + Eq);
    const uint8_t* row = routing + (size_t)(live ? t : 0) * E;
    const bool vec = (E % 16) == 0;   // then every range is whole 16-byte chunks
    // routed flags of experts e0..e0+15 (byte i of the chunk; 0 past the range)
    auto chunk = [&](int e0) -> u32x4 {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (live) {
            if (vec) {
                v = *(const u32x4*)(row + e0);
            } else {
                uint32_t x[4] = {0u, 0u, 0u, 0u};
                for (int i = 0; i < 16 && e0 + i < ee; ++i) x[i >> 2] |= (uint32_t)(row[e0 + i] != 0) << ((i & 3) * 8);
                v = u32x4{x[0], x[1], x[2], x[3]};
            }
        }
        return v;
    };
    auto routed = [](const u32x4& v, int i) { return ((v[i >> 2] >> ((i & 3) * 8)) & 0xffu) != 0u; };

    int c = 0;
    for (int e0 = eb; e0 < ee; e0 += 16) {
        const u32x4 v = chunk(e0);
#pragma unroll
        for (int i = 0; i < 16; ++i) c += (e0 + i < ee && routed(v, i)) ? 1 : 0;
    }
    cnt[w][lane] = c;
    if (threadIdx.x == 0) serr = 0;
    __syncthreads();
    int j = 0;
    for (int w2 = 0; w2 < w; ++w2) j += cnt[w2][lane];
    int err = 0;
    for (int e0 = eb; e0 < ee; e0 += 16) {
        const u32x4 v = chunk(e0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int e = e0 + i;
            bool sel = false;
            if (e < ee && routed(v, i)) {
                if (j < K) {
                    const size_t at = (size_t)t * K + j;
                    row_id[at] = e;
                    copy_prob[at] = probs ? probs[(size_t)t * E + e] : 1.f;
                    ++j;
                    sel = true;
                } else {
                    err |= MOE_FLAG_DUPLICATE;
                }
            }
            const unsigned long long b = __ballot(sel);
            if (lane == 0 && e < ee) msk[e] = b;
        }
    }
    if (w == 3 && in) {
        for (; j < K; ++j) {
            const size_t at = (size_t)t * K + j;
            row_id[at] = -1;
            copy_prob[at] = 0.f;
        }
    }
    if (err) atomicOr(&serr, err);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) tile_mask[(size_t)tile * E + e] = msk[e];
    if (threadIdx.x == 0) tile_err[tile] = serr;
}

__global__ __launch_bounds__(1024) void k_route_scan(
    const uint64_t* __restrict__ tile_mask, const int32_t* __restrict__ tile_err, int n_tiles, int E,
    int pad, int cap, long long R, int32_t* __restrict__ tile_base, int32_t* __restrict__ counts_out,
    int32_t* __restrict__ kept_out, int64_t* __restrict__ seg_off, int64_t* __restrict__ rows_needed,
    int32_t* __restrict__ flag) {
    __shared__ int part[1024];
    __shared__ long long scan[16];     // wavefront totals of the expert scan
    __shared__ int sflag;
    const int tid = threadIdx.x;
    int S = 1;
    while (S * 2 * E <= 1024) S *= 2;          // S groups of tiles, S*E <= 1024 threads
    const int chunk = (n_tiles + S - 1) / S;
    if (tid == 0) sflag = 0;
    __syncthreads();
    int terr = 0;
    for (int i = tid; i < n_tiles; i += 1024) terr |= tile_err[i];
    if (terr) atomicOr(&sflag, terr);

    const int g = tid / E, e = tid - g * E;
    const bool act = tid < S * E;
    const int t0 = g * chunk, t1 = min(n_tiles, t0 + chunk);
    // tile masks are read eight tiles at a time, so their loads overlap
    constexpr int U = 8;
    int sum = 0;
    if (act) {
        int tl = t0;
        for (; tl + U <= t1; tl += U) {
            unsigned long long m[U];
#pragma unroll
            for (int u = 0; u < U; ++u) m[u] = tile_mask[(size_t)(tl + u) * E + e];
#pragma unroll
            for (int u = 0; u < U; ++u) sum += __popcll(m[u]);
        }
        for (; tl < t1; ++tl) sum += __popcll(tile_mask[(size_t)tl * E + e]);
        part[g * E + e] = sum;
    }
    __syncthreads();
    if (act) {
        int run = 0;
        for (int g2 = 0; g2 < g; ++g2) run += part[g2 * E + e];
        int tl = t0;
        for (; tl + U <= t1; tl += U) {
            unsigned long long m[U];
#pragma unroll
            for (int u = 0; u < U; ++u) m[u] = tile_mask[(size_t)(tl + u) * E + e];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                tile_base[(size_t)(tl + u) * E + e] = run;
                run += __popcll(m[u]);
            }
        }
        for (; tl < t1; ++tl) {
            tile_base[(size_t)tl * E + e] = run;
            run += __popcll(tile_mask[(size_t)tl * E + e]);
        }
    }
    long long padded = 0;
    if (tid < E) {
        int cnt = 0;
        for (int g2 = 0; g2 < S; ++g2) cnt += part[g2 * E + tid];
        int kept = cnt;
        if (cap >= 0 && cnt > cap) {
            kept = cap;
            atomicOr(&sflag, MOE_FLAG_CAPACITY);
        }
        counts_out[tid] = cnt;
        kept_out[tid] = kept;
        padded = ((long long)kept + pad - 1) / pad * pad;
    }
    // inclusive scan over experts: within each wavefront by shuffles, then
    // the wavefront totals (16 of them) in LDS
    const int lane = tid & 63, wv = tid >> 6;
    long long incl = padded;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const long long v = __shfl_up(incl, off);
        if (lane >= off) incl += v;
    }
    if (lane == 63) scan[wv] = incl;
    __syncthreads();
    long long before = 0;
    for (int w2 = 0; w2 < wv; ++w2) before += scan[w2];
    incl += before;
    if (tid < E) seg_off[tid] = incl - padded;
    if (tid == E - 1) {
        seg_off[E] = incl;
        *rows_needed = incl;
        if (incl > R) atomicOr(&sflag, MOE_FLAG_OUT_ROWS);
    }
    __syncthreads();
    if (tid == 0) *flag = sflag;
}

__global__ __launch_bounds__(256) void k_route_assign(
    int n_tile_blocks, int n_fill_blocks, int n_tiles, int T, int E, int K, long long R,
    const uint64_t* __restrict__ tile_mask, const int32_t* __restrict__ tile_base,
    const int32_t* __restrict__ kept, const int64_t* __restrict__ seg_off,
    int32_t* __restrict__ row_id, float* __restrict__ copy_prob, int32_t* __restrict__ src_row,
    float* __restrict__ out_probs) {
    if ((int)blockIdx.x < n_tile_blocks) {
        const int lane = threadIdx.x & 63;
        const int tile = blockIdx.x * 4 + (threadIdx.x >> 6);
        if (tile >= n_tiles) return;
        const int t = tile * kTileTok + lane;
        if (t >= T) return;
        const unsigned long long below = (1ull << lane) - 1ull;
        // slots are taken eight at a time: their expert ids, then all the
        // per-expert lookups, are loaded together so their latencies overlap
        constexpr int U = 8;
        for (int j0 = 0; j0 < K; j0 += U) {
            int e[U], tb[U], kp[U];
            unsigned long long tm[U];
            long long so[U];
#pragma unroll
            for (int u = 0; u < U; ++u) e[u] = j0 + u < K ? row_id[(size_t)t * K + j0 + u] : -1;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (e[u] >= 0) {
                    const size_t te = (size_t)tile * E + e[u];
                    tb[u] = tile_base[te];
                    tm[u] = tile_mask[te];
                    so[u] = seg_off[e[u]];
                    kp[u] = kept[e[u]];
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (e[u] < 0) continue;
                const size_t at = (size_t)t * K + j0 + u;
                const int rank = tb[u] + __popcll(tm[u] & below);
                const long long row = so[u] + rank;
                if (rank < kp[u] && row < R) {
                    row_id[at] = (int)row;
                    src_row[row] = t;
                    if (out_probs) out_probs[row] = copy_prob[at];
                } else {
                    row_id[at] = -1;
                    copy_prob[at] = 0.f;
                }
            }
        }
        return;
    }
    // Rows that hold no copy: padding inside segments, and everything past
    // the last segment.
    __shared__ long long s_off[kMaxE + 1];
    __shared__ int s_kept[kMaxE];
    for (int i = threadIdx.x; i <= E; i += 256) s_off[i] = seg_off[i];
    for (int i = threadIdx.x; i < E; i += 256) s_kept[i] = kept[i];
    __syncthreads();
    const long long stride = (long long)n_fill_blocks * 256;
    for (long long r = (long long)(blockIdx.x - n_tile_blocks) * 256 + threadIdx.x; r < R; r += stride) {
        bool assigned = false;
        if (r < s_off[E]) {
            int lo = 0, hi = E - 1;              // last e with s_off[e] <= r
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (s_off[mid] <= r) lo = mid; else hi = mid - 1;
            }
            assigned = r < s_off[lo] + s_kept[lo];
        }
        if (!assigned) {
            src_row[r] = -1;
            if (out_probs) out_probs[r] = 0.f;
        }
    }
}

// Small batches (at most kSmallTiles tiles, i.e. T <= 256) with dense
// routing: the three steps above in one workgroup of 1024 threads, the tile
// masks and bases in LDS.  Decode batches pay one launch instead of three.
// Wavefront w builds tile w's masks exactly as k_route_tiles does (each
// lane's slots in order, so its ranks and duplicate bits are the same), one
// thread per expert scans the tiles and the experts as k_route_scan does,
// wavefront w assigns tile w's slots as k_route_assign does, and every thread
// takes a share of the rows without a copy.  Integer arithmetic throughout,
// so every output equals the three-launch path's.
constexpr int kSmallTiles = 4;
constexpr long long kSmallRows = 16384;    // rows past this go to the three-launch fill

template <int FMT>
__global__ __launch_bounds__(1024) void k_route_small(const void* __restrict__ routing,
                                                      const float* __restrict__ probs,
                                                      const int32_t* __restrict__ T_live_ptr, int T, int E, int K,
                                                      int pad, int cap, long long R, int n_tiles,
                                                      int32_t* __restrict__ row_id, float* __restrict__ copy_prob,
                                                      int32_t* __restrict__ counts_out,
                                                      int32_t* __restrict__ kept_out, int64_t* __restrict__ seg_off,
                                                      int64_t* __restrict__ rows_needed,
                                                      int32_t* __restrict__ src_row, float* __restrict__ out_probs,
                                                      int32_t* __restrict__ flag) {
    static_assert(FMT != MOE_ROUTE_SPARSE_BOOL, "dense routing only");
    __shared__ unsigned long long msk[kSmallTiles][kMaxE];
    __shared__ int tbase[kSmallTiles][kMaxE];
    __shared__ long long s_off[kMaxE + 1];
    __shared__ int s_kept[kMaxE];
    __shared__ long long scan[16];
    __shared__ int sflag;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int T_live = T;
    if (T_live_ptr) T_live = min(max(*T_live_ptr, 0), T);
    for (int i = tid; i < n_tiles * E; i += 1024) msk[i / E][i % E] = 0ull;
    if (tid == 0) sflag = 0;
    __syncthreads();

    // 1. membership masks of tile wv (lane = token), slot expert ids and probabilities
    const int t = wv * kTileTok + lane;
    const bool mine = wv < n_tiles && t < T;
    int err = 0;
    constexpr int U = 8;                   // slots loaded together, so their latencies overlap
    int keep_e[U];                         // K <= U: the slots stay in registers for step 3
    float keep_p[U];
    if (mine) {
        const bool live = t < T_live;
        const unsigned long long bit = 1ull << lane;
        for (int j0 = 0; j0 < K; j0 += U) {
            int ev[U];
            float pv[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const size_t at = (size_t)t * K + min(j0 + u, K - 1);
                ev[u] = (FMT == MOE_ROUTE_DENSE_I16) ? (int)((const int16_t*)routing)[at]
                                                     : ((const int32_t*)routing)[at];
                pv[u] = probs ? probs[at] : 1.f;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (j0 + u >= K) break;
                const size_t at = (size_t)t * K + j0 + u;
                const int e = ev[u];
                int oute = -1;
                float p = 0.f;
                if (live && e != -1) {
                    if (e < -1 || e >= E) {
                        err |= MOE_FLAG_BAD_EXPERT;
                    } else {
                        // this lane alone sets bit `lane`, walking its slots in
                        // order: the old value says whether e occurred earlier
                        const unsigned long long old = atomicOr(&msk[wv][e], bit);
                        if (old & bit) {
                            err |= MOE_FLAG_DUPLICATE;
                        } else {
                            oute = e;
                            p = pv[u];
                        }
                    }
                }
                if (K <= U) {
                    keep_e[u] = oute;
                    keep_p[u] = p;
                } else {
                    row_id[at] = oute;
                    copy_prob[at] = p;
                }
            }
        }
    }
    if (err) atomicOr(&sflag, err);
    __syncthreads();

    // 2. per expert: tile bases, count, capacity, padding; exclusive scan over experts
    long long padded = 0;
    if (tid < E) {
        int run = 0;
        for (int tl = 0; tl < n_tiles; ++tl) {
            tbase[tl][tid] = run;
            run += __popcll(msk[tl][tid]);
        }
        int kept = run;
        if (cap >= 0 && run > cap) {
            kept = cap;
            atomicOr(&sflag, MOE_FLAG_CAPACITY);
        }
        counts_out[tid] = run;
        kept_out[tid] = kept;
        s_kept[tid] = kept;
        padded = ((long long)kept + pad - 1) / pad * pad;
    }
    long long incl = padded;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const long long v = __shfl_up(incl, off);
        if (lane >= off) incl += v;
    }
    if (lane == 63) scan[wv] = incl;
    __syncthreads();
    long long before = 0;
    for (int w2 = 0; w2 < wv; ++w2) before += scan[w2];
    incl += before;
    if (tid < E) {
        s_off[tid] = incl - padded;
        seg_off[tid] = incl - padded;
    }
    if (tid == E - 1) {
        s_off[E] = incl;
        seg_off[E] = incl;
        *rows_needed = incl;
        if (incl > R) atomicOr(&sflag, MOE_FLAG_OUT_ROWS);
    }
    __syncthreads();

    // 3. final rows of tile wv's slots (each thread takes only its own slots: from
    // registers when K <= U, else re-read)
    if (mine) {
        const unsigned long long below = (1ull << lane) - 1ull;
        for (int j0 = 0; j0 < K; j0 += U) {
            int ev[U];
            float pv[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const size_t at = (size_t)t * K + min(j0 + u, K - 1);
                ev[u] = K <= U ? keep_e[u] : row_id[at];
                pv[u] = K <= U ? keep_p[u] : copy_prob[at];
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (j0 + u >= K) break;
                const int e = ev[u];
                const size_t at = (size_t)t * K + j0 + u;
                if (e < 0) {
                    if (K <= U) {              // step 1 left this slot in registers
                        row_id[at] = -1;
                        copy_prob[at] = 0.f;
                    }
                    continue;
                }
                const int rank = tbase[wv][e] + __popcll(msk[wv][e] & below);
                const long long row = s_off[e] + rank;
                if (rank < s_kept[e] && row < R) {
                    row_id[at] = (int)row;
                    if (K <= U) copy_prob[at] = pv[u];    // step 1 left this slot in registers
                    src_row[row] = t;
                    if (out_probs) out_probs[row] = pv[u];
                } else {
                    row_id[at] = -1;
                    copy_prob[at] = 0.f;
                }
            }
        }
    }
    // 4. rows that hold no copy: each expert's padding (by the thread of that
    // expert), then everything past the last segment
    if (tid < E) {
        const long long end = min(s_off[tid + 1], R);
        for (long long r = s_off[tid] + s_kept[tid]; r < end; ++r) {
            src_row[r] = -1;
            if (out_probs) out_probs[r] = 0.f;
        }
    }
    for (long long r = s_off[E] + tid; r < R; r += 1024) {
        src_row[r] = -1;
        if (out_probs) out_probs[r] = 0.f;
    }
    if (tid == 0) *flag = sflag;
}

}  // namespace

hipError_t launch_route(const moe_handle* h, const void* routing, const float* probs,
                        const int32_t* T_live, int32_t* tokens_per_expert, float* out_probs,
                        int32_t* flag, hipStream_t s) {
    const moe_desc& d = h->desc;
    const int nt = h->n_tiles;
    if (nt <= kSmallTiles && d.out_rows <= kSmallRows && d.route_fmt != MOE_ROUTE_SPARSE_BOOL) {
        if (d.route_fmt == MOE_ROUTE_DENSE_I16)
            hipLaunchKernelGGL(k_route_small<MOE_ROUTE_DENSE_I16>, dim3(1), dim3(1024), 0, s, routing, probs, T_live,
                               d.T, d.E, d.K, d.pad_multiple, d.capacity, (long long)d.out_rows, nt, h->row_id,
                               h->copy_prob, tokens_per_expert, h->kept, h->seg_off, h->rows_needed, h->src_row,
                               out_probs, flag);
        else
            hipLaunchKernelGGL(k_route_small<MOE_ROUTE_DENSE_I32>, dim3(1), dim3(1024), 0, s, routing, probs, T_live,
                               d.T, d.E, d.K, d.pad_multiple, d.capacity, (long long)d.out_rows, nt, h->row_id,
                               h->copy_prob, tokens_per_expert, h->kept, h->seg_off, h->rows_needed, h->src_row,
                               out_probs, flag);
        return hipGetLastError();
    }
    if (nt > 0) {
        switch (d.route_fmt) {
            case MOE_ROUTE_DENSE_I16:
                hipLaunchKernelGGL(k_route_tiles<MOE_ROUTE_DENSE_I16>, dim3(nt), dim3(64), 0, s, routing, probs,
                                   T_live, d.T, d.E, d.K, h->tile_mask, h->tile_err, h->row_id, h->copy_prob);
                break;
            case MOE_ROUTE_DENSE_I32:
                hipLaunchKernelGGL(k_route_tiles<MOE_ROUTE_DENSE_I32>, dim3(nt), dim3(64), 0, s, routing, probs,
                                   T_live, d.T, d.E, d.K, h->tile_mask, h->tile_err, h->row_id, h->copy_prob);
                break;
            default:
                hipLaunchKernelGGL(k_route_tiles_sparse, dim3(nt), dim3(256), 0, s, (const uint8_t*)routing, probs,
                                   T_live, d.T, d.E, d.K, h->tile_mask, h->tile_err, h->row_id, h->copy_prob);
                break;
        }
    }
    hipLaunchKernelGGL(k_route_scan, dim3(1), dim3(1024), 0, s, h->tile_mask, h->tile_err, nt, d.E,
                       d.pad_multiple, d.capacity, (long long)d.out_rows, h->tile_base, tokens_per_expert,
                       h->kept, h->seg_off, h->rows_needed, flag);
    const int n_tile_blocks = (nt + 3) / 4;
    long long fb = (d.out_rows + 255) / 256;
    const int n_fill_blocks = (int)(fb < 1024 ? fb : 1024);
    if (n_tile_blocks + n_fill_blocks > 0)
        hipLaunchKernelGGL(k_route_assign, dim3(n_tile_blocks + n_fill_blocks), dim3(256), 0, s, n_tile_blocks,
                           n_fill_blocks, nt, d.T, d.E, d.K, (long long)d.out_rows, h->tile_mask, h->tile_base,
                           h->kept, h->seg_off, h->row_id, h->copy_prob, h->src_row, out_probs);
    return hipGetLastError();
}

}  // namespace moe
