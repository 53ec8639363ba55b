// extern "C" entry points of libmoe_route (declared in include/moe_route.h):
// host-side validation, workspace carving, stale-handle detection and the
// kernel launches.  Nothing here synchronises with the device or allocates
// device memory.
#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <cmath>
#include <cstring>
#include <mutex>
#include <unordered_map>

#include "moe_internal.h"

using namespace moe;

namespace {

std::mutex g_mu;
std::unordered_map<uintptr_t, uint64_t> g_epoch;   // workspace address -> generation

constexpr size_t kAlign = 256;

size_t up(size_t v, size_t a) { return (v + a - 1) / a * a; }
bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool al4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

int check_desc(const moe_desc* d) {
    if (!d) return MOE_EINVAL;
    if (d->route_fmt < MOE_ROUTE_DENSE_I16 || d->route_fmt > MOE_ROUTE_SPARSE_BOOL) return MOE_EINVAL;
    if (d->payload != MOE_BF16 && d->payload != MOE_FP8E4M3_B128) return MOE_EDTYPE;
    if (d->T < 0 || d->E < 1 || d->E > kMaxE || d->K < 1 || d->K > kMaxE || d->pad_multiple < 1 || d->H < 1)
        return MOE_ESHAPE;
    if (d->payload == MOE_BF16 && d->H % 8) return MOE_ESHAPE;
    if (d->payload == MOE_FP8E4M3_B128 && d->H % 128) return MOE_ESHAPE;
    if ((int64_t)d->T * d->K > INT32_MAX) return MOE_ESHAPE;
    if (d->out_rows < 0 || d->out_rows > INT32_MAX) return MOE_ESHAPE;
    return MOE_OK;
}

int64_t bound_rows(const moe_desc* d) {
    const int64_t p = d->pad_multiple;
    const int64_t by_copies = (int64_t)d->T * d->K + (int64_t)d->E * (p - 1);
    if (d->capacity < 0) return by_copies;
    const int64_t by_cap = ((int64_t)d->capacity + p - 1) / p * p * d->E;
    return by_cap < by_copies ? by_cap : by_copies;
}

struct Layout {
    size_t mask, base, err, seg, kept, rn, rowid, cp, src, total;
    int n_tiles;
    int64_t R;
};

int make_layout(const moe_desc* d, Layout* L) {
    int rc = check_desc(d);
    if (rc) return rc;
    const int64_t R = d->out_rows ? d->out_rows : bound_rows(d);
    if (R > INT32_MAX) return MOE_ESHAPE;
    L->R = R;
    L->n_tiles = (d->T + kTileTok - 1) / kTileTok;
    const size_t nt = (size_t)L->n_tiles, E = (size_t)d->E, TK = (size_t)d->T * d->K;
    size_t o = 0;
    L->mask = o;  o = up(o + nt * E * 8, kAlign);
    L->base = o;  o = up(o + nt * E * 4, kAlign);
    L->err = o;   o = up(o + nt * 4, kAlign);
    L->seg = o;   o = up(o + (E + 1) * 8, kAlign);
    L->kept = o;  o = up(o + E * 4, kAlign);
    L->rn = o;    o = up(o + 8, kAlign);
    L->rowid = o; o = up(o + TK * 4, kAlign);
    L->cp = o;    o = up(o + TK * 4, kAlign);
    L->src = o;   o = up(o + (size_t)R * 4, kAlign);
    L->total = o;
    return MOE_OK;
}

int check_handle(const moe_handle* h, bool need_routing) {
    if (!h) return MOE_EINVAL;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        auto it = g_epoch.find((uintptr_t)h->ws);
        if (it == g_epoch.end() || it->second != h->epoch) return MOE_ESTALE;
    }
    if (need_routing && h->state < 1) return MOE_ESTALE;
    return MOE_OK;
}

// Argument checks of a permute (shared by moe_permute and moe_dispatch, which
// runs them before it enqueues the routing preprocessing).
int check_permute_args(const moe_desc& d, const void* d_x, const float* d_x_scales, const void* d_out,
                       const float* d_out_scales) {
    const bool fp8 = d.payload == MOE_FP8E4M3_B128;
    if (d.T > 0 && (!d_x || !d_out)) return MOE_EINVAL;
    if (fp8 && d.T > 0 && (!d_x_scales || !d_out_scales)) return MOE_EINVAL;
    if (!fp8 && (d_x_scales || d_out_scales)) return MOE_EDTYPE;
    if ((d_x && !al16(d_x)) || (d_out && !al16(d_out))) return MOE_EALIGN;
    if ((d_x_scales && !al4(d_x_scales)) || (d_out_scales && !al4(d_out_scales))) return MOE_EALIGN;
    return MOE_OK;
}

int num_cu() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
    if (dev < 64 && cache[dev] > 0) return cache[dev];
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return -1;
    if (dev < 64) cache[dev] = n;
    return n;
}

int hip_rc(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_EINVAL: return "invalid argument (null pointer or unknown enum)";
        case MOE_ESHAPE: return "shape outside the supported range";
        case MOE_EDTYPE: return "unsupported dtype or format";
        case MOE_EALIGN: return "device pointer not 16-byte aligned";
        case MOE_ESTALE: return "stale handle (workspace re-initialised or no routing metadata)";
        case MOE_EHIP: return "HIP runtime error";
        case MOE_EUNSUPPORTED: return "not supported";
        case MOE_ENOSPC: return "workspace or scratch too small";
        case MOE_EBUSY: return "ring slot still in use (reused before its release)";
        case MOE_ESTATE: return "ring slot not acquired (double release)";
        default: return "unknown status";
    }
}

int64_t moe_out_rows_bound(const moe_desc* desc) {
    if (check_desc(desc)) return -1;
    return bound_rows(desc);
}

int64_t moe_routing_bytes(const moe_desc* desc) {
    if (check_desc(desc)) return -1;
    if (desc->route_fmt == MOE_ROUTE_SPARSE_BOOL) return (int64_t)desc->T * desc->E;
    return (int64_t)desc->T * desc->K * (desc->route_fmt == MOE_ROUTE_DENSE_I16 ? 2 : 4);
}

int64_t moe_capacity_from_rows(int64_t rows, double factor) {
    if (rows < 0 || !(factor > 0.0)) return -1;
    const double c = std::ceil((double)rows * factor);
    if (c > (double)INT64_MAX / 2) return -1;
    const int64_t ci = (int64_t)c;
    return (ci + 3) / 4 * 4;
}

size_t moe_workspace_bytes(const moe_desc* desc) {
    Layout L;
    if (make_layout(desc, &L)) return 0;
    return L.total;
}

int moe_handle_init(const moe_desc* desc, void* d_ws, size_t ws_bytes, moe_handle* h) {
    if (!h) return MOE_EINVAL;
    Layout L;
    int rc = make_layout(desc, &L);
    if (rc) return rc;
    if (!d_ws) return MOE_EINVAL;
    if (!al16(d_ws)) return MOE_EALIGN;
    if (ws_bytes < L.total) return MOE_ENOSPC;
    std::memset(h, 0, sizeof(*h));
    h->desc = *desc;
    h->desc.out_rows = L.R;
    h->n_tiles = L.n_tiles;
    h->ws = d_ws;
    h->ws_bytes = ws_bytes;
    char* b = (char*)d_ws;
    h->tile_mask = (uint64_t*)(b + L.mask);
    h->tile_base = (int32_t*)(b + L.base);
    h->tile_err = (int32_t*)(b + L.err);
    h->seg_off = (int64_t*)(b + L.seg);
    h->kept = (int32_t*)(b + L.kept);
    h->rows_needed = (int64_t*)(b + L.rn);
    h->row_id = (int32_t*)(b + L.rowid);
    h->copy_prob = (float*)(b + L.cp);
    h->src_row = (int32_t*)(b + L.src);
    std::lock_guard<std::mutex> lk(g_mu);
    h->epoch = ++g_epoch[(uintptr_t)d_ws];
    return MOE_OK;
}

int moe_route_preprocess(moe_handle* h, const void* d_routing, const float* d_probs,
                         const int32_t* d_T_live, int32_t* d_tokens_per_expert, float* d_out_probs,
                         int32_t* d_flag, void* stream) {
    int rc = check_handle(h, false);
    if (rc) return rc;
    const moe_desc& d = h->desc;
    if (!d_tokens_per_expert || !d_flag) return MOE_EINVAL;
    if (d.T > 0 && !d_routing) return MOE_EINVAL;
    if (d_routing && !al16(d_routing)) return MOE_EALIGN;
    if ((d_probs && !al4(d_probs)) || (d_out_probs && !al4(d_out_probs)) || !al4(d_tokens_per_expert) ||
        !al4(d_flag) || (d_T_live && !al4(d_T_live)))
        return MOE_EALIGN;
    rc = hip_rc(launch_route(h, d_routing, d_probs, d_T_live, d_tokens_per_expert, d_out_probs, d_flag,
                             (hipStream_t)stream));
    if (rc == MOE_OK) h->state = 1;
    return rc;
}

int moe_permute(const moe_handle* h, const void* d_x, const float* d_x_scales, void* d_out,
                float* d_out_scales, void* stream) {
    int rc = check_handle(h, true);
    if (rc) return rc;
    rc = check_permute_args(h->desc, d_x, d_x_scales, d_out, d_out_scales);
    if (rc) return rc;
    return hip_rc(launch_permute(h, d_x, d_x_scales, d_out, d_out_scales, (hipStream_t)stream));
}

int moe_permute_quantize(const moe_handle* h, const void* d_x, void* d_out, float* d_out_scales, void* stream) {
    int rc = check_handle(h, true);
    if (rc) return rc;
    const moe_desc& d = h->desc;
    if (d.payload != MOE_FP8E4M3_B128) return MOE_EDTYPE;
    if (d.T > 0 && (!d_x || !d_out || !d_out_scales)) return MOE_EINVAL;
    if ((d_x && !al16(d_x)) || (d_out && !al16(d_out))) return MOE_EALIGN;
    if (d_out_scales && !al4(d_out_scales)) return MOE_EALIGN;
    return hip_rc(launch_permute_quant(h, d_x, d_out, d_out_scales, (hipStream_t)stream));
}

int moe_dispatch(moe_handle* h, const void* d_routing, const float* d_probs, const int32_t* d_T_live,
                 const void* d_x, const float* d_x_scales, void* d_out, float* d_out_scales,
                 float* d_out_probs, int32_t* d_tokens_per_expert, int32_t* d_flag, void* stream) {
    int rc = check_handle(h, false);
    if (rc) return rc;
    // every argument check of the permute half runs before anything is
    // enqueued, so a rejected call leaves the handle and outputs untouched
    rc = check_permute_args(h->desc, d_x, d_x_scales, d_out, d_out_scales);
    if (rc) return rc;
    rc = moe_route_preprocess(h, d_routing, d_probs, d_T_live, d_tokens_per_expert, d_out_probs, d_flag, stream);
    if (rc) return rc;
    return moe_permute(h, d_x, d_x_scales, d_out, d_out_scales, stream);
}

size_t moe_mlp_scratch_bytes(const moe_handle* h, int32_t F, int32_t wdtype) {
    if (!h || F <= 0) return 0;
    const size_t R = (size_t)h->desc.out_rows;
    if (wdtype == MOE_BF16) return up(R * (size_t)F * 2, kAlign);
    if (wdtype == MOE_FP8E4M3_B128) {
        if (F % 128 || h->desc.H % 128) return 0;
        return up(fp8_mlp_scratch_bytes((long long)R, h->desc.H, F), kAlign);
    }
    return 0;
}

namespace {

// Host-side checks of one weight tensor of the MLP (no device access).
int check_mlp_weights(const moe_handle* h, int32_t F, int32_t wdtype, const void* w, const float* w_scales) {
    int rc = check_handle(h, true);
    if (rc) return rc;
    const moe_desc& d = h->desc;
    if (F <= 0) return MOE_ESHAPE;
    if (d.payload != MOE_BF16 && wdtype != MOE_FP8E4M3_B128) return MOE_EDTYPE;
    if (!w) return MOE_EINVAL;
    if (!al16(w)) return MOE_EALIGN;
    if (moe_mlp_scratch_bytes(h, F, wdtype) == 0) return MOE_ESHAPE;
    if (wdtype == MOE_BF16) {
        if (w_scales) return MOE_EDTYPE;
        if (d.H % 256 || F % 128) return MOE_ESHAPE;
    } else if (wdtype == MOE_FP8E4M3_B128) {
        if (!w_scales) return MOE_EINVAL;
        if (!al4(w_scales)) return MOE_EALIGN;
        if (d.H % 128 || F % 128) return MOE_ESHAPE;
    } else {
        return MOE_EDTYPE;
    }
    return MOE_OK;
}

// Checks shared by the MLP entry points; *ncu receives the CU count.
int check_mlp(const moe_handle* h, int32_t F, int32_t wdtype, const void* w, const float* w_scales,
              const void* scratch, size_t scratch_bytes, int* ncu) {
    int rc = check_mlp_weights(h, F, wdtype, w, w_scales);
    if (rc) return rc;
    if (!scratch) return MOE_EINVAL;
    if (!al16(scratch)) return MOE_EALIGN;
    if (scratch_bytes < moe_mlp_scratch_bytes(h, F, wdtype)) return MOE_ENOSPC;
    *ncu = num_cu();
    return *ncu > 0 ? MOE_OK : MOE_EHIP;
}

// Host checks of the permuted rows FC1 reads.
int check_perm(const moe_handle* h, const void* d_perm, const float* d_perm_scales) {
    // fp8 permuted rows (quantised on dispatch) carry their scales; bf16 rows none
    const bool fp8_rows = h->desc.payload == MOE_FP8E4M3_B128;
    if (fp8_rows != (d_perm_scales != nullptr)) return fp8_rows ? MOE_EINVAL : MOE_EDTYPE;
    if (!d_perm) return MOE_EINVAL;
    if (!al16(d_perm) || (d_perm_scales && !al4(d_perm_scales))) return MOE_EALIGN;
    return MOE_OK;
}

}  // namespace

}  // extern "C"

namespace moe {

int check_mlp_host(const moe_handle* h, int32_t F, int32_t wdtype, const void* d_perm, const float* d_perm_scales,
                   const void* d_w1, const float* d_w1_scales, const void* d_w2, const float* d_w2_scales,
                   const void* d_expert_out) {
    int rc = check_mlp_weights(h, F, wdtype, d_w2, d_w2_scales);
    if (rc) return rc;
    rc = check_mlp_weights(h, F, wdtype, d_w1, d_w1_scales);
    if (rc) return rc;
    rc = check_perm(h, d_perm, d_perm_scales);
    if (rc) return rc;
    if (!d_expert_out) return MOE_EINVAL;
    return al16(d_expert_out) ? MOE_OK : MOE_EALIGN;
}

}  // namespace moe

extern "C" {

int moe_grouped_fc1_swiglu(const moe_handle* h, int32_t F, int32_t wdtype, const void* d_perm,
                           const float* d_perm_scales, const void* d_w1, const float* d_w1_scales,
                           void* d_scratch, size_t scratch_bytes, void* stream) {
    int ncu = 0;
    int rc = check_mlp(h, F, wdtype, d_w1, d_w1_scales, d_scratch, scratch_bytes, &ncu);
    if (rc) return rc;
    rc = check_perm(h, d_perm, d_perm_scales);
    if (rc) return rc;
    if (wdtype == MOE_FP8E4M3_B128)
        return hip_rc(launch_gemm_fp8(h, 0, F, d_perm, d_perm_scales, d_w1, d_w1_scales, d_scratch, nullptr,
                                      (hipStream_t)stream));
    return hip_rc(launch_gemm_bf16(h, 0, F, d_perm, d_w1, d_scratch, nullptr, ncu, (hipStream_t)stream));
}

int moe_grouped_fc2(const moe_handle* h, int32_t F, int32_t wdtype, const void* d_w2,
                    const float* d_w2_scales, void* d_scratch, size_t scratch_bytes,
                    void* d_expert_out, void* stream) {
    int ncu = 0;
    int rc = check_mlp(h, F, wdtype, d_w2, d_w2_scales, d_scratch, scratch_bytes, &ncu);
    if (rc) return rc;
    if (!d_expert_out) return MOE_EINVAL;
    if (!al16(d_expert_out)) return MOE_EALIGN;
    if (wdtype == MOE_FP8E4M3_B128)
        return hip_rc(launch_gemm_fp8(h, 1, F, nullptr, nullptr, d_w2, d_w2_scales, d_scratch, d_expert_out,
                                      (hipStream_t)stream));
    return hip_rc(launch_gemm_bf16(h, 1, F, d_scratch, d_w2, d_expert_out, nullptr, ncu, (hipStream_t)stream));
}

int moe_grouped_fc2_fp8out(const moe_handle* h, int32_t F, int32_t wdtype, const void* d_w2,
                           const float* d_w2_scales, void* d_scratch, size_t scratch_bytes, void* d_out_q,
                           float* d_out_scales, void* stream) {
    int ncu = 0;
    int rc = check_mlp(h, F, wdtype, d_w2, d_w2_scales, d_scratch, scratch_bytes, &ncu);
    if (rc) return rc;
    if (wdtype != MOE_BF16) return MOE_EUNSUPPORTED;
    if (!d_out_q || !d_out_scales) return MOE_EINVAL;
    if (!al16(d_out_q) || !al4(d_out_scales)) return MOE_EALIGN;
    return hip_rc(launch_gemm_bf16(h, 1, F, d_scratch, d_w2, d_out_q, d_out_scales, ncu, (hipStream_t)stream));
}

int moe_grouped_swiglu_mlp(const moe_handle* h, int32_t F, int32_t wdtype, const void* d_perm,
                           const float* d_perm_scales, const void* d_w1, const float* d_w1_scales,
                           const void* d_w2, const float* d_w2_scales, void* d_scratch,
                           size_t scratch_bytes, void* d_expert_out, void* stream) {
    int ncu = 0;
    int rc = check_mlp(h, F, wdtype, d_w2, d_w2_scales, d_scratch, scratch_bytes, &ncu);
    if (rc) return rc;
    // every host check of both halves runs before FC1 is enqueued
    rc = check_mlp_host(h, F, wdtype, d_perm, d_perm_scales, d_w1, d_w1_scales, d_w2, d_w2_scales, d_expert_out);
    if (rc) return rc;
    rc = moe_grouped_fc1_swiglu(h, F, wdtype, d_perm, d_perm_scales, d_w1, d_w1_scales, d_scratch,
                                scratch_bytes, stream);
    if (rc) return rc;
    return moe_grouped_fc2(h, F, wdtype, d_w2, d_w2_scales, d_scratch, scratch_bytes, d_expert_out, stream);
}

// bound of every wait of the persistent decode kernel (100 MHz ticks)
constexpr long long kDecodeWaitTicksDefault = 25000000;   // 0.25 s
static std::atomic<long long> g_decode_wait_ticks{kDecodeWaitTicksDefault};

void moe_decode_layer_set_wait_bound(int64_t ticks) {
    g_decode_wait_ticks.store(ticks > 0 ? (long long)ticks : kDecodeWaitTicksDefault);
}

size_t moe_decode_layer_scratch_bytes(const moe_handle* h, int32_t F) {
    if (!h || F <= 0 || F % 128 || h->desc.H % 128) return 0;
    return up(decode_layer_scratch_bytes((long long)h->desc.out_rows, h->desc.H, F), kAlign);
}

int moe_decode_layer_fp8(const moe_handle* h, int32_t F, const void* d_x, const void* d_w1, const float* d_w1_scales,
                         const void* d_w2, const float* d_w2_scales, void* d_scratch, size_t scratch_bytes,
                         void* d_expert_out, int32_t apply_probs, void* d_y, int32_t* d_status, void* stream) {
    int rc = check_handle(h, true);
    if (rc) return rc;
    const moe_desc& d = h->desc;
    if (d.payload != MOE_BF16) return MOE_EDTYPE;             // token rows are bf16, quantised here
    if (F <= 0 || F % 128 || d.H % 128) return MOE_ESHAPE;
    if (!d_w1 || !d_w1_scales || !d_w2 || !d_w2_scales || !d_scratch || !d_status) return MOE_EINVAL;
    if (d.T > 0 && (!d_x || !d_expert_out || !d_y)) return MOE_EINVAL;
    if (!al16(d_w1) || !al16(d_w2) || !al4(d_w1_scales) || !al4(d_w2_scales) || !al16(d_scratch) ||
        !al4(d_status))
        return MOE_EALIGN;
    if ((d_x && !al16(d_x)) || (d_expert_out && !al16(d_expert_out)) || (d_y && !al16(d_y))) return MOE_EALIGN;
    if (scratch_bytes < moe_decode_layer_scratch_bytes(h, F)) return MOE_ENOSPC;
    const int ncu = num_cu();
    if (ncu <= 0) return MOE_EHIP;
    return hip_rc(launch_decode_layer(h, F, d_x, d_w1, d_w1_scales, d_w2, d_w2_scales, d_scratch, d_expert_out,
                                      apply_probs ? 1 : 0, d_y, d_status, g_decode_wait_ticks.load(), ncu,
                                      (hipStream_t)stream));
}

size_t moe_decode_fused_scratch_bytes(const moe_handle* h, int32_t F) {
    if (!h || F <= 0 || !decode_fused_shape_ok(h->desc.H, F)) return 0;
    const moe_desc& d = h->desc;
    return up(decode_fused_scratch_bytes((long long)d.out_rows, d.T, d.K, d.H, F, d.E), kAlign);
}

int moe_decode_fused_fp8(const moe_handle* h, int32_t F, const void* d_x, const void* d_w1, const float* d_w1_scales,
                         const void* d_w2, const float* d_w2_scales, void* d_scratch, size_t scratch_bytes,
                         void* d_expert_out, int32_t apply_probs, void* d_y, void* stream) {
    int rc = check_handle(h, true);
    if (rc) return rc;
    const moe_desc& d = h->desc;
    if (d.payload != MOE_BF16) return MOE_EDTYPE;             // token rows are bf16, quantised here
    if (F <= 0 || !decode_fused_shape_ok(d.H, F)) return MOE_ESHAPE;
    if (!d_w1 || !d_w1_scales || !d_w2 || !d_w2_scales || !d_scratch) return MOE_EINVAL;
    if (d.T > 0 && (!d_x || !d_expert_out || !d_y)) return MOE_EINVAL;
    if (!al16(d_w1) || !al16(d_w2) || !al4(d_w1_scales) || !al4(d_w2_scales) || !al16(d_scratch))
        return MOE_EALIGN;
    if ((d_x && !al16(d_x)) || (d_expert_out && !al16(d_expert_out)) || (d_y && !al16(d_y))) return MOE_EALIGN;
    if (scratch_bytes < moe_decode_fused_scratch_bytes(h, F)) return MOE_ENOSPC;
    const int ncu = num_cu();
    if (ncu <= 0) return MOE_EHIP;
    return hip_rc(launch_decode_fused(h, F, d_x, d_w1, d_w1_scales, d_w2, d_w2_scales, d_scratch, d_expert_out,
                                      apply_probs ? 1 : 0, d_y, ncu, (hipStream_t)stream));
}

int moe_combine(const moe_handle* h, const void* d_expert_out, int32_t apply_probs, void* d_y,
                void* stream) {
    int rc = check_handle(h, true);
    if (rc) return rc;
    const moe_desc& d = h->desc;
    if (d.T > 0 && (!d_expert_out || !d_y)) return MOE_EINVAL;
    if ((d_expert_out && !al16(d_expert_out)) || (d_y && !al16(d_y))) return MOE_EALIGN;
    if (d.H % 8) return MOE_ESHAPE;
    return hip_rc(launch_combine(h, d_expert_out, apply_probs ? 1 : 0, d_y, (hipStream_t)stream));
}

int moe_combine_fp8(const moe_handle* h, const void* d_expert_out_q, const float* d_expert_out_scales,
                    int32_t apply_probs, void* d_y, void* stream) {
    int rc = check_handle(h, true);
    if (rc) return rc;
    const moe_desc& d = h->desc;
    if (d.H % 128) return MOE_ESHAPE;
    if (d.T > 0 && (!d_expert_out_q || !d_expert_out_scales || !d_y)) return MOE_EINVAL;
    if ((d_expert_out_q && !al16(d_expert_out_q)) || (d_y && !al16(d_y))) return MOE_EALIGN;
    if (d_expert_out_scales && !al4(d_expert_out_scales)) return MOE_EALIGN;
    return hip_rc(launch_combine_fp8(h, d_expert_out_q, d_expert_out_scales, apply_probs ? 1 : 0, d_y,
                                     (hipStream_t)stream));
}

int moe_dispatch_backward(const moe_handle* h, const void* d_grad_out, const float* d_grad_out_probs,
                          void* d_grad_x, float* d_grad_probs, void* stream) {
    int rc = check_handle(h, true);
    if (rc) return rc;
    const moe_desc& d = h->desc;
    if (d.T > 0 && (!d_grad_out || !d_grad_x)) return MOE_EINVAL;
    if (d_grad_probs && !d_grad_out_probs) return MOE_EINVAL;
    if ((d_grad_out && !al16(d_grad_out)) || (d_grad_x && !al16(d_grad_x))) return MOE_EALIGN;
    if ((d_grad_out_probs && !al4(d_grad_out_probs)) || (d_grad_probs && !al4(d_grad_probs))) return MOE_EALIGN;
    if (d.H % 8) return MOE_ESHAPE;
    rc = hip_rc(launch_combine(h, d_grad_out, 0, d_grad_x, (hipStream_t)stream));
    if (rc || !d_grad_probs) return rc;
    return hip_rc(launch_probs_gather(h, d_grad_out_probs, d_grad_probs, (hipStream_t)stream));
}

int moe_combine_backward(const moe_handle* h, const void* d_grad_y, const void* d_expert_out,
                         int32_t apply_probs, void* d_grad_expert_out, float* d_grad_probs, void* stream) {
    int rc = check_handle(h, true);
    if (rc) return rc;
    const moe_desc& d = h->desc;
    if (d.T > 0 && (!d_grad_y || !d_grad_expert_out)) return MOE_EINVAL;
    if (d.T > 0 && d_grad_probs && apply_probs && !d_expert_out) return MOE_EINVAL;
    if ((d_grad_y && !al16(d_grad_y)) || (d_expert_out && !al16(d_expert_out)) ||
        (d_grad_expert_out && !al16(d_grad_expert_out)))
        return MOE_EALIGN;
    if (d_grad_probs && !al4(d_grad_probs)) return MOE_EALIGN;
    if (d.H % 8) return MOE_ESHAPE;
    return hip_rc(launch_combine_backward(h, d_grad_y, d_expert_out, apply_probs ? 1 : 0, d_grad_expert_out,
                                          d_grad_probs, (hipStream_t)stream));
}

}  // extern "C"
