// Caller-owned buffer ring (extern "C", declared in include/moe_route.h).
//
// Operation: Megatron-LM PR #6800 "Reuse caller-owned HybridEP dispatch and
// expert output buffers" (sections "Summary", "Motivation", "Known
// limitations"): dispatch outputs and FC2 outputs live in a fixed ring of
// persistent slots owned by the application; the final consumer of a slot
// records a release event on its own stream, and the next producer of that
// slot waits for that event on the device, so no host or stream-wide
// synchronisation is needed and the storage stays bounded.  Reuse before the
// release and a second release both fail explicitly.
//
// Host logic only: the slots are carved from the caller's device buffer; the
// only HIP calls are event create / record / stream-wait / destroy.  Events
// are created lazily at a slot's first release, so a ring can be set up on a
// host without a device.
//
// Graph capture: a release recorded while its stream is being captured
// belongs to that capture; an acquire inside the same capture waits on it
// (a join inside the graph), an acquire outside it does not (graph replays
// are ordered by their stream).  A release recorded outside a capture is not
// waited on inside one: the capture starts after the caller's
// synchronisation, so the eager warm-up has finished by then.
#include <hip/hip_runtime.h>

#include <cstring>

#include "moe_route.h"

namespace {

enum : int32_t { kFree = 0, kAcquired = 1 };
enum : int32_t { kNoEvent = 0, kEagerEvent = 1, kCapturedEvent = 2 };

bool capture_id(hipStream_t s, unsigned long long* id) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    unsigned long long cid = 0;
    if (hipStreamGetCaptureInfo(s, &st, &cid) != hipSuccess) return false;
    if (st != hipStreamCaptureStatusActive) return false;
    *id = cid;
    return true;
}

}  // namespace

extern "C" {

int moe_ring_init(moe_ring* r, void* d_base, size_t slot_bytes, int32_t n_slots) {
    if (!r || !d_base) return MOE_EINVAL;
    if (n_slots < 1 || n_slots > MOE_RING_MAX_SLOTS || slot_bytes == 0 || slot_bytes % 256) return MOE_ESHAPE;
    if ((uintptr_t)d_base % 256) return MOE_EALIGN;
    std::memset(r, 0, sizeof(*r));
    r->base = d_base;
    r->slot_bytes = slot_bytes;
    r->n_slots = n_slots;
    return MOE_OK;
}

int moe_ring_acquire(moe_ring* r, void* stream, void** d_slot, int32_t* slot) {
    if (!r || !d_slot || !slot || r->n_slots < 1) return MOE_EINVAL;
    const int32_t s = r->next;
    if (r->state[s] != kFree) return MOE_EBUSY;    // early reuse: the last use was never released
    hipStream_t st = (hipStream_t)stream;
    if (r->event_kind[s] != kNoEvent) {   // the slot was released before: join its final consumer
        unsigned long long cid = 0;
        const bool capturing = capture_id(st, &cid);
        const bool wait = r->event_kind[s] == kEagerEvent ? !capturing : (capturing && r->event_capture[s] == cid);
        if (wait && hipStreamWaitEvent(st, (hipEvent_t)r->event[s], 0) != hipSuccess) return MOE_EHIP;
    }
    r->state[s] = kAcquired;
    r->next = (s + 1) % r->n_slots;
    r->acquisitions++;
    *slot = s;
    *d_slot = (char*)r->base + (size_t)s * r->slot_bytes;
    return MOE_OK;
}

int moe_ring_release(moe_ring* r, int32_t slot, void* stream) {
    if (!r || slot < 0 || slot >= r->n_slots) return MOE_EINVAL;
    if (r->state[slot] != kAcquired) return MOE_ESTATE;   // double release, or never acquired
    if (!r->event[slot]) {
        hipEvent_t e = nullptr;
        if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) return MOE_EHIP;
        r->event[slot] = e;
    }
    hipStream_t st = (hipStream_t)stream;
    unsigned long long cid = 0;
    const bool capturing = capture_id(st, &cid);
    if (hipEventRecord((hipEvent_t)r->event[slot], st) != hipSuccess) return MOE_EHIP;
    r->event_kind[slot] = capturing ? kCapturedEvent : kEagerEvent;
    r->event_capture[slot] = capturing ? cid : 0;
    r->state[slot] = kFree;
    return MOE_OK;
}

int moe_ring_destroy(moe_ring* r) {
    if (!r) return MOE_EINVAL;
    int rc = MOE_OK;
    for (int32_t s = 0; s < MOE_RING_MAX_SLOTS; ++s)
        if (r->event[s]) {
            if (hipEventDestroy((hipEvent_t)r->event[s]) != hipSuccess) rc = MOE_EHIP;
            r->event[s] = nullptr;
        }
    r->n_slots = 0;
    return rc;
}

}  // extern "C"
