"""The C-ABI library loads, exports every symbol include/moe_route.h
declares, and its host-only logic (validation, sizing, workspace carving,
stale-handle detection, page-pinned helpers) behaves as documented.  No call
here reaches the GPU: every device call below is rejected by host checks."""
import ctypes as C
import json
import os
import re

import numpy as np
import pytest

import oracle
from combine_routing_preprocess_amd import _abi as A
from combine_routing_preprocess_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_route.h")
GOLD = json.load(open(os.path.join(ROOT, "tests", "golden", "page_values.json")))


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(moe_[a-z_0-9]+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 12, names
    L = A.lib()
    for n in names:
        assert hasattr(L, n), n
    assert sorted(n for n, _, _ in A.SIGNATURES) == names


def _desc(**kw):
    base = dict(T=100, H=256, E=8, K=2, route_fmt="dense_i16", payload="bf16", pad_multiple=4, capacity=None,
                out_rows=0)
    base.update(kw)
    return api.make_desc(**base)


def test_status_strings():
    for s in range(-8, 1):
        assert A.status_string(s)


def test_out_rows_bound_is_safe_and_reached():
    L = A.lib()
    r = np.random.default_rng(0)
    for _ in range(100):
        T, E = int(r.integers(0, 50)), int(r.integers(1, 9))
        K, pad, cap = int(r.integers(1, E + 1)), int(r.integers(1, 6)), int(r.integers(-1, 10))
        d = api.make_desc(T, 64, E, K, pad_multiple=pad, capacity=None if cap < 0 else cap)
        bound = L.moe_out_rows_bound(C.byref(d))
        idx = np.argsort(r.random((T, E)), axis=1)[:, :K].astype(np.int16)
        rt = oracle.route(idx, 0, E, K, pad=pad, cap=cap, R=10 ** 6)
        assert rt["rows_needed"] <= bound
    # reached: one token per expert with a large padding multiple, no capacity
    d = api.make_desc(4, 64, 4, 1, pad_multiple=8)
    assert L.moe_out_rows_bound(C.byref(d)) == 4 + 4 * 7
    rt = oracle.route(np.arange(4, dtype=np.int16).reshape(4, 1), 0, 4, 1, pad=8, R=100)
    assert rt["rows_needed"] == 32
    # reached through the capacity term: every expert full
    d = api.make_desc(8, 64, 2, 2, pad_multiple=3, capacity=4)
    assert L.moe_out_rows_bound(C.byref(d)) == 2 * 6


def test_page_value_helpers():
    g = GOLD["routing_bytes"]
    tok = g["tokens_per_rank"] * g["world_size"]
    assert api.routing_bytes(tok, g["experts"], g["topk"], "sparse_bool") == g["sparse_bool_bytes_per_rank"]
    assert api.routing_bytes(tok, g["experts"], g["topk"], "dense_i16") == g["dense_int16_bytes_per_rank"]
    c = GOLD["capacity_calibration"]
    assert api.capacity_from_rows(c["rows"], c["factor"]) == c["capacity"]
    assert api.capacity_from_rows(10, 1.5) == 16
    assert api.capacity_from_rows(-1, 1.5) == -1


@pytest.mark.parametrize("kw,status", [
    (dict(E=0), A.MOE_ESHAPE), (dict(E=1025), A.MOE_ESHAPE), (dict(K=0), A.MOE_ESHAPE),
    (dict(T=-1), A.MOE_ESHAPE), (dict(pad_multiple=0), A.MOE_ESHAPE), (dict(H=12), A.MOE_ESHAPE),
    (dict(payload="fp8", H=192), A.MOE_ESHAPE), (dict(out_rows=-5), A.MOE_ESHAPE),
    (dict(out_rows=2 ** 31), A.MOE_ESHAPE),
])
def test_invalid_descriptors_are_rejected(kw, status):
    d = _desc(**kw)
    L = A.lib()
    assert L.moe_workspace_bytes(C.byref(d)) == 0
    buf = (C.c_uint8 * 4096)()
    h = A.MoeHandle()
    assert L.moe_handle_init(C.byref(d), C.cast(buf, C.c_void_p), 4096, C.byref(h)) == status


def test_bad_enum_and_null():
    L = A.lib()
    d = _desc()
    d.route_fmt = 7
    h = A.MoeHandle()
    assert L.moe_handle_init(C.byref(d), C.c_void_p(256), 1 << 20, C.byref(h)) == A.MOE_EINVAL
    d = _desc()
    d.payload = 9
    assert L.moe_handle_init(C.byref(d), C.c_void_p(256), 1 << 20, C.byref(h)) == A.MOE_EDTYPE
    d = _desc()
    assert L.moe_handle_init(C.byref(d), None, 1 << 20, C.byref(h)) == A.MOE_EINVAL
    assert L.moe_handle_init(C.byref(d), C.c_void_p(264), 1 << 20, C.byref(h)) == A.MOE_EALIGN


def _host_handle(desc, extra=0):
    """Initialise a handle over a host buffer: moe_handle_init only carves
    addresses, it never dereferences the workspace."""
    L = A.lib()
    n = L.moe_workspace_bytes(C.byref(desc))
    buf = (C.c_uint8 * (n + 256 + extra))()
    base = (C.addressof(buf) + 255) // 256 * 256
    h = A.MoeHandle()
    rc = L.moe_handle_init(C.byref(desc), C.c_void_p(base), n, C.byref(h))
    return rc, h, base, n, buf


def test_workspace_carving():
    d = _desc(T=1000, E=32, K=8, pad_multiple=16, capacity=300)
    rc, h, base, n, _buf = _host_handle(d)
    assert rc == 0
    R = h.desc.out_rows
    assert R == min(32 * 304, 1000 * 8 + 32 * 15)
    assert h.n_tiles == (1000 + 63) // 64
    fields = [("tile_mask", h.n_tiles * 32 * 8), ("tile_base", h.n_tiles * 32 * 4), ("tile_err", h.n_tiles * 4),
              ("seg_off", 33 * 8), ("kept", 32 * 4), ("rows_needed", 8), ("row_id", 8000 * 4),
              ("copy_prob", 8000 * 4), ("src_row", R * 4)]
    spans = sorted((getattr(h, f) - base, sz) for f, sz in fields)
    for (o1, s1), (o2, _) in zip(spans, spans[1:]):
        assert o1 + s1 <= o2                      # no overlap
    assert all(o % 256 == 0 for o, _ in spans)
    assert spans[-1][0] + spans[-1][1] <= n
    # too small a workspace
    L = A.lib()
    h2 = A.MoeHandle()
    assert L.moe_handle_init(C.byref(d), C.c_void_p(base), n - 1, C.byref(h2)) == A.MOE_ENOSPC


def test_stale_handle_and_missing_routing_are_rejected_before_launch():
    L = A.lib()
    d = _desc()
    rc, h1, base, n, _buf = _host_handle(d)
    assert rc == 0
    # no routing metadata yet: permute / MLP / combine refuse
    x = C.c_void_p(base)
    assert L.moe_permute(C.byref(h1), x, None, x, None, None) == A.MOE_ESTALE
    assert L.moe_combine(C.byref(h1), x, 1, x, None) == A.MOE_ESTALE
    assert L.moe_grouped_swiglu_mlp(C.byref(h1), 128, 0, x, None, x, None, x, None, x, 1 << 30, x, None) == A.MOE_ESTALE
    # re-initialising the workspace makes the first handle stale
    h2 = A.MoeHandle()
    assert L.moe_handle_init(C.byref(d), C.c_void_p(base), n, C.byref(h2)) == 0
    assert h2.epoch == h1.epoch + 1
    assert L.moe_route_preprocess(C.byref(h1), x, None, None, x, None, x, None) == A.MOE_ESTALE
    # null required pointers
    assert L.moe_route_preprocess(C.byref(h2), None, None, None, x, None, x, None) == A.MOE_EINVAL
    assert L.moe_route_preprocess(C.byref(h2), x, None, None, None, None, x, None) == A.MOE_EINVAL
    # misaligned routing
    assert L.moe_route_preprocess(C.byref(h2), C.c_void_p(base + 2), None, None, x, None, x, None) == A.MOE_EALIGN


def test_backward_argument_checks_before_launch():
    L = A.lib()
    rc, h, base, n, _buf = _host_handle(_desc())
    assert rc == 0
    x = C.c_void_p(base)
    # no routing metadata yet
    assert L.moe_dispatch_backward(C.byref(h), x, None, x, None, None) == A.MOE_ESTALE
    assert L.moe_combine_backward(C.byref(h), x, x, 1, x, None, None) == A.MOE_ESTALE
    h.state = 1   # as if routing had been enqueued; every case below fails its checks first
    assert L.moe_dispatch_backward(C.byref(h), None, None, x, None, None) == A.MOE_EINVAL
    assert L.moe_dispatch_backward(C.byref(h), x, None, None, None, None) == A.MOE_EINVAL
    assert L.moe_dispatch_backward(C.byref(h), x, None, x, x, None) == A.MOE_EINVAL      # grad_probs needs row grads
    assert L.moe_dispatch_backward(C.byref(h), C.c_void_p(base + 8), None, x, None, None) == A.MOE_EALIGN
    assert L.moe_dispatch_backward(C.byref(h), x, C.c_void_p(base + 2), x, x, None) == A.MOE_EALIGN
    assert L.moe_combine_backward(C.byref(h), None, x, 1, x, None, None) == A.MOE_EINVAL
    assert L.moe_combine_backward(C.byref(h), x, x, 1, None, None, None) == A.MOE_EINVAL
    assert L.moe_combine_backward(C.byref(h), x, None, 1, x, x, None) == A.MOE_EINVAL    # dot needs expert_out
    assert L.moe_combine_backward(C.byref(h), x, x, 1, C.c_void_p(base + 4), None, None) == A.MOE_EALIGN
    assert L.moe_combine_backward(C.byref(h), x, x, 1, x, C.c_void_p(base + 1), None) == A.MOE_EALIGN


def test_ring_rotation_and_explicit_failures_on_the_host():
    """Ring bookkeeping before any event exists touches no device: init
    validation, rotation over the caller's slots, early reuse (MOE_EBUSY) and
    release of a slot that is not acquired (MOE_ESTATE)."""
    L = A.lib()
    r = A.MoeRing()
    base = 1 << 40                                  # never dereferenced
    assert L.moe_ring_init(C.byref(r), None, 256, 2) == A.MOE_EINVAL
    assert L.moe_ring_init(C.byref(r), C.c_void_p(base), 256, 0) == A.MOE_ESHAPE
    assert L.moe_ring_init(C.byref(r), C.c_void_p(base), 256, A.RING_MAX_SLOTS + 1) == A.MOE_ESHAPE
    assert L.moe_ring_init(C.byref(r), C.c_void_p(base), 100, 2) == A.MOE_ESHAPE
    assert L.moe_ring_init(C.byref(r), C.c_void_p(base + 16), 256, 2) == A.MOE_EALIGN
    assert L.moe_ring_init(C.byref(r), C.c_void_p(base), 4096, 3) == 0
    assert L.moe_ring_release(C.byref(r), 0, None) == A.MOE_ESTATE      # never acquired
    assert L.moe_ring_release(C.byref(r), 3, None) == A.MOE_EINVAL
    got = []
    for _ in range(3):
        p, i = C.c_void_p(), C.c_int32()
        assert L.moe_ring_acquire(C.byref(r), None, C.byref(p), C.byref(i)) == 0
        got.append((i.value, p.value))
    assert got == [(0, base), (1, base + 4096), (2, base + 8192)]
    p, i = C.c_void_p(), C.c_int32()
    assert L.moe_ring_acquire(C.byref(r), None, C.byref(p), C.byref(i)) == A.MOE_EBUSY   # slot 0 in use
    assert r.acquisitions == 3
    assert L.moe_ring_destroy(C.byref(r)) == 0


def test_scratch_sizing():
    d = _desc(T=64, E=4, K=2, pad_multiple=1)
    rc, h, base, n, _buf = _host_handle(d)
    L = A.lib()
    R = h.desc.out_rows
    assert L.moe_mlp_scratch_bytes(C.byref(h), 256, A.BF16) >= R * 256 * 2
    assert L.moe_mlp_scratch_bytes(C.byref(h), 256, A.FP8E4M3_B128) >= R * 256 + R * 2 * 4
    assert L.moe_mlp_scratch_bytes(C.byref(h), 100, A.FP8E4M3_B128) == 0
    assert L.moe_mlp_scratch_bytes(C.byref(h), 0, A.BF16) == 0


def test_dispatch_rejects_misaligned_scales_before_routing():
    """moe_dispatch runs every permute argument check before it enqueues the
    routing preprocessing: a misaligned scale pointer returns MOE_EALIGN with
    nothing enqueued and the handle still without routing metadata."""
    L = A.lib()
    d = _desc(H=256, payload="fp8")
    rc, h, base, n, _buf = _host_handle(d)
    assert rc == 0
    x = C.c_void_p(base)
    odd = C.c_void_p(base + 2)
    for xs, os_ in ((x, odd), (odd, x)):
        assert L.moe_dispatch(C.byref(h), x, None, None, x, xs, x, os_, None, x, x, None) == A.MOE_EALIGN
        assert h.state == 0
    # the same checks on a bf16 payload: scales are refused as a dtype error
    d = _desc(H=256)
    rc, h, base, n, _buf = _host_handle(d)
    x = C.c_void_p(base)
    assert L.moe_dispatch(C.byref(h), x, None, None, x, x, x, None, None, x, x, None) == A.MOE_EDTYPE
    assert L.moe_dispatch(C.byref(h), x, None, None, C.c_void_p(base + 8), None, x, None, None, x, x,
                          None) == A.MOE_EALIGN
    assert h.state == 0


def _cpu_dispatcher(**kw):
    """A Dispatcher whose workspace is host memory: handle initialisation only
    carves addresses, and every check below fails before any library call
    that would touch a device."""
    import torch
    from combine_routing_preprocess_amd import Dispatcher
    args = dict(T=64, H=256, E=4, K=2)
    args.update(kw)
    return Dispatcher(args.pop("T"), args.pop("H"), args.pop("E"), args.pop("K"), device="cpu", **args), torch


def test_mlp_binding_rejects_bad_weights_scratch_and_out():
    import pytest
    d, torch = _cpu_dispatcher()
    E, H, F, R = 4, 256, 128, d.R
    bf = torch.bfloat16
    perm = torch.zeros((R, H), dtype=bf)
    w1 = torch.zeros((E, 2 * F, H), dtype=bf)
    w2 = torch.zeros((E, H, F), dtype=bf)
    scratch = torch.zeros(d.mlp_scratch_bytes(F), dtype=torch.uint8)
    out = torch.zeros((R, H), dtype=bf)
    bad_w1 = [torch.zeros((E + 1, 2 * F, H), dtype=bf), torch.zeros((E, 2 * F, H + 8), dtype=bf),
              torch.zeros((E, 2 * F + 1, H), dtype=bf), torch.zeros((E, 2 * F, H), dtype=torch.float32),
              torch.zeros((2 * F, H), dtype=bf)]
    for w in bad_w1:
        with pytest.raises(ValueError):
            d.fc1(perm, w, scratch)
        with pytest.raises(ValueError):
            d.grouped_mlp(perm, w, w2, scratch=scratch, out=out)
    bad_w2 = [torch.zeros((E, H, F), dtype=torch.float16), torch.zeros((E, H + 8, F), dtype=bf),
              torch.zeros((E - 1, H, F), dtype=bf), torch.zeros((E, H, 2 * F), dtype=bf)]
    for w in bad_w2:
        with pytest.raises(ValueError):
            d.grouped_mlp(perm, w1, w, scratch=scratch, out=out)
    # fp8 weights without, or with wrongly shaped, block scales
    w1q = torch.zeros((E, 2 * F, H), dtype=torch.uint8)
    w2q = torch.zeros((E, H, F), dtype=torch.uint8)
    s1 = torch.ones((E, 2 * F // 128, H // 128))
    with pytest.raises(ValueError):
        d.grouped_mlp(perm, w1q, w2q, w2_scales=torch.ones((E, H // 128, F // 128)))
    with pytest.raises(ValueError):
        d.grouped_mlp(perm, w1q, w2q, w1_scales=s1, w2_scales=torch.ones((E, H // 128, 2)))
    with pytest.raises(ValueError):
        d.fc1(perm, w1, scratch, w1_scales=s1)                       # bf16 weights take no scales
    # scratch too small, out of the wrong shape or dtype
    with pytest.raises(ValueError):
        d.fc1(perm, w1, scratch[:-1])
    for o in (torch.zeros((R - 1, H), dtype=bf), torch.zeros((R, H), dtype=torch.float16)):
        with pytest.raises(ValueError):
            d.grouped_mlp(perm, w1, w2, scratch=scratch, out=o)
    # fc2 needs an fc1 first, with the same FFN width, dtype and scratch
    with pytest.raises(ValueError):
        d.fc2(w2, scratch, out)
    d._fc1_done = (F, "bf16", scratch.data_ptr())
    with pytest.raises(ValueError):
        d.fc2(torch.zeros((E, H, 2 * F), dtype=bf), torch.zeros(d.mlp_scratch_bytes(2 * F), dtype=torch.uint8), out)
    with pytest.raises(ValueError):
        d.fc2(w2, torch.zeros(d.mlp_scratch_bytes(F), dtype=torch.uint8), out)   # another scratch
    with pytest.raises(ValueError):
        d.fc2(w2, scratch, torch.zeros((R, H + 8), dtype=bf))
    with pytest.raises(ValueError):
        d.fc2_fp8out(torch.zeros((E, H, F), dtype=torch.uint8), scratch)


def test_noalloc_mlp_rejects_sizes_beyond_its_array_on_the_host():
    """moe_grouped_swiglu_mlp_noalloc refuses a problem whose activations do
    not fit its fixed device array before touching any device."""
    L = A.lib()
    d = _desc(T=8192, H=7168, E=256, K=8, pad_multiple=128)
    rc, h, base, n, _buf = _host_handle(d)
    assert rc == 0
    assert L.moe_mlp_scratch_bytes(C.byref(h), 2048, A.BF16) > A.NOALLOC_SCRATCH_BYTES
    x = C.c_void_p(base)
    assert L.moe_grouped_swiglu_mlp_noalloc(C.byref(h), 2048, A.BF16, x, None, x, None, x, None, x,
                                            None) == A.MOE_ESTALE      # no routing metadata yet
    h.state = 1   # as if routing had been enqueued; every case below fails before any device call
    assert L.moe_grouped_swiglu_mlp_noalloc(C.byref(h), 2048, A.BF16, x, None, x, None, x, None, x,
                                            None) == A.MOE_ENOSPC
    assert L.moe_grouped_swiglu_mlp_noalloc(C.byref(h), 100, A.BF16, x, None, x, None, x, None, x,
                                            None) == A.MOE_ESHAPE
    assert L.moe_grouped_swiglu_mlp_noalloc(None, 2048, A.BF16, x, None, x, None, x, None, x, None) == A.MOE_EINVAL
    assert L.moe_grouped_swiglu_mlp_noalloc(C.byref(h), 2048, A.BF16, x, None, x, None, x, None, None,
                                            None) == A.MOE_EINVAL
    assert L.moe_grouped_swiglu_mlp_noalloc(C.byref(h), 2048, A.BF16, x, None, x, None, x, None,
                                            C.c_void_p(base + 8), None) == A.MOE_EALIGN


def test_decode_fused_argument_checks_before_launch():
    """moe_decode_fused_fp8 refuses bad arguments before any device call, and
    its scratch covers the FC2 partials of every copy."""
    L = A.lib()
    d = _desc(T=16, H=256, E=8, K=2, pad_multiple=16)
    rc, h, base, n, _buf = _host_handle(d)
    assert rc == 0
    x = C.c_void_p(base)
    need = L.moe_decode_fused_scratch_bytes(C.byref(h), 256)
    assert need >= (256 // 128) * 16 * 2 * 256 * 4          # [F/128, T*K, H] fp32 partials
    assert L.moe_decode_fused_scratch_bytes(C.byref(h), 100) == 0
    call = lambda **kw: L.moe_decode_fused_fp8(
        C.byref(kw.get("h", h)), kw.get("F", 256), kw.get("x", x), kw.get("w1", x), kw.get("w1s", x),
        kw.get("w2", x), kw.get("w2s", x), kw.get("scr", x), kw.get("nbytes", need), kw.get("eo", x), 1,
        kw.get("y", x), None)
    assert call() == A.MOE_ESTALE                     # no routing metadata yet
    h.state = 1                                        # every case below fails before any device call
    assert call(F=100) == A.MOE_ESHAPE
    assert call(w1=None) == A.MOE_EINVAL
    assert call(w2s=None) == A.MOE_EINVAL
    assert call(y=None) == A.MOE_EINVAL
    assert call(eo=None) == A.MOE_EINVAL
    assert call(w2=C.c_void_p(base + 8)) == A.MOE_EALIGN
    assert call(w1s=C.c_void_p(base + 2)) == A.MOE_EALIGN
    assert call(nbytes=need - 1) == A.MOE_ENOSPC
    dw = _desc(T=16, H=8320, E=8, K=2)                 # H / 128 = 65 K blocks: past the kernel's limit
    rc, hw, basew, nw, _bufw = _host_handle(dw)
    assert rc == 0
    hw.state = 1
    assert L.moe_decode_fused_scratch_bytes(C.byref(hw), 256) == 0
    assert call(h=hw) == A.MOE_ESHAPE
    d8 = _desc(T=16, H=256, E=8, K=2, payload="fp8")
    rc, h8, base8, n8, _buf8 = _host_handle(d8)
    h8.state = 1
    assert call(h=h8, nbytes=1 << 30) == A.MOE_EDTYPE


def test_decode_layer_argument_checks_before_launch():
    """moe_decode_layer_fp8 refuses bad arguments before any device call."""
    L = A.lib()
    d = _desc(T=16, H=256, E=8, K=2, pad_multiple=16)
    rc, h, base, n, _buf = _host_handle(d)
    assert rc == 0
    x = C.c_void_p(base)
    need = L.moe_decode_layer_scratch_bytes(C.byref(h), 256)
    assert need >= L.moe_mlp_scratch_bytes(C.byref(h), 256, A.FP8E4M3_B128)
    assert L.moe_decode_layer_scratch_bytes(C.byref(h), 100) == 0
    call = lambda **kw: L.moe_decode_layer_fp8(
        C.byref(h), kw.get("F", 256), kw.get("x", x), kw.get("w1", x), kw.get("w1s", x), kw.get("w2", x),
        kw.get("w2s", x), kw.get("scr", x), kw.get("nbytes", need), kw.get("eo", x), 1, kw.get("y", x),
        kw.get("st", x), None)
    assert call() == A.MOE_ESTALE                     # no routing metadata yet
    h.state = 1                                        # every case below fails before any device call
    assert call(F=100) == A.MOE_ESHAPE
    assert call(w1=None) == A.MOE_EINVAL
    assert call(st=None) == A.MOE_EINVAL
    assert call(y=None) == A.MOE_EINVAL
    assert call(w2=C.c_void_p(base + 8)) == A.MOE_EALIGN
    assert call(st=C.c_void_p(base + 2)) == A.MOE_EALIGN
    assert call(nbytes=need - 1) == A.MOE_ENOSPC
    d8 = _desc(T=16, H=256, E=8, K=2, payload="fp8")
    rc, h8, base8, n8, _buf8 = _host_handle(d8)
    h8.state = 1
    assert L.moe_decode_layer_fp8(C.byref(h8), 256, x, x, x, x, x, x, 1 << 30, x, 1, x, x, None) == A.MOE_EDTYPE
