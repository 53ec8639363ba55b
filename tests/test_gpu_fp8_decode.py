"""fp8-weight (W8A8, 128x128 weight-block scales) grouped MLP and the
decode-sized layer with HIP-graph replay, against the oracle.  Tolerance for
fp8: per-row relative L2 <= 5e-2."""
import numpy as np
import pytest
import torch

import moe_synth as S
import oracle
import combine_routing_preprocess_amd._abi as A
from combine_routing_preprocess_amd import Dispatcher
from gpu_util import DEV, dev, host_bf16, log, rel_l2, require_clear_flag, row_rel_l2

pytestmark = pytest.mark.gpu
TOL8 = 5e-2


def _check(got_bits, want_bits, what, tol=TOL8):
    g = S.bf16_to_float(got_bits)
    w = S.bf16_to_float(want_bits)
    assert rel_l2(g, w) < tol, (what, rel_l2(g, w))
    rr = row_rel_l2(g, w)
    assert rr.max() < tol, (what, rr.max(), int(rr.argmax()))


@pytest.mark.parametrize("counts,H,F", [
    ([0, 1, 15, 17, 70], 256, 256),
    ([3, 0, 64, 65], 512, 128),
])
def test_fp8_mlp_ragged(counts, H, F):
    E = len(counts)
    T = int(sum(counts))
    idx = np.repeat(np.arange(E), counts).astype(np.int16)[:, None]
    idx = idx[np.random.default_rng(T).permutation(T)]
    x = S.bf16_normal((T, H), 200 + T)
    w1q, w1s = S.weights_fp8_blocks(E, 2 * F, H, 201, std=0.05)
    w2q, w2s = S.weights_fp8_blocks(E, H, F, 202, std=0.05)
    log("fp8 mlp ragged", counts, H, F)
    d = Dispatcher(T, H, E, 1, pad_multiple=16)
    perm, *_ = d.dispatch(dev(x), dev(idx))
    y = d.grouped_mlp(perm, w1q.to(DEV), w2q.to(DEV), w1_scales=w1s.to(DEV), w2_scales=w2s.to(DEV))
    torch.cuda.synchronize()
    rt = oracle.route(idx, 0, E, 1, None, 16, -1, d.R)
    P = oracle.permute_rows(x, rt["row_id"], d.R)
    got = host_bf16(y)
    for e in range(E):
        s, k = int(rt["seg_off"][e]), int(rt["counts"][e])
        if k == 0:
            continue
        want = oracle.expert_mlp_fp8(P[s:s + k], w1q[e].numpy(), w1s[e].numpy(), w2q[e].numpy(), w2s[e].numpy())
        _check(got[s:s + k], want, f"expert {e}")


@pytest.fixture(scope="module")
def fp8_weights():
    """256 experts, H 7168, FFN 2048, e4m3 weights drawn N(0, 0.02) with
    128x128 block scales (W1 7.5 GB + W2 3.8 GB on the device)."""
    c = S.CONFIGS["decode_fp8_7168_e256"]
    w1q, w1s = S.weights_fp8_blocks(c.E, 2 * c.F, c.H, c.seed + 1, device=DEV)
    w2q, w2s = S.weights_fp8_blocks(c.E, c.H, c.F, c.seed + 2, device=DEV)
    yield c, w1q, w1s, w2q, w2s


def _decode_case(c, T):
    bucket = S.next_pow2_bucket(T)
    idx, pr = S.route_sigmoid_topk(bucket, c.E, c.K, c.seed + T)
    x = S.bf16_normal((bucket, c.H), c.seed + T)
    return bucket, idx, pr, x


@pytest.mark.parametrize("T", [16, 64, 100, 256])
def test_decode_layer_all_live_tokens(fp8_weights, T):
    """The fp8 decode layer in buckets 16, 64, 128 (100 live tokens) and 256:
    every live token against the oracle, and the tokens past the live count
    exactly zero."""
    c, w1q, w1s, w2q, w2s = fp8_weights
    bucket, idx, pr, x = _decode_case(c, T)
    log("fp8 decode layer", T, bucket)
    d = Dispatcher(bucket, c.H, c.E, c.K, pad_multiple=c.pad)
    tl = torch.tensor([T], dtype=torch.int32, device=DEV)
    y = d.layer(dev(x), dev(idx), dev(pr), w1q, w2q, w1_scales=w1s, w2_scales=w2s, T_live=tl)
    torch.cuda.synchronize()
    rt = oracle.route(idx, 0, c.E, c.K, pr, c.pad, -1, d.R, T)
    assert np.array_equal(d.row_id.cpu().numpy(), rt["row_id"])
    toks = list(range(T))
    want = oracle.layer_tokens(toks, x, rt, lambda e, rows: oracle.expert_mlp_fp8(
        rows, w1q[e].cpu().numpy(), w1s[e].cpu().numpy(), w2q[e].cpu().numpy(), w2s[e].cpu().numpy()))
    _check(host_bf16(y[toks]), want, f"T {T}")
    # tokens past the live count are unrouted: their output is exactly zero
    if T < bucket:
        assert torch.count_nonzero(y[T:].float()).item() == 0


def test_decode_graph_replay_matches_eager(fp8_weights):
    """Capture dispatch + FC1 + FC2 + combine once per bucket; replay with new
    inputs copied into the captured buffers; every replay equals the eager
    run on the same inputs bit for bit."""
    c, w1q, w1s, w2q, w2s = fp8_weights
    for bucket in (16, 64):
        log("fp8 decode graph", bucket)
        d = Dispatcher(bucket, c.H, c.E, c.K, pad_multiple=c.pad)
        # captured buffers, filled with a valid routing before the warm-up and
        # the capture: the step ends with the device-side overflow assert
        _, idx, pr, x = _decode_case(c, bucket)
        xb = dev(x).view(torch.bfloat16)
        rb = dev(idx)
        pb = dev(pr)
        tl = torch.tensor([bucket], dtype=torch.int32, device=DEV)
        require_clear_flag(d, rb, pb, tl)
        perm = torch.empty((d.R, c.H), dtype=torch.bfloat16, device=DEV)
        scratch = d.alloc_mlp_scratch(c.F, "fp8")
        eo = torch.empty((d.R, c.H), dtype=torch.bfloat16, device=DEV)
        yb = torch.empty((bucket, c.H), dtype=torch.bfloat16, device=DEV)

        def step():
            d.layer(xb, rb, pb, w1q, w2q, w1_scales=w1s, w2_scales=w2s, T_live=tl, perm=perm, scratch=scratch,
                    expert_out=eo, out=yb, check_overflow=True)

        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step()
        torch.cuda.current_stream().wait_stream(s)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        for rep, T in enumerate((bucket, bucket // 2 + 1, 1, 0)):
            _, idx, pr, x = _decode_case(c, bucket)
            idx = np.roll(idx, rep, axis=0)
            xb.copy_(dev(x).view(torch.bfloat16))
            rb.copy_(dev(idx))
            pb.copy_(dev(pr))
            tl.fill_(T)
            require_clear_flag(d, rb, pb, tl)      # the replay recomputes this same flag
            g.replay()
            torch.cuda.synchronize()
            replay = yb.clone()
            step()
            torch.cuda.synchronize()
            assert torch.equal(replay.view(torch.int16), yb.view(torch.int16)), (bucket, rep)
            assert int(d.flag.item()) == 0


@pytest.mark.parametrize("T", [16, 100])
def test_layer_quantise_on_dispatch_matches_permute_then_quantise(fp8_weights, T):
    """layer() on a handle of fp8 payload (routing metadata, quantise-on-
    dispatch, fp8 grouped MLP, combine) equals layer() on a bf16 handle
    (permute, row quantiser, fp8 grouped MLP, combine) bit for bit, live
    count below the bucket included."""
    c, w1q, w1s, w2q, w2s = fp8_weights
    bucket, idx, pr, x = _decode_case(c, T)
    log("layer quantise-on-dispatch", T, bucket)
    tl = torch.tensor([T], dtype=torch.int32, device=DEV)
    d8 = Dispatcher(bucket, c.H, c.E, c.K, pad_multiple=c.pad, payload="fp8")
    y8 = d8.layer(dev(x), dev(idx), dev(pr), w1q, w2q, w1_scales=w1s, w2_scales=w2s, T_live=tl,
                  check_overflow=True)
    d = Dispatcher(bucket, c.H, c.E, c.K, pad_multiple=c.pad)
    y = d.layer(dev(x), dev(idx), dev(pr), w1q, w2q, w1_scales=w1s, w2_scales=w2s, T_live=tl)
    torch.cuda.synchronize()
    assert int(d8.flag.item()) == 0
    assert torch.equal(y8.view(torch.int16), y.view(torch.int16))


def _megakernel_case(c, d, x, idx, pr, tl, w1q, w1s, w2q, w2s, scratch=None, status_init=3):
    """preprocess + the persistent decode layer; returns (y, expert_out,
    status).  The status word starts at `status_init` (bits 0 and 1 are
    cleared by the call, bit 2 is the caller's abort request)."""
    scratch = scratch if scratch is not None else torch.empty(d.decode_layer_scratch_bytes(c.F), dtype=torch.uint8,
                                                              device=DEV)
    eo = torch.empty((d.R, c.H), dtype=torch.bfloat16, device=DEV)
    y = torch.full((d.T, c.H), 7.0, dtype=torch.bfloat16, device=DEV)
    st = torch.full((1,), status_init, dtype=torch.int32, device=DEV)
    d.preprocess(dev(idx), dev(pr), tl)
    d.decode_layer_fp8(dev(x), w1q, w2q, w1s, w2s, scratch=scratch, expert_out=eo, out=y, status=st)
    return y, eo, st


@pytest.mark.parametrize("T", [16, 64, 100, 256])
def test_decode_megakernel_matches_separate_launches_and_oracle(fp8_weights, T):
    """The persistent decode layer (quantise-on-dispatch, FC1, activation
    quantiser, FC2, combine in one launch) equals the separate launches bit
    for bit, and every live token agrees with the oracle."""
    c, w1q, w1s, w2q, w2s = fp8_weights
    bucket, idx, pr, x = _decode_case(c, T)
    log("decode megakernel", T, bucket)
    tl = torch.tensor([T], dtype=torch.int32, device=DEV)
    d = Dispatcher(bucket, c.H, c.E, c.K, pad_multiple=c.pad)
    y, eo, st = _megakernel_case(c, d, x, idx, pr, tl, w1q, w1s, w2q, w2s)
    d2 = Dispatcher(bucket, c.H, c.E, c.K, pad_multiple=c.pad)
    y2 = d2.layer(dev(x), dev(idx), dev(pr), w1q, w2q, w1_scales=w1s, w2_scales=w2s, T_live=tl)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    rt = oracle.route(idx, 0, c.E, c.K, pr, c.pad, -1, d.R, T)
    want = oracle.layer_tokens(list(range(T)), x, rt, lambda e, rows: oracle.expert_mlp_fp8(
        rows, w1q[e].cpu().numpy(), w1s[e].cpu().numpy(), w2q[e].cpu().numpy(), w2s[e].cpu().numpy()))
    _check(host_bf16(y[:T]), want, f"megakernel T {T}")
    if T < bucket:
        assert torch.count_nonzero(y[T:].float()).item() == 0


def test_decode_megakernel_graph_replay_and_empty_batch(fp8_weights):
    """preprocess + the persistent decode layer captured once per bucket and
    replayed with new inputs (live counts bucket, half, 1 and 0): every replay
    equals the eager run bit for bit with a clear status word."""
    c, w1q, w1s, w2q, w2s = fp8_weights
    for bucket in (16, 64):
        log("decode megakernel graph", bucket)
        d = Dispatcher(bucket, c.H, c.E, c.K, pad_multiple=c.pad)
        _, idx, pr, x = _decode_case(c, bucket)
        xb, rb, pb = dev(x).view(torch.bfloat16), dev(idx), dev(pr)
        tl = torch.tensor([bucket], dtype=torch.int32, device=DEV)
        scr = torch.empty(d.decode_layer_scratch_bytes(c.F), dtype=torch.uint8, device=DEV)
        eo = torch.empty((d.R, c.H), dtype=torch.bfloat16, device=DEV)
        yb = torch.empty((bucket, c.H), dtype=torch.bfloat16, device=DEV)
        st = torch.empty(1, dtype=torch.int32, device=DEV)

        def step():
            d.preprocess(rb, pb, tl)
            d.decode_layer_fp8(xb, w1q, w2q, w1s, w2s, scratch=scr, expert_out=eo, out=yb, status=st)

        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step()
        torch.cuda.current_stream().wait_stream(s)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        for rep, T in enumerate((bucket, bucket // 2 + 1, 1, 0)):
            _, idx, pr, x = _decode_case(c, bucket)
            rb.copy_(dev(np.roll(idx, rep + 1, axis=0)))
            pb.copy_(dev(pr))
            xb.copy_(dev(x).view(torch.bfloat16))
            tl.fill_(T)
            g.replay()
            torch.cuda.synchronize()
            assert int(st.item()) == 0, (bucket, rep)
            replay = yb.clone()
            step()
            torch.cuda.synchronize()
            assert int(st.item()) == 0
            assert torch.equal(replay.view(torch.int16), yb.view(torch.int16)), (bucket, rep)
            if T == 0:
                assert torch.count_nonzero(yb.float()).item() == 0


def test_decode_megakernel_abort_and_wait_bound(fp8_weights):
    """Failure handling forced from the host, each call ending normally: the
    caller's abort bit makes every wait return at once (the status keeps
    bit 2 and gains nothing else); a wait bound of one tick makes waits run
    past it (status bit 0); the next call, with the default bound and a clear
    status, is bit-identical to the separate launches."""
    c, w1q, w1s, w2q, w2s = fp8_weights
    bucket, idx, pr, x = _decode_case(c, 16)
    tl = torch.tensor([16], dtype=torch.int32, device=DEV)
    d = Dispatcher(bucket, c.H, c.E, c.K, pad_multiple=c.pad)
    log("decode megakernel abort")
    _, _, st = _megakernel_case(c, d, x, idx, pr, tl, w1q, w1s, w2q, w2s, status_init=4)
    torch.cuda.synchronize()
    assert int(st.item()) == 4
    log("decode megakernel wait bound 1 tick")
    A.lib().moe_decode_layer_set_wait_bound(1)
    try:
        _, _, st = _megakernel_case(c, d, x, idx, pr, tl, w1q, w1s, w2q, w2s, status_init=0)
        torch.cuda.synchronize()
    finally:
        A.lib().moe_decode_layer_set_wait_bound(0)
    assert int(st.item()) & 3 == 1
    log("decode megakernel after the forced failures")
    y, _, st = _megakernel_case(c, d, x, idx, pr, tl, w1q, w1s, w2q, w2s, status_init=0)
    d2 = Dispatcher(bucket, c.H, c.E, c.K, pad_multiple=c.pad)
    y2 = d2.layer(dev(x), dev(idx), dev(pr), w1q, w2q, w1_scales=w1s, w2_scales=w2s, T_live=tl)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("apply_probs", [True, False])
def test_decode_megakernel_sparse_routing_and_capacity(apply_probs):
    """The persistent decode layer on a Boolean routing map with a capacity
    that drops copies (some tokens lose all of theirs, and their rows must
    come out zero): bit-identical to the separate launches on the same
    handle state, with and without the probability weights, against the
    oracle, and with a clear status."""
    T, H, E, K, F, pad, cap = 48, 256, 6, 3, 256, 8, 20
    idx, pr = S.route_softmax_topk(T, E, K, 77)
    smap, sprob = S.dense_to_sparse(idx, E, pr)
    x = S.bf16_normal((T, H), 78)
    w1q, w1s = S.weights_fp8_blocks(E, 2 * F, H, 79, std=0.05)
    w2q, w2s = S.weights_fp8_blocks(E, H, F, 80, std=0.05)
    W = [t.to(DEV) for t in (w1q, w1s, w2q, w2s)]
    log("decode megakernel sparse", apply_probs)
    d = Dispatcher(T, H, E, K, route_fmt="sparse_bool", pad_multiple=pad, capacity=cap)
    scr = torch.empty(d.decode_layer_scratch_bytes(F), dtype=torch.uint8, device=DEV)
    eo = torch.zeros((d.R, H), dtype=torch.bfloat16, device=DEV)
    y = torch.full((T, H), 7.0, dtype=torch.bfloat16, device=DEV)
    st = torch.full((1,), 3, dtype=torch.int32, device=DEV)
    d.preprocess(dev(smap), dev(sprob))
    d.decode_layer_fp8(dev(x), W[0], W[2], W[1], W[3], scratch=scr, expert_out=eo, out=y, status=st,
                       apply_probs=apply_probs)
    d2 = Dispatcher(T, H, E, K, route_fmt="sparse_bool", pad_multiple=pad, capacity=cap)
    perm, *_ = d2.dispatch(dev(x), dev(smap), dev(sprob))
    eo2 = d2.grouped_mlp(perm, W[0], W[2], w1_scales=W[1], w2_scales=W[3])
    y2 = d2.combine(eo2, apply_probs=apply_probs)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert int(d.flag.item()) & 1                      # the capacity dropped copies
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    kept_rows = (d.src_row >= 0).nonzero().flatten()
    assert torch.equal(eo[kept_rows].view(torch.int16), eo2[kept_rows].view(torch.int16))
    rt = oracle.route(smap, oracle.FMT_SPARSE_U8, E, K, sprob, pad, cap, d.R)
    want = oracle.layer_tokens(np.arange(T), x, rt, lambda e, rows: oracle.expert_mlp_fp8(
        rows, w1q[e].numpy(), w1s[e].numpy(), w2q[e].numpy(), w2s[e].numpy()), apply_probs=apply_probs)
    _check(host_bf16(y), want, "megakernel sparse")
    none = (rt["row_id"] < 0).all(axis=1)
    assert none.any()
    assert torch.count_nonzero(y[torch.from_numpy(np.nonzero(none)[0]).to(DEV)].float()).item() == 0


def test_decode_megakernel_random_batches_back_to_back(fp8_weights):
    """Ten decode batches at the full layer width, one after another on the
    same scratch, expert-output and output buffers: random live counts
    (1..256), softmax or Zipf-skewed routing, some with a capacity that
    drops copies.  Each is bit-identical to the separate launches with a
    clear status; the skewed ones pile many rows on a few experts, so
    several passes over an expert's weights and uneven queues are covered."""
    c, w1q, w1s, w2q, w2s = fp8_weights
    r = np.random.default_rng(2024)
    scr = eo = y = None
    for case in range(10):
        T = int(r.integers(1, 257))
        bucket = S.next_pow2_bucket(T)
        if case % 2:
            idx, pr = S.route_zipf_gumbel(bucket, c.E, c.K, 500 + case)
        else:
            idx, pr = S.route_softmax_topk(bucket, c.E, c.K, 500 + case)
        x = S.bf16_normal((bucket, c.H), 600 + case)
        cap = int(r.integers(8, 40)) if case % 3 == 0 else None
        log("decode megakernel random", case, T, bucket, cap)
        tl = torch.tensor([T], dtype=torch.int32, device=DEV)
        d = Dispatcher(bucket, c.H, c.E, c.K, pad_multiple=c.pad, capacity=cap)
        need = d.decode_layer_scratch_bytes(c.F)
        if scr is None or scr.numel() < need:
            scr = torch.empty(need, dtype=torch.uint8, device=DEV)
        if eo is None or eo.shape[0] < d.R:
            eo = torch.empty((d.R, c.H), dtype=torch.bfloat16, device=DEV)
        if y is None or y.shape[0] < bucket:
            y = torch.empty((bucket, c.H), dtype=torch.bfloat16, device=DEV)
        st = torch.full((1,), 3, dtype=torch.int32, device=DEV)
        yv, eov = y[:bucket], eo[:d.R]
        d.preprocess(dev(idx), dev(pr), tl)
        d.decode_layer_fp8(dev(x), w1q, w2q, w1s, w2s, scratch=scr, expert_out=eov, out=yv, status=st)
        d2 = Dispatcher(bucket, c.H, c.E, c.K, pad_multiple=c.pad, capacity=cap)
        y2 = d2.layer(dev(x), dev(idx), dev(pr), w1q, w2q, w1_scales=w1s, w2_scales=w2s, T_live=tl)
        torch.cuda.synchronize()
        assert int(st.item()) == 0, case
        assert torch.equal(yv.view(torch.int16), y2.view(torch.int16)), case


@pytest.mark.parametrize("T,H,E,K,F,pad", [(33, 256, 8, 2, 256, 16), (1, 128, 4, 1, 128, 1), (70, 384, 5, 3, 128, 8)])
def test_decode_megakernel_small_shapes(T, H, E, K, F, pad):
    """Small shapes, ragged expert counts: bit-identical to the separate
    launches, and against the oracle."""
    idx, pr = S.route_softmax_topk(T, E, K, 40 + T)
    x = S.bf16_normal((T, H), 41 + T)
    w1q, w1s = S.weights_fp8_blocks(E, 2 * F, H, 42, std=0.05)
    w2q, w2s = S.weights_fp8_blocks(E, H, F, 43, std=0.05)
    W = [t.to(DEV) for t in (w1q, w1s, w2q, w2s)]
    log("decode megakernel small", T, H, E, K, F, pad)
    d = Dispatcher(T, H, E, K, pad_multiple=pad)
    scr = torch.empty(d.decode_layer_scratch_bytes(F), dtype=torch.uint8, device=DEV)
    eo = torch.empty((d.R, H), dtype=torch.bfloat16, device=DEV)
    y = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    st = torch.full((1,), 3, dtype=torch.int32, device=DEV)
    d.preprocess(dev(idx), dev(pr))
    d.decode_layer_fp8(dev(x), W[0], W[2], W[1], W[3], scratch=scr, expert_out=eo, out=y, status=st)
    d2 = Dispatcher(T, H, E, K, pad_multiple=pad)
    y2 = d2.layer(dev(x), dev(idx), dev(pr), W[0], W[2], w1_scales=W[1], w2_scales=W[3])
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    rt = oracle.route(idx, 0, E, K, pr, pad, -1, d.R)
    want = oracle.layer_tokens(np.arange(T), x, rt, lambda e, rows: oracle.expert_mlp_fp8(
        rows, w1q[e].numpy(), w1s[e].numpy(), w2q[e].numpy(), w2s[e].numpy()))
    _check(host_bf16(y), want, "megakernel small")


# ---- fused decode layer (quantise-on-dispatch launch + one persistent kernel) ----

def _fused_run(d, x, idx, pr, tl, w1, w1s, w2, w2s, F, H):
    """preprocess + the fused decode layer on fresh buffers; returns (y, expert_out)."""
    scratch = torch.empty(d.decode_fused_scratch_bytes(F), dtype=torch.uint8, device=DEV)
    scratch.fill_(0xA5)                                # the call must not depend on scratch contents
    eo = torch.zeros((d.R, H), dtype=torch.bfloat16, device=DEV)
    y = torch.full((d.T, H), 7.0, dtype=torch.bfloat16, device=DEV)
    d.preprocess(dev(idx), dev(pr), tl)
    d.decode_fused_fp8(dev(x), w1, w2, w1s, w2s, scratch=scratch, expert_out=eo, out=y)
    return y, eo


def _separate_run(d, x, idx, pr, tl, w1, w1s, w2, w2s):
    """The same layer as separate launches: dispatch, fp8 grouped MLP, combine."""
    perm, *_ = d.dispatch(dev(x), dev(idx), dev(pr), T_live=tl)
    eo = d.grouped_mlp(perm, w1, w2, w1_scales=w1s, w2_scales=w2s)
    y = d.combine(eo)
    return y, eo


def _assert_same_as_separate(d, y, eo, y2, eo2):
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    kept_rows = (d.src_row >= 0).nonzero().flatten()
    assert torch.equal(eo[kept_rows].view(torch.int16), eo2[kept_rows].view(torch.int16))


@pytest.mark.parametrize("T", [16, 64, 100, 256])
def test_decode_fused_matches_separate_launches_and_oracle(fp8_weights, T):
    """The fused decode layer in buckets 16, 64, 128 (100 live) and 256:
    output and expert rows bit-identical to the separate launches, live
    tokens against the oracle (all of them up to 64, every third above),
    tokens past the live count exactly zero."""
    c, w1q, w1s, w2q, w2s = fp8_weights
    bucket, idx, pr, x = _decode_case(c, T)
    log("fused decode", T, bucket)
    tl = torch.tensor([T], dtype=torch.int32, device=DEV)
    d = Dispatcher(bucket, c.H, c.E, c.K, pad_multiple=c.pad)
    y, eo = _fused_run(d, x, idx, pr, tl, w1q, w1s, w2q, w2s, c.F, c.H)
    d2 = Dispatcher(bucket, c.H, c.E, c.K, pad_multiple=c.pad)
    y2, eo2 = _separate_run(d2, x, idx, pr, tl, w1q, w1s, w2q, w2s)
    torch.cuda.synchronize()
    _assert_same_as_separate(d, y, eo, y2, eo2)
    rt = oracle.route(idx, 0, c.E, c.K, pr, c.pad, -1, d.R, T)
    toks = list(range(T)) if T <= 64 else list(range(0, T, 3))
    want = oracle.layer_tokens(toks, x, rt, lambda e, rows: oracle.expert_mlp_fp8(
        rows, w1q[e].cpu().numpy(), w1s[e].cpu().numpy(), w2q[e].cpu().numpy(), w2s[e].cpu().numpy()))
    _check(host_bf16(y[toks]), want, f"fused T {T}")
    if T < bucket:
        assert torch.count_nonzero(y[T:].float()).item() == 0


def test_decode_fused_graph_replay(fp8_weights):
    """preprocess + the fused decode layer captured once per bucket and
    replayed with new inputs and live counts (bucket, half, 1, 0): every
    replay equals the eager run bit for bit; no live token gives all zeros."""
    c, w1q, w1s, w2q, w2s = fp8_weights
    for bucket in (16, 64):
        log("fused decode graph", bucket)
        d = Dispatcher(bucket, c.H, c.E, c.K, pad_multiple=c.pad)
        _, idx, pr, x = _decode_case(c, bucket)
        xb, rb, pb = dev(x).view(torch.bfloat16), dev(idx), dev(pr)
        tl = torch.tensor([bucket], dtype=torch.int32, device=DEV)
        scr = torch.empty(d.decode_fused_scratch_bytes(c.F), dtype=torch.uint8, device=DEV)
        eo = torch.empty((d.R, c.H), dtype=torch.bfloat16, device=DEV)
        yb = torch.empty((bucket, c.H), dtype=torch.bfloat16, device=DEV)

        def step():
            d.preprocess(rb, pb, tl)
            d.decode_fused_fp8(xb, w1q, w2q, w1s, w2s, scratch=scr, expert_out=eo, out=yb)

        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step()
        torch.cuda.current_stream().wait_stream(s)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        for rep, T in enumerate((bucket, bucket // 2 + 1, 1, 0)):
            _, idx, pr, x = _decode_case(c, bucket)
            rb.copy_(dev(np.roll(idx, rep + 1, axis=0)))
            pb.copy_(dev(pr))
            xb.copy_(dev(x).view(torch.bfloat16))
            tl.fill_(T)
            yb.fill_(3.0)
            g.replay()
            torch.cuda.synchronize()
            replay = yb.clone()
            yb.fill_(5.0)
            step()
            torch.cuda.synchronize()
            assert torch.equal(replay.view(torch.int16), yb.view(torch.int16)), (bucket, rep)
            if T == 0:
                assert torch.count_nonzero(yb.float()).item() == 0


@pytest.mark.parametrize("T,H,E,K,F,pad,counts", [
    (33, 256, 8, 2, 256, 16, None),
    (1, 128, 4, 1, 128, 1, None),
    (70, 384, 5, 3, 128, 8, None),                   # > 32 rows per expert: passes of 32 and the rest
    (67, 256, 5, 1, 256, 4, [0, 1, 16, 17, 33]),     # one and two token blocks, a pass boundary
])
def test_decode_fused_small_shapes(T, H, E, K, F, pad, counts):
    """Small and ragged shapes (a final half stage of W2 rows at H = 128 and
    384, several passes over an expert's weights): bit-identical to the
    separate launches, and against the oracle."""
    if counts is None:
        idx, pr = S.route_softmax_topk(T, E, K, 40 + T)
    else:
        idx = np.repeat(np.arange(E), counts).astype(np.int16)[:, None]
        idx = idx[np.random.default_rng(T).permutation(T)]
        pr = np.ones((T, K), np.float32)
    x = S.bf16_normal((T, H), 41 + T)
    w1q, w1s = S.weights_fp8_blocks(E, 2 * F, H, 42, std=0.05)
    w2q, w2s = S.weights_fp8_blocks(E, H, F, 43, std=0.05)
    W = [t.to(DEV) for t in (w1q, w1s, w2q, w2s)]
    log("fused decode small", T, H, E, K, F, pad)
    tl = torch.tensor([T], dtype=torch.int32, device=DEV)
    d = Dispatcher(T, H, E, K, pad_multiple=pad)
    y, eo = _fused_run(d, x, idx, pr, tl, W[0], W[1], W[2], W[3], F, H)
    d2 = Dispatcher(T, H, E, K, pad_multiple=pad)
    y2, eo2 = _separate_run(d2, x, idx, pr, tl, W[0], W[1], W[2], W[3])
    torch.cuda.synchronize()
    _assert_same_as_separate(d, y, eo, y2, eo2)
    rt = oracle.route(idx, 0, E, K, pr, pad, -1, d.R)
    want = oracle.layer_tokens(np.arange(T), x, rt, lambda e, rows: oracle.expert_mlp_fp8(
        rows, w1q[e].numpy(), w1s[e].numpy(), w2q[e].numpy(), w2s[e].numpy()))
    _check(host_bf16(y), want, "fused small")


@pytest.mark.parametrize("apply_probs", [True, False])
def test_decode_fused_sparse_routing_and_capacity(apply_probs):
    """The fused decode layer on a Boolean routing map with a capacity that
    drops copies (some tokens lose all of theirs): bit-identical to the
    separate launches on the same handle state, with and without the
    probability weights, and against the oracle."""
    T, H, E, K, F, pad, cap = 48, 256, 6, 3, 256, 8, 20
    idx, pr = S.route_softmax_topk(T, E, K, 77)
    smap, sprob = S.dense_to_sparse(idx, E, pr)
    x = S.bf16_normal((T, H), 78)
    w1q, w1s = S.weights_fp8_blocks(E, 2 * F, H, 79, std=0.05)
    w2q, w2s = S.weights_fp8_blocks(E, H, F, 80, std=0.05)
    W = [t.to(DEV) for t in (w1q, w1s, w2q, w2s)]
    log("fused decode sparse", apply_probs)
    d = Dispatcher(T, H, E, K, route_fmt="sparse_bool", pad_multiple=pad, capacity=cap)
    scratch = torch.empty(d.decode_fused_scratch_bytes(F), dtype=torch.uint8, device=DEV)
    eo = torch.zeros((d.R, H), dtype=torch.bfloat16, device=DEV)
    y = torch.full((T, H), 7.0, dtype=torch.bfloat16, device=DEV)
    d.preprocess(dev(smap), dev(sprob))
    d.decode_fused_fp8(dev(x), W[0], W[2], W[1], W[3], scratch=scratch, expert_out=eo, out=y,
                       apply_probs=apply_probs)
    d2 = Dispatcher(T, H, E, K, route_fmt="sparse_bool", pad_multiple=pad, capacity=cap)
    perm, *_ = d2.dispatch(dev(x), dev(smap), dev(sprob))
    eo2 = d2.grouped_mlp(perm, W[0], W[2], w1_scales=W[1], w2_scales=W[3])
    y2 = d2.combine(eo2, apply_probs=apply_probs)
    torch.cuda.synchronize()
    assert int(d.flag.item()) & 1                      # the capacity dropped copies
    _assert_same_as_separate(d, y, eo, y2, eo2)
    rt = oracle.route(smap, oracle.FMT_SPARSE_U8, E, K, sprob, pad, cap, d.R)
    want = oracle.layer_tokens(np.arange(T), x, rt, lambda e, rows: oracle.expert_mlp_fp8(
        rows, w1q[e].numpy(), w1s[e].numpy(), w2q[e].numpy(), w2s[e].numpy()), apply_probs=apply_probs)
    _check(host_bf16(y), want, "fused sparse")
    none = (rt["row_id"] < 0).all(axis=1)
    assert none.any()
    assert torch.count_nonzero(y[torch.from_numpy(np.nonzero(none)[0]).to(DEV)].float()).item() == 0
