"""Backward of dispatch and of combine on the GPU against the oracle.

Token gradients (a sum of copies in fp32) must match within one bf16 unit in
the last place and almost everywhere exactly; row gradients (one exactly
rounded product) and gathered probability gradients bit for bit; the
probability gradient of the combine (an fp32 dot product over H) within the
fp32 summation bound of its reduction tree."""
import numpy as np
import pytest
import torch

import moe_synth as S
import oracle
from combine_routing_preprocess_amd import Dispatcher, assert_no_overflow
from gpu_util import DEV, FMT_NAME, dev, host_bf16, log

pytestmark = pytest.mark.gpu


def _ulp_diff(a_bits, b_bits):
    """Distance in bf16 units in the last place (same-sign finite values)."""
    a = a_bits.astype(np.int32)
    b = b_bits.astype(np.int32)
    ka = np.where(a & 0x8000, -(a & 0x7FFF), a)
    kb = np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(ka - kb)


def _dot_tol(gy_f, Y_f, H):
    """fp32 bound for the GPU's dot product, from the depth of its summation
    tree.  Rows of up to 16 pieces of 64 chunks: each lane sums the 8
    products of its chunk in order, 6 butterfly levels reduce a piece, and
    the pieces are added in order.  Longer rows: each lane sums 8 products
    per chunk it walks, then 6 butterfly levels.  Plus the oracle's rounding
    of its double result to float."""
    pieces = (H // 8 + 63) // 64
    n = (8 + 6 + pieces if pieces <= 16 else 8 * pieces + 6) + 1
    return n * 2.0 ** -24 * np.abs(gy_f * Y_f).sum(axis=-1)


def _routing(T, E, K, fmt, seed):
    idx, pr = S.route_softmax_topk(T, E, K, seed)
    if T > 3 and K > 1:
        idx = idx.copy()
        idx[1, K - 1] = -1                  # empty slot
        idx[2, K - 1] = idx[2, 0]           # duplicate, dropped
    if fmt == oracle.FMT_SPARSE_U8:
        return S.dense_to_sparse(idx, E, pr)
    return idx.astype(np.int16 if fmt == oracle.FMT_DENSE_I16 else np.int32), pr


CASES = [
    # T, H, E, K, pad, cap, fmt
    (70, 64, 5, 3, 4, -1, oracle.FMT_DENSE_I16),
    (300, 1024, 16, 4, 32, -1, oracle.FMT_SPARSE_U8),
    (129, 512, 8, 8, 1, 20, oracle.FMT_DENSE_I32),
    (257, 2056, 12, 3, 7, 40, oracle.FMT_SPARSE_U8),      # ragged row (257 chunks), drops
    (33, 8200, 6, 2, 1, -1, oracle.FMT_DENSE_I16),        # row longer than the register-held path
    (40, 1536, 160, 96, 2, -1, oracle.FMT_DENSE_I32),     # K > 64: two passes of the probability sum
    (20, 8192, 4, 2, 1, -1, oracle.FMT_DENSE_I16),        # 16 pieces: the longest row one workgroup holds
    (5, 512, 1024, 1024, 1, -1, oracle.FMT_DENSE_I16),    # K = E = 1024, the largest partial table
    (1, 8, 1, 1, 1, -1, oracle.FMT_DENSE_I16),
    (0, 256, 4, 2, 1, -1, oracle.FMT_DENSE_I16),
]


@pytest.mark.parametrize("T,H,E,K,pad,cap,fmt", CASES)
@pytest.mark.parametrize("apply", [True, False])
def test_backward_matches_oracle(T, H, E, K, pad, cap, fmt, apply):
    sparse = fmt == oracle.FMT_SPARSE_U8
    routing, probs = _routing(T, E, K, fmt, T + H)
    log("backward", T, H, E, K, pad, cap, fmt, apply)
    d = Dispatcher(T, H, E, K, route_fmt=FMT_NAME[fmt], pad_multiple=pad, capacity=None if cap < 0 else cap)
    d.preprocess(dev(routing), dev(probs))
    rt = oracle.route(routing, fmt, E, K, probs, pad, cap, d.R)
    R = d.R
    G = S.bf16_normal((R, H), 7 + T)
    gop = np.random.default_rng(8 + T).standard_normal(R).astype(np.float32)
    Y = S.bf16_normal((R, H), 9 + T)
    gy = S.bf16_normal((T, H), 10 + T)

    # ---- dispatch backward -------------------------------------------------
    gx, gp = d.dispatch_backward(dev(G), dev(gop))
    # ---- combine backward (canary rows after R stay untouched) --------------
    canary = torch.full((R + 2, H), 1.5, dtype=torch.bfloat16, device=DEV)
    gY, gq = d.combine_backward(dev(gy), dev(Y), apply, out=canary[:R])
    torch.cuda.synchronize()

    wx, wp = oracle.dispatch_backward(G, rt, E, sparse, gop)
    gx_h = host_bf16(gx)
    if T:
        assert _ulp_diff(gx_h, wx).max() <= 1
        assert (gx_h == wx).mean() > 0.999
    assert np.array_equal(gp.cpu().numpy().view(np.uint32), wp.view(np.uint32))

    wY, wq = oracle.combine_backward(gy, Y, rt, E, sparse, apply)
    rows = np.nonzero(rt["src_row"] >= 0)[0]
    got = host_bf16(canary)
    assert np.array_equal(got[rows], wY[rows])
    assert np.all(got[R:] == 0x3FC0)
    gq_h = gq.cpu().numpy()
    assert gq_h.shape == wq.shape
    if not apply:
        assert not gq_h.any()
    else:
        tk, jk = np.nonzero(rt["row_id"] >= 0)
        cols = rt["copy_expert"][tk, jk] if sparse else jk
        tol = np.zeros_like(wq)
        tol[tk, cols] = _dot_tol(S.bf16_to_float(gy)[tk].astype(np.float64),
                                 S.bf16_to_float(Y)[rt["row_id"][tk, jk]].astype(np.float64), H)
        assert np.all(np.abs(gq_h.astype(np.float64) - wq) <= tol + 2.0 ** -24 * np.abs(wq))
        off = np.ones(wq.shape, bool)
        off[tk, cols] = False
        assert not gq_h[off].any()          # unrouted / dropped entries are 0


def test_backward_full_size_sampled():
    """8192 x 7168 bf16, 256 experts top-8 sigmoid routing, padding 128: the
    whole backward runs at full size; sampled tokens are checked against the
    oracle on the rows they touch."""
    c = S.CONFIGS["dsv3_layer_8192x7168_e256"]
    idx, pr = S.route_sigmoid_topk(c.T, c.E, c.K, c.seed)
    log("backward full size")
    d = Dispatcher(c.T, c.H, c.E, c.K, pad_multiple=c.pad)
    d.preprocess(dev(idx), dev(pr))
    g = torch.Generator(device=DEV)
    g.manual_seed(c.seed + 50)
    G = torch.randn((d.R, c.H), generator=g, device=DEV).to(torch.bfloat16)
    Y = torch.randn((d.R, c.H), generator=g, device=DEV).to(torch.bfloat16)
    gy = torch.randn((c.T, c.H), generator=g, device=DEV).to(torch.bfloat16)
    gop = torch.randn(d.R, generator=g, device=DEV)
    gx, gp = d.dispatch_backward(G, gop)
    gY, gq = d.combine_backward(gy, Y, True)
    torch.cuda.synchronize()

    rt = oracle.route(idx, 0, c.E, c.K, pr, c.pad, -1, d.R)
    assert np.array_equal(d.row_id.cpu().numpy(), rt["row_id"])
    sample = np.sort(np.random.default_rng(3).choice(c.T, 48, replace=False))
    # compact sub-problem: the sampled tokens and the rows of their copies
    rid = rt["row_id"][sample]
    keep = rid >= 0
    rows = rid[keep]
    sub_rid = np.full(rid.shape, -1, np.int32)
    sub_rid[keep] = np.arange(keep.sum(), dtype=np.int32)
    sub = dict(row_id=sub_rid, copy_expert=rt["copy_expert"][sample], copy_prob=rt["copy_prob"][sample])
    rows_t = torch.from_numpy(rows.astype(np.int64)).to(DEV)
    G_s = host_bf16(G.index_select(0, rows_t))
    Y_s = host_bf16(Y.index_select(0, rows_t))
    gy_s = host_bf16(gy[torch.from_numpy(sample).to(DEV)])
    gop_s = gop.index_select(0, rows_t).cpu().numpy()

    wx, wp = oracle.dispatch_backward(G_s, sub, c.E, False, gop_s)
    gx_s = host_bf16(gx)[sample]
    assert _ulp_diff(gx_s, wx).max() <= 1 and (gx_s == wx).mean() > 0.999
    assert np.array_equal(gp.cpu().numpy()[sample].view(np.uint32), wp.view(np.uint32))

    wY, wq = oracle.combine_backward(gy_s, Y_s, sub, c.E, False, True)
    assert np.array_equal(host_bf16(gY.index_select(0, rows_t)), wY)
    tol = np.zeros_like(wq)
    tol[keep] = _dot_tol(S.bf16_to_float(gy_s).astype(np.float64)[np.nonzero(keep)[0]],
                         S.bf16_to_float(Y_s).astype(np.float64), c.H)
    gq_s = gq.cpu().numpy()[sample].astype(np.float64)
    assert np.all(np.abs(gq_s - wq) <= tol + 2.0 ** -24 * np.abs(wq))


def test_backward_graph_replay_matches_eager():
    """dispatch_backward + combine_backward (Boolean-map routing, so the
    probability tables are cleared by the fill kernel) captured in one HIP
    graph and replayed with new gradients, each replay checked against the
    eager result."""
    T, H, E, K = 300, 1024, 16, 4
    routing, probs = _routing(T, E, K, oracle.FMT_SPARSE_U8, 91)
    d = Dispatcher(T, H, E, K, route_fmt="sparse_bool", pad_multiple=8)
    d.preprocess(dev(routing), dev(probs))
    G = torch.empty((d.R, H), dtype=torch.bfloat16, device=DEV)
    Y = dev(S.bf16_normal((d.R, H), 92))
    gy = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    gop = torch.empty(d.R, dtype=torch.float32, device=DEV)
    gx = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    gp = torch.empty((T, E), dtype=torch.float32, device=DEV)
    gY = torch.empty((d.R, H), dtype=torch.bfloat16, device=DEV)
    gq = torch.empty((T, E), dtype=torch.float32, device=DEV)

    def step():
        d.dispatch_backward(G, gop, out=gx, grad_probs=gp)
        d.combine_backward(gy, Y, True, out=gY, grad_probs=gq)
        assert_no_overflow(d.flag)            # captured; the forward routing fits

    def fill(i):
        G.copy_(dev(S.bf16_normal((d.R, H), 100 + i)))
        gy.copy_(dev(S.bf16_normal((T, H), 200 + i)))
        gop.copy_(torch.from_numpy(np.random.default_rng(300 + i).standard_normal(d.R).astype(np.float32)))

    log("backward graph replay")
    torch.cuda.synchronize()
    assert int(d.flag.item()) == 0                                   # before any step with the device assert
    fill(0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    rows = d.src_row >= 0
    for i in range(1, 4):
        fill(i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (gx.clone(), gp.clone(), gY[rows].clone(), gq.clone())
        step()                                        # eager on the same inputs
        torch.cuda.synchronize()
        assert torch.equal(got[0], gx) and torch.equal(got[1], gp), i
        assert torch.equal(got[2], gY[rows]) and torch.equal(got[3], gq), i
