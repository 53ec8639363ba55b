"""Pins for the oracle's dispatch and combine backward functions.

The forward operations are restated with torch index operations in float64
and differentiated by torch.autograd, an implementation independent of the
oracle's loops; special cases reduce to a plain gather and to the (separately
pinned) permute.  CPU only."""
import numpy as np
import pytest
import torch

import moe_synth as S
import oracle


def _f(bits):
    return S.bf16_to_float(bits).astype(np.float64)


def _bf16_torch(v64):
    return torch.from_numpy(np.asarray(v64, np.float64)).to(torch.float32).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _nearest_ok(got_bits, exact):
    """got is a bf16 value at least as close to `exact` as torch's rounding of
    it (float64 -> float32 -> bf16, which can round twice), and equal to it
    almost everywhere."""
    want = _bf16_torch(exact)
    g, w = _f(got_bits), _f(want)
    ok = (got_bits == want) | (np.abs(g - exact) <= np.abs(w - exact))
    return bool(ok.all()) and float((got_bits == want).mean()) > 0.999


def _case(fmt, with_probs, cap, T=48, E=8, K=3, H=40, seed=21):
    idx, pr = S.route_softmax_topk(T, E, K, seed)
    idx = idx.copy()
    idx[3, 1] = -1                     # an empty slot
    idx[5, 2] = idx[5, 0]              # a duplicate (dropped by the routing)
    if fmt == oracle.FMT_SPARSE_U8:
        routing, probs = S.dense_to_sparse(idx, E, pr)
    else:
        routing, probs = idx, pr
    probs = probs if with_probs else None
    rt = oracle.route(routing, fmt, E, K, probs, pad=4, cap=cap)
    return routing, probs, rt


def _kept(rt):
    tk, jk = np.nonzero(rt["row_id"] >= 0)
    return tk, jk, rt["row_id"][tk, jk]


def _probs_param(probs, rt, fmt, tk, jk, E=8):
    """Probability tensor in the routing's shape (ones without probs) and the
    kept copies' entries of it, as an autograd leaf."""
    T, K = rt["row_id"].shape
    if probs is None:
        probs_shape = (T, E if fmt == oracle.FMT_SPARSE_U8 else K)
        p = torch.ones(probs_shape, dtype=torch.float64, requires_grad=True)
    else:
        p = torch.tensor(np.asarray(probs, np.float64), requires_grad=True)
    cols = rt["copy_expert"][tk, jk] if fmt == oracle.FMT_SPARSE_U8 else jk
    return p, p[torch.from_numpy(tk), torch.from_numpy(np.asarray(cols, np.int64))]


FMTS = [oracle.FMT_DENSE_I16, oracle.FMT_SPARSE_U8]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("with_probs", [True, False])
@pytest.mark.parametrize("cap", [-1, 11])
def test_dispatch_backward_matches_autograd(fmt, with_probs, cap):
    E, H = 8, 40
    routing, probs, rt = _case(fmt, with_probs, cap)
    T, K = rt["row_id"].shape
    R = rt["R"]
    tk, jk, rows = _kept(rt)
    if cap > 0:
        assert rt["flag"] & oracle.FLAG_CAPACITY and len(rows) < T * K - 2   # copies were dropped
    G = S.bf16_normal((R, H), 31)
    gop = np.random.default_rng(32).standard_normal(R).astype(np.float32)
    gx, gp = oracle.dispatch_backward(G, rt, E, fmt == oracle.FMT_SPARSE_U8, gop if with_probs else None)

    x = torch.zeros((T, H), dtype=torch.float64, requires_grad=True)
    p, p_sel = _probs_param(probs, rt, fmt, tk, jk)
    rows_t = torch.from_numpy(rows.astype(np.int64))
    out = torch.zeros((R, H), dtype=torch.float64).index_copy(0, rows_t, x[torch.from_numpy(tk)])
    out_p = torch.zeros(R, dtype=torch.float64).index_copy(0, rows_t, p_sel)
    loss = (out * torch.from_numpy(_f(G))).sum() + (out_p * torch.from_numpy(gop.astype(np.float64))).sum()
    loss.backward()
    assert _nearest_ok(gx, x.grad.numpy())
    if with_probs:
        assert gp.shape == tuple(p.shape)
        assert np.array_equal(gp.astype(np.float64), p.grad.numpy())
    else:
        assert gp is None


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("apply_probs", [True, False])
@pytest.mark.parametrize("cap", [-1, 11])
def test_combine_backward_matches_autograd(fmt, apply_probs, cap):
    E, H = 8, 40
    routing, probs, rt = _case(fmt, True, cap)
    T, K = rt["row_id"].shape
    R = rt["R"]
    tk, jk, rows = _kept(rt)
    Y = S.bf16_normal((R, H), 41)
    gy = S.bf16_normal((T, H), 42)
    gY, gp = oracle.combine_backward(gy, Y, rt, E, fmt == oracle.FMT_SPARSE_U8, apply_probs, fill=0x7FC1)

    Yt = torch.tensor(_f(Y), requires_grad=True)
    p, p_sel = _probs_param(probs, rt, fmt, tk, jk)
    w = p_sel if apply_probs else torch.ones_like(p_sel)
    y = torch.zeros((T, H), dtype=torch.float64).index_add(
        0, torch.from_numpy(tk), w[:, None] * Yt[torch.from_numpy(rows.astype(np.int64))])
    (y * torch.from_numpy(_f(gy))).sum().backward()
    g = Yt.grad.numpy()
    assert _nearest_ok(gY[rows], g[rows])
    untouched = np.ones(R, bool)
    untouched[rows] = False
    assert (gY[untouched] == 0x7FC1).all()
    want_p = p.grad.numpy() if p.grad is not None else np.zeros(tuple(p.shape))   # unused without probs
    assert gp.shape == want_p.shape
    if not apply_probs:
        assert not gp.any() and not want_p.any()
    else:
        # both are double sums of the same H products in different orders,
        # then the oracle rounds to float: within float rounding of each other
        mag = np.zeros_like(want_p)
        terms = np.abs(_f(gy)[tk] * _f(Y)[rows]).sum(axis=1)
        cols = rt["copy_expert"][tk, jk] if fmt == oracle.FMT_SPARSE_U8 else jk
        mag[tk, cols] = terms
        assert np.all(np.abs(gp - want_p) <= 2.0 ** -24 * np.abs(want_p) + 1e-12 * mag)
        assert np.count_nonzero(want_p) == len(rows)


def test_dispatch_backward_top1_is_a_gather():
    """With one copy per token and nothing dropped, the token gradient is the
    gradient row of its copy, bit for bit."""
    idx, pr = S.route_softmax_topk(64, 8, 1, 51)
    rt = oracle.route(idx, oracle.FMT_DENSE_I16, 8, 1, pr, pad=1)
    G = S.bf16_normal((rt["R"], 24), 52)
    gx, _ = oracle.dispatch_backward(G, rt, 8, False)
    assert np.array_equal(gx, G[rt["row_id"][:, 0]])


def test_combine_backward_without_probs_is_the_permute():
    """Without probabilities the row gradients are the token gradient copied
    to every kept copy's row: the forward permute of grad_y."""
    routing, probs, rt = _case(oracle.FMT_DENSE_I16, True, 11)
    gy = S.bf16_normal((rt["row_id"].shape[0], 40), 61)
    Y = S.bf16_normal((rt["R"], 40), 62)
    gY, gp = oracle.combine_backward(gy, Y, rt, 8, False, apply_probs=False, fill=3)
    assert np.array_equal(gY, oracle.permute_rows(gy, rt["row_id"], rt["R"], fill=3))
    assert not gp.any()


def test_backward_empty_batch():
    rt = oracle.route(np.zeros((0, 2), np.int16), oracle.FMT_DENSE_I16, 4, 2, None, pad=1)
    gx, gp = oracle.dispatch_backward(np.zeros((0, 8), np.uint16), rt, 4, False, np.zeros(0, np.float32))
    assert gx.shape == (0, 8) and gp.shape == (0, 2)
    gY, gp = oracle.combine_backward(np.zeros((0, 8), np.uint16), np.zeros((0, 8), np.uint16), rt, 4, False)
    assert gY.shape == (0, 8) and gp.shape == (0, 2)
