"""Permute (K2) and combine (K5) on the GPU against the oracle.  Permuted
payload rows (bf16 and fp8 + scales) must match byte for byte; combine must
agree within 1e-2 relative and reproduce the input exactly in the identity
cases the oracle proves exact."""
import numpy as np
import pytest
import torch

import moe_synth as S
import oracle
from combine_routing_preprocess_amd import Dispatcher
from gpu_util import DEV, dev, host_bf16, log, rel_l2, row_rel_l2

pytestmark = pytest.mark.gpu


def _kept_rows(src_row):
    return np.nonzero(src_row >= 0)[0]


@pytest.mark.parametrize("T,H,E,K,pad,cap,fmt", [
    (1, 8, 1, 1, 1, -1, 0), (70, 64, 5, 3, 4, -1, 0), (300, 1024, 16, 4, 32, -1, 1),
    (129, 512, 8, 8, 1, 20, 2), (0, 256, 4, 2, 1, -1, 0), (1000, 2056, 12, 3, 7, 200, 0),
])
def test_permute_bf16_small(T, H, E, K, pad, cap, fmt):
    r = np.random.default_rng(T + H)
    if fmt == 2:
        routing = (r.random((T, E)) < 0.5).astype(np.uint8)
    else:
        routing = np.argsort(r.random((T, E)), axis=1)[:, :K].astype(np.int16 if fmt == 0 else np.int32)
    x = S.bf16_normal((T, H), T + 5)
    log("permute small", T, H, E, K, pad, cap, fmt)
    d = Dispatcher(T, H, E, K, route_fmt={0: "dense_i16", 1: "dense_i32", 2: "sparse_bool"}[fmt], pad_multiple=pad,
                   capacity=None if cap < 0 else cap)
    guard = torch.full((d.R + 3, H), 1.5, dtype=torch.bfloat16, device=DEV)   # 3 canary rows after R
    out, _, flag, _, _ = d.dispatch(dev(x), dev(routing), out=guard[:d.R])
    torch.cuda.synchronize()
    rt = oracle.route(routing, fmt, E, K, None, pad, cap, d.R)
    want = oracle.permute_rows(x, rt["row_id"], d.R)
    got = host_bf16(guard)
    rows = _kept_rows(rt["src_row"])
    assert np.array_equal(got[rows], want[rows])
    assert np.all(got[d.R:] == 0x3FC0)          # canaries untouched
    assert int(flag.item()) == rt["flag"]


def test_permute_and_combine_identity_full_size():
    """8192 x 7168 bf16, 32 experts, top-8 uniform routing, softmax probs,
    capacity 1.5x the largest count: byte-exact permute; identity experts and
    probabilities summing to 1 give back x exactly."""
    c = S.CONFIGS["permute_combine_8192x7168_e32"]
    idx, pr = S.route_uniform_distinct(c.T, c.E, c.K, c.seed)
    base = oracle.route(idx, 0, c.E, c.K, pr)
    cap = oracle.capacity_from_rows(int(base["counts"].max()), 1.5)
    x = S.bf16_normal((c.T, c.H), c.seed)
    log("permute+combine, 32-expert shape", cap)
    d = Dispatcher(c.T, c.H, c.E, c.K, capacity=cap)
    xd = dev(x)
    out_probs = torch.empty(d.R, dtype=torch.float32, device=DEV)
    perm, tpe, flag, _, _ = d.dispatch(xd, dev(idx), dev(pr), out_probs=out_probs)
    y = d.combine(perm)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    rt = oracle.route(idx, 0, c.E, c.K, pr, 1, cap, d.R)
    assert np.array_equal(tpe.cpu().numpy(), rt["counts"])
    want = oracle.permute_rows(x, rt["row_id"], d.R)
    rows = _kept_rows(rt["src_row"])
    got = host_bf16(perm)
    assert np.array_equal(got[rows], want[rows])
    assert np.array_equal(out_probs.cpu().numpy().view(np.uint32), rt["perm_prob"].view(np.uint32))
    yo = oracle.combine_bf16(want, rt["row_id"], rt["copy_prob"])
    assert np.array_equal(yo, x)                      # oracle: exact identity
    assert np.array_equal(host_bf16(y), x)            # GPU: exact identity


def test_combine_weighted_matches_oracle():
    """Random expert outputs (not identity), probabilities, dropped copies."""
    c = S.CONFIGS["permute_combine_8192x7168_e32"]
    T = 2048
    idx, pr = S.route_uniform_distinct(T, c.E, c.K, 5)
    base = oracle.route(idx, 0, c.E, c.K, pr)
    cap = int(base["counts"].max()) - 40            # force dropped copies
    d = Dispatcher(T, c.H, c.E, c.K, capacity=cap)
    log("combine weighted", cap)
    d.preprocess(dev(idx), dev(pr))
    Y = S.bf16_normal((d.R, c.H), 6)
    y = d.combine(dev(Y))
    y0 = d.combine(dev(Y), apply_probs=False)
    torch.cuda.synchronize()
    assert int(d.flag.item()) & oracle.FLAG_CAPACITY
    rt = oracle.route(idx, 0, c.E, c.K, pr, 1, cap, d.R)
    assert np.array_equal(d.row_id.cpu().numpy(), rt["row_id"])
    for apply, got in ((True, y), (False, y0)):
        want = oracle.combine_bf16(Y, rt["row_id"], rt["copy_prob"], apply)
        g = S.bf16_to_float(host_bf16(got))
        w = S.bf16_to_float(want)
        assert rel_l2(g, w) < 1e-2
        assert row_rel_l2(g, w).max() < 1e-2
        assert np.mean(host_bf16(got) == want) > 0.99
    # tokens that lost every copy come out as exact zeros
    lost = np.nonzero((rt["row_id"] < 0).all(axis=1))[0]
    assert np.all(host_bf16(y)[lost] & 0x7FFF == 0)


def test_combine_top1_is_exact_inverse():
    T, H, E = 777, 1024, 9
    idx = np.random.default_rng(4).integers(0, E, (T, 1)).astype(np.int16)
    x = S.bf16_normal((T, H), 8)
    log("combine top1")
    d = Dispatcher(T, H, E, 1, pad_multiple=5)
    perm, *_ = d.dispatch(dev(x), dev(idx))
    y = d.combine(perm, apply_probs=False)
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16(y), x)


@pytest.mark.parametrize("fmt", [oracle.FMT_DENSE_I16, oracle.FMT_SPARSE_U8])
def test_permute_fp8_stress_full_size(fmt):
    """8192 x 7168 e4m3 payload with per-128-column scales, 256 experts,
    top-36 Zipf routing; dense and sparse encodings give byte-identical output."""
    c = S.CONFIGS["route_stress_fp8_8192x7168_e256"]
    idx, pr = S.route_zipf_gumbel(c.T, c.E, c.K, c.seed)
    routing = idx if fmt == oracle.FMT_DENSE_I16 else S.dense_to_sparse(idx, c.E)[0]
    xq, xs = S.quantize_rows_fp8_torch(S.bf16_normal((c.T, c.H), c.seed))
    log("permute fp8, routing stress", fmt)
    d = Dispatcher(c.T, c.H, c.E, c.K, route_fmt="dense_i16" if fmt == 0 else "sparse_bool", payload="fp8")
    out, _, flag, _, osc = d.dispatch(dev(xq), dev(routing), x_scales=dev(xs))
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    rt = oracle.route(routing, fmt, c.E, c.K, None, 1, -1, d.R)
    rows = _kept_rows(rt["src_row"])
    assert len(rows) == c.T * c.K
    got = out.cpu().numpy()
    want = oracle.permute_rows(xq, rt["row_id"], d.R)
    assert np.array_equal(got[rows], want[rows])
    wsc = oracle.permute_rows(xs, rt["row_id"], d.R)
    assert np.array_equal(osc.cpu().numpy()[rows].view(np.uint32), wsc[rows].view(np.uint32))


@pytest.mark.parametrize("T,H,E,K", [(5, 2056, 7, 3), (16, 7168, 256, 8), (33, 1000, 9, 4)])
def test_combine_small_batch_column_slices(T, H, E, K):
    """Few tokens: each row is cut into column slices over several wavefronts
    (the last slice can be a single 16-byte chunk); weighted combine must
    still match the oracle, and dispatch + identity combine must round-trip."""
    r = np.random.default_rng(T * 31 + H)
    idx = np.argsort(r.random((T, E)), axis=1)[:, :K].astype(np.int16)
    lg = r.standard_normal((T, K))
    pr = (np.exp(lg) / np.exp(lg).sum(axis=1, keepdims=True)).astype(np.float32)
    log("combine small slices", T, H, E, K)
    d = Dispatcher(T, H, E, K, pad_multiple=3)
    d.preprocess(dev(idx), dev(pr))
    Y = S.bf16_normal((d.R, H), T + 77)
    y = d.combine(dev(Y))
    x = S.bf16_normal((T, H), T + 78)
    perm, *_ = d.dispatch(dev(x), dev(idx), dev(pr))
    yi = d.combine(perm)
    torch.cuda.synchronize()
    rt = oracle.route(idx, 0, E, K, pr, 3, -1, d.R)
    want = oracle.combine_bf16(Y, rt["row_id"], rt["copy_prob"])
    g, w = S.bf16_to_float(host_bf16(y)), S.bf16_to_float(want)
    assert row_rel_l2(g, w).max() < 1e-2
    assert np.mean(host_bf16(y) == want) > 0.99
    # probabilities sum to 1 and every copy survives: the weighted sum rounds back to x
    assert np.array_equal(host_bf16(yi), x)


@pytest.mark.parametrize("T,H,E,K", [(7, 1152, 6, 3), (1, 7168, 256, 8)])
def test_permute_fp8_small_batch(T, H, E, K):
    """fp8 rows with scales at batch sizes that split rows into slices."""
    r = np.random.default_rng(T + 2 * H)
    idx = np.argsort(r.random((T, E)), axis=1)[:, :K].astype(np.int16)
    xq, xs = S.quantize_rows_fp8_torch(S.bf16_normal((T, H), T + 9))
    log("permute fp8 small", T, H, E, K)
    d = Dispatcher(T, H, E, K, payload="fp8", pad_multiple=4)
    out, _, flag, _, osc = d.dispatch(dev(xq), dev(idx), x_scales=dev(xs))
    torch.cuda.synchronize()
    rt = oracle.route(idx, 0, E, K, None, 4, -1, d.R)
    rows = _kept_rows(rt["src_row"])
    assert np.array_equal(out.cpu().numpy()[rows], oracle.permute_rows(xq, rt["row_id"], d.R)[rows])
    wsc = oracle.permute_rows(xs, rt["row_id"], d.R)
    assert np.array_equal(osc.cpu().numpy()[rows].view(np.uint32), wsc[rows].view(np.uint32))
    assert int(flag.item()) == 0


@pytest.mark.parametrize("T,H", [(4096, 1000), (4097, 2056), (5000, 520)])
def test_workgroup_per_token_ragged_rows(T, H):
    """At 4096 tokens and more, permute and combine take one workgroup per
    token with 1 KB pieces dealt to its wavefronts in turn.  Row widths whose
    last piece is partial (H/8 chunks not a multiple of 64), with capacity
    drops: permuted rows byte-exact, weighted combine against the oracle,
    dispatch + identity combine round-trips the kept tokens."""
    E, K, cap = 9, 3, None
    r = np.random.default_rng(T + H)
    idx = np.argsort(r.random((T, E)), axis=1)[:, :K].astype(np.int16)
    lg = r.standard_normal((T, K))
    pr = (np.exp(lg) / np.exp(lg).sum(axis=1, keepdims=True)).astype(np.float32)
    cap = int(T * K / E * 0.98)                     # a few copies dropped
    x = S.bf16_normal((T, H), T + 5)
    log("workgroup per token, ragged", T, H, cap)
    d = Dispatcher(T, H, E, K, pad_multiple=2, capacity=cap)
    perm, *_ = d.dispatch(dev(x), dev(idx), dev(pr))
    Y = S.bf16_normal((d.R, H), T + 6)
    y = d.combine(dev(Y))
    yi = d.combine(perm)
    torch.cuda.synchronize()
    rt = oracle.route(idx, 0, E, K, pr, 2, cap, d.R)
    rows = _kept_rows(rt["src_row"])
    assert np.array_equal(host_bf16(perm)[rows], oracle.permute_rows(x, rt["row_id"], d.R)[rows])
    want = oracle.combine_bf16(Y, rt["row_id"], rt["copy_prob"])
    g, w = S.bf16_to_float(host_bf16(y)), S.bf16_to_float(want)
    assert row_rel_l2(g, w).max() < 1e-2
    assert np.mean(host_bf16(y) == want) > 0.99
    full = (rt["row_id"] >= 0).all(axis=1)          # tokens with every copy kept
    assert np.array_equal(host_bf16(yi)[full], x[full])


@pytest.mark.parametrize("T,H", [(4096, 1152), (4100, 1920)])
def test_workgroup_per_token_fp8_ragged_rows(T, H):
    """fp8 rows (H/16 chunks, not a multiple of 64) through the workgroup-per-
    token permute (codes and scales byte-exact) and the fp8 combine format's
    workgroup-per-token combine (against the oracle on the same codes)."""
    E, K = 6, 2
    r = np.random.default_rng(T * 3 + H)
    idx = np.argsort(r.random((T, E)), axis=1)[:, :K].astype(np.int16)
    pr = np.full((T, K), 0.5, np.float32)
    xq, xs = S.quantize_rows_fp8_torch(S.bf16_normal((T, H), T + 8))
    log("workgroup per token, fp8 ragged", T, H)
    d = Dispatcher(T, H, E, K, payload="fp8", pad_multiple=4)
    out, _, flag, _, osc = d.dispatch(dev(xq), dev(idx), dev(pr), x_scales=dev(xs))
    torch.cuda.synchronize()
    rt = oracle.route(idx, 0, E, K, pr, 4, -1, d.R)
    rows = _kept_rows(rt["src_row"])
    assert np.array_equal(out.cpu().numpy()[rows], oracle.permute_rows(xq, rt["row_id"], d.R)[rows])
    wsc = oracle.permute_rows(xs, rt["row_id"], d.R)
    assert np.array_equal(osc.cpu().numpy()[rows].view(np.uint32), wsc[rows].view(np.uint32))
    assert int(flag.item()) == 0
    # the permuted codes and scales are a valid fp8 combine input
    yc = d.combine_fp8(out, osc)
    torch.cuda.synchronize()
    want = oracle.combine_fp8(out.cpu().numpy(), osc.cpu().numpy(), rt["row_id"], rt["copy_prob"])
    g = host_bf16(yc)
    assert row_rel_l2(S.bf16_to_float(g), S.bf16_to_float(want)).max() < 1e-2
    assert np.mean(g == want) > 0.99


def test_empty_batch():
    log("empty batch")
    d = Dispatcher(0, 256, 8, 2, pad_multiple=16)
    x = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    idx = torch.empty((0, 2), dtype=torch.int16, device=DEV)
    perm, tpe, flag, _, _ = d.dispatch(x, idx)
    y = d.combine(torch.empty((d.R, 256), dtype=torch.bfloat16, device=DEV))
    torch.cuda.synchronize()
    assert d.R == 8 * 15 and int(flag.item()) == 0 and tpe.sum().item() == 0 and y.shape == (0, 256)
    assert int(d.rows_needed.item()) == 0
