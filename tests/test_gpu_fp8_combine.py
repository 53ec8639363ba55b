"""The fp8 combine format on the GPU: FC2 writes e4m3 codes with 1x128 scales,
the combine dequantises.  FC2's codes and scales are checked against the
oracle's quantiser applied to the oracle's float32 FC2 sums.  Both take the
quantisation decision in fp32, but on FC2 sums that already differ by the
MLP's own rounding (the activations are bf16 values computed in different
orders), so the bar is the MLP's: dequantised rows and scales within 1e-2.
The combine is checked against the oracle on the GPU's own codes."""
import numpy as np
import pytest
import torch

import moe_synth as S
import oracle
from combine_routing_preprocess_amd import Dispatcher, assert_no_overflow
from gpu_util import DEV, dev, host_bf16, log, rel_l2, row_rel_l2

pytestmark = pytest.mark.gpu


def _deq(q, s):
    return torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).to(torch.float64).numpy() \
        * np.repeat(np.asarray(s, np.float64), 128, axis=1)


def _small_layer():
    c = S.CONFIGS["small_layer_512x1024"]
    idx, pr = S.route_softmax_topk(c.T, c.E, c.K, c.seed)
    x = S.bf16_normal((c.T, c.H), c.seed)
    w1 = S.bf16_normal((c.E, 2 * c.F, c.H), c.seed + 1, std=0.02)
    w2 = S.bf16_normal((c.E, c.H, c.F), c.seed + 2, std=0.02)
    return c, idx, pr, x, w1, w2


def test_fc2_fp8out_and_combine_small_layer():
    c, idx, pr, x, w1, w2 = _small_layer()
    log("fp8 combine format, small layer")
    d = Dispatcher(c.T, c.H, c.E, c.K, pad_multiple=c.pad)
    perm, *_ = d.dispatch(dev(x), dev(idx), dev(pr))
    scratch = d.alloc_mlp_scratch(c.F)
    W1, W2 = dev(w1), dev(w2)
    d.fc1(perm, W1, scratch)
    yb = torch.empty((d.R, c.H), dtype=torch.bfloat16, device=DEV)
    d.fc2(W2, scratch, yb)
    q, s = d.fc2_fp8out(W2, scratch)
    out = d.combine_fp8(q, s)
    out0 = d.combine_fp8(q, s, apply_probs=False)
    torch.cuda.synchronize()

    rt = oracle.route(idx, 0, c.E, c.K, pr, c.pad, -1, d.R)
    P = oracle.permute_rows(x, rt["row_id"], d.R)
    qh, sh = q.cpu().numpy(), s.cpu().numpy()
    for e in range(c.E):
        s0, k = int(rt["seg_off"][e]), int(rt["counts"][e])
        if k == 0:
            continue
        _, y32 = oracle.expert_mlp_bf16(P[s0:s0 + k], w1[e], w2[e], return_y32=True)
        wq, ws = oracle.quant_rows_e4m3(y32)
        gq, gs = qh[s0:s0 + k], sh[s0:s0 + k]
        assert np.all(np.abs(gs / ws - 1.0) <= 1e-2), e
        assert rel_l2(_deq(gq, gs), _deq(wq, ws)) < 1e-2, e
        assert row_rel_l2(_deq(gq, gs), _deq(wq, ws)).max() < 5e-2, e
    # against FC2's bf16 output of the same run: fp8 rounding only
    rows = np.nonzero(rt["src_row"] >= 0)[0]
    yb_f = S.bf16_to_float(host_bf16(yb)[rows]).astype(np.float64)
    assert rel_l2(_deq(qh[rows], sh[rows]), yb_f) < 2.0 ** -4
    # combine on the GPU's own codes
    for got, apply in ((out, True), (out0, False)):
        want = oracle.combine_fp8(qh, sh, rt["row_id"], rt["copy_prob"], apply)
        g = host_bf16(got)
        assert row_rel_l2(S.bf16_to_float(g), S.bf16_to_float(want)).max() < 1e-2
        assert np.mean(g == want) > 0.99


@pytest.mark.parametrize("T,H,E,K", [(0, 256, 4, 2), (1, 128, 1, 1), (37, 1152, 6, 3)])
def test_combine_fp8_edges(T, H, E, K):
    """Empty batch, a single token, a row whose 72 chunks are not a multiple
    of a wavefront's 128; random codes and scales, dropped copies."""
    r = np.random.default_rng(T + H)
    idx = np.argsort(r.random((T, E)), axis=1)[:, :K].astype(np.int16)
    pr = r.random((T, K)).astype(np.float32)
    d = Dispatcher(T, H, E, K, capacity=max(1, T * K // E - 1))
    d.preprocess(dev(idx), dev(pr))
    rt = oracle.route(idx, 0, E, K, pr, 1, max(1, T * K // E - 1), d.R)
    v = (r.standard_normal((d.R, H)) * 3).astype(np.float32)
    q, s = oracle.quant_rows_e4m3(v)
    log("combine fp8 edges", T, H, E, K)
    y = d.combine_fp8(dev(q), dev(s))
    torch.cuda.synchronize()
    want = oracle.combine_fp8(q, s, rt["row_id"], rt["copy_prob"])
    g = host_bf16(y)
    assert g.shape == want.shape
    if T:
        assert row_rel_l2(S.bf16_to_float(g), S.bf16_to_float(want)).max() < 1e-2
        assert np.mean(g == want) > 0.99


def test_fp8_combine_format_full_size_sampled():
    """8192 x 7168, 256 experts top-8, FFN 2048: FC2 into the fp8 format
    agrees with FC2's bf16 output up to fp8 rounding at full size, and the
    combine of sampled tokens matches the oracle on the GPU's codes."""
    c = S.CONFIGS["dsv3_layer_8192x7168_e256"]
    idx, pr = S.route_sigmoid_topk(c.T, c.E, c.K, c.seed)
    x = torch.from_numpy(S.bf16_normal((c.T, c.H), c.seed).view(np.int16)).to(DEV).view(torch.bfloat16)
    w1 = S.weights_bf16(c.E, 2 * c.F, c.H, c.seed + 1, device=DEV)
    w2 = S.weights_bf16(c.E, c.H, c.F, c.seed + 2, device=DEV)
    log("fp8 combine format, full size")
    d = Dispatcher(c.T, c.H, c.E, c.K, pad_multiple=c.pad)
    perm, *_ = d.dispatch(x, dev(idx), dev(pr))
    scratch = d.alloc_mlp_scratch(c.F)
    d.fc1(perm, w1, scratch)
    yb = torch.empty((d.R, c.H), dtype=torch.bfloat16, device=DEV)
    d.fc2(w2, scratch, yb)
    q, s = d.fc2_fp8out(w2, scratch)
    y = d.combine_fp8(q, s)
    torch.cuda.synchronize()
    rows = torch.nonzero(d.src_row >= 0).flatten()
    deq = q[rows].view(torch.float8_e4m3fn).to(torch.float32) * s[rows].repeat_interleave(128, dim=1)
    ref = yb[rows].to(torch.float32)
    assert float(torch.linalg.norm(deq - ref) / torch.linalg.norm(ref)) < 2.0 ** -4

    rt = oracle.route(idx, 0, c.E, c.K, pr, c.pad, -1, d.R)
    sample = np.sort(np.random.default_rng(5).choice(c.T, 48, replace=False))
    rid = rt["row_id"][sample]
    keep = rid >= 0
    sub_rid = np.full(rid.shape, -1, np.int32)
    sub_rid[keep] = np.arange(keep.sum(), dtype=np.int32)
    rows_t = torch.from_numpy(rid[keep].astype(np.int64)).to(DEV)
    want = oracle.combine_fp8(q.index_select(0, rows_t).cpu().numpy(), s.index_select(0, rows_t).cpu().numpy(),
                              sub_rid, rt["copy_prob"][sample])
    g = host_bf16(y)[sample]
    assert row_rel_l2(S.bf16_to_float(g), S.bf16_to_float(want)).max() < 1e-2
    assert np.mean(g == want) > 0.99


def test_fp8_formats_graph_replay_matches_eager():
    """Quantise-on-dispatch, FC2 into the fp8 format and the fp8 combine (and
    the bf16 FC1 between them) captured in one graph; every replay with new
    tokens equals the eager result."""
    c, idx, pr, x, w1, w2 = _small_layer()
    W1, W2 = dev(w1), dev(w2)
    d = Dispatcher(c.T, c.H, c.E, c.K, pad_multiple=c.pad)
    dq = Dispatcher(c.T, c.H, c.E, c.K, payload="fp8", pad_multiple=c.pad)
    rt, pt = dev(idx), dev(pr)
    d.preprocess(rt, pt)
    dq.preprocess(rt, pt)
    xt = torch.empty((c.T, c.H), dtype=torch.bfloat16, device=DEV)
    perm = torch.empty((d.R, c.H), dtype=torch.bfloat16, device=DEV)
    pq = torch.empty((dq.R, c.H), dtype=torch.uint8, device=DEV)
    ps = torch.empty((dq.R, c.H // 128), dtype=torch.float32, device=DEV)
    scr = d.alloc_mlp_scratch(c.F)
    eq = torch.empty((d.R, c.H), dtype=torch.uint8, device=DEV)
    es = torch.empty((d.R, c.H // 128), dtype=torch.float32, device=DEV)
    y = torch.empty((c.T, c.H), dtype=torch.bfloat16, device=DEV)

    def step():
        dq.permute_quantize(xt, out=pq, out_scales=ps)
        d.permute(xt, out=perm)
        d.fc1(perm, W1, scr)
        d.fc2_fp8out(W2, scr, out=eq, out_scales=es)
        d.combine_fp8(eq, es, out=y)
        assert_no_overflow(d.flag)            # captured; the routing above fits
        assert_no_overflow(dq.flag)

    log("fp8 formats graph replay")
    torch.cuda.synchronize()
    assert int(d.flag.item()) == 0 and int(dq.flag.item()) == 0     # before any step with the device assert
    xt.copy_(dev(x))
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
        xt.copy_(dev(S.bf16_normal((c.T, c.H), 400 + i)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (pq[rows].clone(), ps[rows].clone(), eq[rows].clone(), es[rows].clone(), y.clone())
        step()
        torch.cuda.synchronize()
        assert torch.equal(got[0], pq[rows]) and torch.equal(got[1], ps[rows]), i
        assert torch.equal(got[2], eq[rows]) and torch.equal(got[3], es[rows]), i
        assert torch.equal(got[4], y), i
