"""Quantise-on-dispatch on the GPU against the oracle: bf16 token rows are
quantised per 1x128 block inside the permute; codes and scales must match
the oracle's quantiser followed by its permute byte for byte, and rows
quantised this way must drive the fp8 expert MLP to exactly the result of
the bf16 dispatch (which quantises the same rows inside the MLP)."""
import numpy as np
import pytest
import torch

import moe_synth as S
import oracle
from combine_routing_preprocess_amd import Dispatcher
from gpu_util import DEV, FMT_NAME, dev, host_bf16, log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,H,E,K,pad,cap,fmt", [
    (70, 128, 5, 3, 4, -1, oracle.FMT_DENSE_I16),
    (300, 1152, 16, 4, 16, -1, oracle.FMT_SPARSE_U8),     # 9 column blocks: a ragged block group
    (129, 7168, 8, 8, 1, 20, oracle.FMT_DENSE_I32),       # capacity drops
    (1, 256, 1, 1, 1, -1, oracle.FMT_DENSE_I16),
    (0, 256, 4, 2, 1, -1, oracle.FMT_DENSE_I16),
])
def test_permute_quantize_matches_oracle(T, H, E, K, pad, cap, fmt):
    r = np.random.default_rng(T + H)
    if fmt == oracle.FMT_SPARSE_U8:
        routing = (r.random((T, E)) < 0.3).astype(np.uint8)
    else:
        routing = np.argsort(r.random((T, E)), axis=1)[:, :K].astype(np.int16 if fmt == 0 else np.int32)
    x = S.bf16_normal((T, H), T + 7)
    if T > 2:
        x[1] = 0                                    # an all-zero row: scale 1, zero codes
        x[2, :128] = S.bf16_normal((1, 128), 9, std=1e3)[0]   # large values saturate nothing (scale absorbs)
    log("permute_quantize", T, H, E, K, pad, cap, fmt)
    d = Dispatcher(T, H, E, K, route_fmt=FMT_NAME[fmt], payload="fp8", pad_multiple=pad,
                   capacity=None if cap < 0 else cap)
    d.preprocess(dev(routing))
    q_guard = torch.full((d.R + 2, H), 0x5A, dtype=torch.uint8, device=DEV)
    s_guard = torch.full((d.R + 2, H // 128), -7.0, dtype=torch.float32, device=DEV)
    d.permute_quantize(dev(x), out=q_guard[:d.R], out_scales=s_guard[:d.R])
    torch.cuda.synchronize()
    rt = oracle.route(routing, fmt, E, K, None, pad, cap, d.R)
    xq, xs = oracle.quant_rows_e4m3(S.bf16_to_float(x))
    want_q = oracle.permute_rows(xq, rt["row_id"], d.R)
    want_s = oracle.permute_rows(xs, rt["row_id"], d.R)
    rows = np.nonzero(rt["src_row"] >= 0)[0]
    got_q = q_guard.cpu().numpy()
    got_s = s_guard.cpu().numpy()
    assert np.array_equal(got_q[rows], want_q[rows])
    assert np.array_equal(got_s[rows].view(np.uint32), want_s[rows].view(np.uint32))
    assert np.all(got_q[d.R:] == 0x5A) and np.all(got_s[d.R:] == -7.0)


@pytest.mark.parametrize("T", [16, 100])
def test_quantized_dispatch_feeds_fp8_mlp(T):
    """fp8 weights: dispatching bf16 rows (quantised inside FC1) and
    dispatching rows quantised on the way give bit-identical layers."""
    E, K, H, F = 16, 4, 1024, 256
    idx, pr = S.route_sigmoid_topk(T, E, K, 300 + T)
    x = dev(S.bf16_normal((T, H), 301 + T))
    w1q, w1s = S.weights_fp8_blocks(E, 2 * F, H, 302, device=DEV)
    w2q, w2s = S.weights_fp8_blocks(E, H, F, 303, device=DEV)
    log("quantised dispatch -> fp8 mlp", T)
    a = Dispatcher(T, H, E, K, pad_multiple=16)
    perm, *_ = a.dispatch(x, dev(idx), dev(pr))
    ya = a.grouped_mlp(perm, w1q, w2q, w1_scales=w1s, w2_scales=w2s)
    oa = a.combine(ya)
    b = Dispatcher(T, H, E, K, payload="fp8", pad_multiple=16)
    b.preprocess(dev(idx), dev(pr))
    q, qs = b.permute_quantize(x)
    yb = b.grouped_mlp(q, w1q, w2q, w1_scales=w1s, w2_scales=w2s, perm_scales=qs)
    ob = b.combine(yb)
    torch.cuda.synchronize()
    rows = (a.src_row >= 0)
    assert torch.equal(b.src_row, a.src_row)
    assert torch.equal(ya[rows], yb[rows])
    assert torch.equal(oa, ob)
