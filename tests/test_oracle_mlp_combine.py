"""Pins for the oracle's permute, combine and expert-MLP functions against
numpy / torch library routines, special cases and invariants.  CPU only."""
import numpy as np
import pytest
import torch

import moe_synth as S
import oracle


def _bf16(v64: np.ndarray) -> np.ndarray:
    """Reference bf16 rounding through torch (float64 -> float32 -> bf16)."""
    return torch.from_numpy(np.asarray(v64, np.float64)).to(torch.float32).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _f(bits):
    return S.bf16_to_float(bits).astype(np.float64)


def _rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30)


# ---- permute ---------------------------------------------------------------
def test_permute_matches_numpy_scatter():
    idx, pr = S.route_softmax_topk(64, 8, 3, 11)
    rt = oracle.route(idx, 0, 8, 3, pr, pad=4)
    x = S.bf16_normal((64, 48), 12)
    out = oracle.permute_rows(x, rt["row_id"], rt["R"], fill=0xFFFF)
    want = np.full((rt["R"], 48), 0xFFFF, np.uint16)
    m = rt["row_id"].reshape(-1) >= 0
    want[rt["row_id"].reshape(-1)[m]] = np.repeat(x, 3, axis=0)[m]
    assert np.array_equal(out, want)
    # fp8 payload and its scale rows travel together
    q = np.random.default_rng(0).integers(0, 256, (64, 256), dtype=np.uint8)
    sc = np.random.default_rng(1).random((64, 2)).astype(np.float32)
    oq = oracle.permute_rows(q, rt["row_id"], rt["R"])
    os_ = oracle.permute_rows(sc, rt["row_id"], rt["R"])
    for t in range(64):
        for j in range(3):
            r = rt["row_id"][t, j]
            assert np.array_equal(oq[r], q[t]) and np.array_equal(os_[r], sc[t])


# ---- combine ---------------------------------------------------------------
def test_combine_matches_numpy_weighted_gather():
    r = np.random.default_rng(5)
    T, K, H, R = 40, 4, 96, 200
    Y = S.bf16_normal((R, H), 6)
    rid = np.stack([r.choice(R, K, replace=False) for _ in range(T)]).astype(np.int32)
    rid[r.random((T, K)) < 0.2] = -1
    cp = r.random((T, K)).astype(np.float32)
    got = oracle.combine_bf16(Y, rid, cp)
    Yf = _f(Y)
    w = np.where(rid >= 0, cp.astype(np.float64), 0.0)
    acc = np.einsum("tk,tkh->th", w, Yf[np.maximum(rid, 0)])
    want = _bf16(acc)
    assert _rel_l2(_f(got), _f(want)) < 1e-3
    assert np.mean(got == want) > 0.99
    got1 = oracle.combine_bf16(Y, rid, cp, apply_probs=False)
    acc1 = np.einsum("tk,tkh->th", (rid >= 0).astype(np.float64), Yf[np.maximum(rid, 0)])
    assert np.mean(got1 == _bf16(acc1)) > 0.99


def test_combine_of_dispatch_with_identity_experts_is_the_input():
    """Identity experts and probabilities summing to 1: combine(dispatch(x)) = x."""
    T, E, K, H = 300, 16, 4, 64
    idx, _ = S.route_uniform_distinct(T, E, K, 21)
    lg = np.random.default_rng(22).standard_normal((T, K))
    p = np.exp(lg) / np.exp(lg).sum(1, keepdims=True)
    rt = oracle.route(idx, 0, E, K, p.astype(np.float32), pad=8)
    x = S.bf16_normal((T, H), 23)
    Y = oracle.permute_rows(x, rt["row_id"], rt["R"])
    assert np.array_equal(oracle.combine_bf16(Y, rt["row_id"], rt["copy_prob"]), x)


def test_combine_top1_without_probs_is_the_inverse_permutation():
    T, E, H = 100, 5, 32
    idx = np.random.default_rng(3).integers(0, E, (T, 1)).astype(np.int16)
    rt = oracle.route(idx, 0, E, 1, pad=3)
    x = S.bf16_normal((T, H), 4)
    Y = oracle.permute_rows(x, rt["row_id"], rt["R"])
    assert np.array_equal(oracle.combine_bf16(Y, rt["row_id"], rt["copy_prob"], apply_probs=False), x)


def test_combine_dropped_copies_add_zero():
    idx = np.array([[0, 1], [0, 1], [0, 1]], np.int16)
    pr = np.full((3, 2), 0.5, np.float32)
    rt = oracle.route(idx, 0, 2, 2, pr, cap=2)             # token 2 loses both copies
    x = S.bf16_normal((3, 16), 9)
    Y = oracle.permute_rows(x, rt["row_id"], rt["R"])
    y = oracle.combine_bf16(Y, rt["row_id"], rt["copy_prob"])
    assert np.array_equal(y[:2], x[:2]) and np.all(y[2] == 0)


# ---- expert MLP ------------------------------------------------------------
def _mlp_ref_bf16(x, w1, w2):
    F = w1.shape[0] // 2
    xf, w1f, w2f = _f(x), _f(w1), _f(w2)
    g = xf @ w1f[:F].T
    u = xf @ w1f[F:].T
    a = _bf16((g * torch.sigmoid(torch.from_numpy(g)).numpy()) * u)
    return _bf16(_f(a) @ w2f.T), a


@pytest.mark.parametrize("n,H,F", [(1, 128, 64), (7, 256, 128), (33, 512, 256)])
def test_expert_mlp_bf16_matches_numpy(n, H, F):
    x = S.bf16_normal((n, H), 31)
    w1 = S.bf16_normal((2 * F, H), 32, std=0.05)
    w2 = S.bf16_normal((H, F), 33, std=0.05)
    y, a = oracle.expert_mlp_bf16(x, w1, w2, return_a=True)
    yr, ar = _mlp_ref_bf16(x, w1, w2)
    assert np.mean(a == ar) > 0.995
    assert _rel_l2(_f(y), _f(yr)) < 2e-3
    assert np.mean(y == yr) > 0.95


def test_expert_mlp_bf16_gate_and_up_halves():
    """Swapping the halves changes the result (silu is applied to rows
    [0,F) only); zero weights give an exactly zero output."""
    n, H, F = 4, 128, 32
    x = S.bf16_normal((n, H), 41)
    w1 = S.bf16_normal((2 * F, H), 42, std=0.1)
    w2 = S.bf16_normal((H, F), 43, std=0.1)
    y = oracle.expert_mlp_bf16(x, w1, w2)
    sw = np.concatenate([w1[F:], w1[:F]])
    assert not np.array_equal(y, oracle.expert_mlp_bf16(x, sw, w2))
    assert np.all(oracle.expert_mlp_bf16(x, np.zeros_like(w1), w2) & 0x7FFF == 0)
    assert np.all(oracle.expert_mlp_bf16(x, w1, np.zeros_like(w2)) & 0x7FFF == 0)


def _mlp_ref_fp8(x, w1q, w1s, w2q, w2s):
    """numpy/torch W8A8 reference: torch's e4m3 casts and decodes, fp64 matmuls."""
    F = w1q.shape[0] // 2
    H = x.shape[1]

    def quant(v32):
        t = torch.from_numpy(v32).view(v32.shape[0], -1, 128)
        am = t.abs().amax(2)
        s = torch.where(am > 0, am / 448.0, torch.ones_like(am))
        q = (t / s[:, :, None]).clamp(-448, 448).to(torch.float8_e4m3fn).to(torch.float64)
        return (q * s[:, :, None].to(torch.float64)).reshape(v32.shape).numpy()

    def deq(q, s):
        v = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        return v * np.kron(s.astype(np.float64), np.ones((128, 128)))

    xd = quant(S.bf16_to_float(x))
    W1 = deq(w1q, w1s)
    W2 = deq(w2q, w2s)
    g, u = xd @ W1[:F].T, xd @ W1[F:].T
    a = (g * torch.sigmoid(torch.from_numpy(g)).numpy() * u).astype(np.float32)
    return _bf16(quant(a) @ W2.T)


def test_expert_mlp_fp8_matches_numpy():
    n, H, F = 5, 256, 256
    x = S.bf16_normal((n, H), 51)
    w1q, w1s = S.weights_fp8_blocks(1, 2 * F, H, 52, std=0.05)
    w2q, w2s = S.weights_fp8_blocks(1, H, F, 53, std=0.05)
    w1q, w1s, w2q, w2s = (t[0].numpy() for t in (w1q, w1s, w2q, w2s))
    y = oracle.expert_mlp_fp8(x, w1q, w1s, w2q, w2s)
    yr = _mlp_ref_fp8(x, w1q, w1s, w2q, w2s)
    assert _rel_l2(_f(y), _f(yr)) < 1e-3
    assert np.mean(y == yr) > 0.9


def test_layer_tokens_composes_route_mlp_combine():
    """Sampled-token layer output equals the full permute -> per-expert MLP
    -> combine pipeline on a small problem."""
    c = S.CONFIGS["small_layer_512x1024"]
    T, E, K, H, F = 64, 4, 2, 128, 64
    idx, pr = S.route_softmax_topk(T, E, K, 61)
    rt = oracle.route(idx, 0, E, K, pr, pad=c.pad)
    x = S.bf16_normal((T, H), 62)
    W1 = S.bf16_normal((E, 2 * F, H), 63, std=0.05)
    W2 = S.bf16_normal((E, H, F), 64, std=0.05)
    perm = oracle.permute_rows(x, rt["row_id"], rt["R"])
    Y = np.zeros_like(perm)
    for e in range(E):
        s, k = rt["seg_off"][e], rt["counts"][e]
        Y[s:s + k] = oracle.expert_mlp_bf16(perm[s:s + k], W1[e], W2[e])
    full = oracle.combine_bf16(Y, rt["row_id"], rt["copy_prob"])
    toks = [0, 5, 17, 63]
    part = oracle.layer_tokens(toks, x, rt, lambda e, rows: oracle.expert_mlp_bf16(rows, W1[e], W2[e]))
    assert np.array_equal(part, full[toks])


# ---- fp8 combine format -------------------------------------------------------
def test_expert_mlp_float_output_matches_numpy():
    """The float32 view of FC2's sums (what an fp8 output format quantises) is
    the fp64 product of the bf16 activations with W2, rounded once to
    float32, and rounds to the bf16 output."""
    n, H, F = 9, 256, 128
    x = S.bf16_normal((n, H), 71)
    w1 = S.bf16_normal((2 * F, H), 72, std=0.05)
    w2 = S.bf16_normal((H, F), 73, std=0.05)
    y, a, y32 = oracle.expert_mlp_bf16(x, w1, w2, return_a=True, return_y32=True)
    ref = _f(a) @ _f(w2).T                                  # numpy fp64 from the oracle's own a
    assert np.all(np.abs(y32.astype(np.float64) - ref) <= 2.0 ** -24 * np.abs(ref) + 1e-30)
    assert np.mean(_bf16(y32.astype(np.float64)) == y) > 0.999


def test_combine_fp8_matches_torch_dequantised_gather():
    """Dequantise with torch's float8_e4m3fn, weight and sum in fp64 with
    numpy, round to bf16: the oracle must be that value (nearest rounding)."""
    r = np.random.default_rng(81)
    T, K, H, R = 30, 4, 384, 150
    v = (r.standard_normal((R, H)) * np.exp(r.standard_normal((R, 1)))).astype(np.float32)
    q, s = oracle.quant_rows_e4m3(v)
    rid = np.stack([r.choice(R, K, replace=False) for _ in range(T)]).astype(np.int32)
    rid[r.random((T, K)) < 0.25] = -1
    cp = r.random((T, K)).astype(np.float32)
    got = oracle.combine_fp8(q, s, rid, cp)
    deq = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy() * np.repeat(s, 128, axis=1)
    w = np.where(rid >= 0, cp.astype(np.float64), 0.0)
    exact = np.einsum("tk,tkh->th", w, deq[np.maximum(rid, 0)])
    want = _bf16(exact)
    ok = (got == want) | (np.abs(_f(got) - exact) <= np.abs(_f(want) - exact))
    assert ok.all() and np.mean(got == want) > 0.999
    # without probabilities: the plain sum of the dequantised copies
    got1 = oracle.combine_fp8(q, s, rid, cp, apply_probs=False)
    exact1 = np.einsum("tk,tkh->th", (rid >= 0).astype(np.float64), deq[np.maximum(rid, 0)])
    want1 = _bf16(exact1)
    assert np.all((got1 == want1) | (np.abs(_f(got1) - exact1) <= np.abs(_f(want1) - exact1)))
