"""Routing metadata on the GPU (K1) against the oracle: counts, segment
offsets, row map, copy probabilities, row sources, permuted probabilities,
rows needed and the overflow flag must match bit for bit."""
import numpy as np
import pytest

import moe_synth as S
import oracle
from gpu_util import assert_route_equal, gpu_route, log

pytestmark = pytest.mark.gpu


def _case(seed):
    r = np.random.default_rng(10_000 + seed)
    big = seed % 10 == 0
    T = int(r.integers(0, 3000 if big else 300))
    E = int(r.choice([1, 2, 3, 7, 16, 33, 64, 256, 1024] if big else [1, 2, 3, 5, 8, 16, 31, 64]))
    K = int(r.integers(1, min(E, 40) + 1))
    fmt = int(r.integers(0, 3))
    pad = int(r.choice([1, 1, 2, 3, 16, 128]))
    cap = int(r.choice([-1, -1, 0, 1, 5, 50]))
    if fmt == oracle.FMT_SPARSE_U8:
        routing = (r.random((T, E)) < min(0.9, 1.5 * K / E)).astype(np.uint8)
        probs = r.random((T, E)).astype(np.float32)
    else:
        lo = -2 if seed % 3 == 0 else -1
        routing = r.integers(lo, E + (1 if seed % 3 == 0 else 0), (T, K))
        if seed % 3 == 1:      # distinct experts per row
            routing = np.argsort(r.random((T, E)), axis=1)[:, :K]
        routing = routing.astype(np.int16 if fmt == 0 else np.int32)
        probs = r.random((T, K)).astype(np.float32)
    if seed % 4 == 0:
        probs = None
    bound = oracle.out_rows_bound(T, E, K, pad, cap)
    # out_rows = 0 means "use the bound", so an explicit R starts at 1
    R = None if (seed % 5 or bound < 1) else int(r.integers(1, bound + 1))
    T_live = None if seed % 6 else int(r.integers(0, T + 1))
    return routing, fmt, E, K, probs, pad, cap, R, T_live


@pytest.mark.parametrize("seed", range(120))
def test_random_routing_matches_oracle(seed):
    routing, fmt, E, K, probs, pad, cap, R, T_live = _case(seed)
    log("route random", seed, routing.shape, fmt, E, K, pad, cap, R, T_live)
    g, _ = gpu_route(routing, fmt, E, K, probs, pad, cap, R, T_live)
    o = oracle.route(routing, fmt, E, K, probs, pad, cap, g["R"], T_live)
    assert_route_equal(g, o, f"seed {seed}")


def _workload(name):
    c = S.CONFIGS[name]
    if name == "small_layer_512x1024":
        return c, S.route_softmax_topk(c.T, c.E, c.K, c.seed)
    if name == "permute_combine_8192x7168_e32":
        return c, S.route_uniform_distinct(c.T, c.E, c.K, c.seed)
    if name == "route_stress_fp8_8192x7168_e256":
        return c, S.route_zipf_gumbel(c.T, c.E, c.K, c.seed)
    return c, S.route_sigmoid_topk(c.T, c.E, c.K, c.seed)


@pytest.mark.parametrize("name", ["small_layer_512x1024", "permute_combine_8192x7168_e32", "dsv3_layer_8192x7168_e256"])
def test_workload_routing_matches_oracle(name):
    c, (idx, pr) = _workload(name)
    log("route workload", name)
    g, _ = gpu_route(idx, oracle.FMT_DENSE_I16, c.E, c.K, pr, c.pad)
    o = oracle.route(idx, oracle.FMT_DENSE_I16, c.E, c.K, pr, c.pad, -1, g["R"])
    assert_route_equal(g, o, name)
    assert g["counts"].sum() == c.T * c.K


@pytest.mark.parametrize("with_probs", [False, True])
def test_stress_routing_dense_and_sparse(with_probs):
    """8192 tokens, 256 experts, top-36, Zipf-skewed: both encodings match the
    oracle and each other."""
    c, (idx, pr) = _workload("route_stress_fp8_8192x7168_e256")
    m, pe = S.dense_to_sparse(idx, c.E, pr)
    log("route stress", with_probs)
    gd, _ = gpu_route(idx, oracle.FMT_DENSE_I16, c.E, c.K, pr if with_probs else None)
    gs, _ = gpu_route(m, oracle.FMT_SPARSE_U8, c.E, c.K, pe if with_probs else None)
    od = oracle.route(idx, oracle.FMT_DENSE_I16, c.E, c.K, pr if with_probs else None, 1, -1, gd["R"])
    os_ = oracle.route(m, oracle.FMT_SPARSE_U8, c.E, c.K, pe if with_probs else None, 1, -1, gs["R"])
    assert_route_equal(gd, od, "dense")
    assert_route_equal(gs, os_, "sparse")
    for k in ("counts", "seg_off", "src_row", "perm_prob"):
        assert np.array_equal(gd[k], gs[k]), k
    assert gd["counts"].max() == c.T            # the hottest experts receive every token


def test_capacity_factors_and_overflow():
    c, (idx, pr) = _workload("permute_combine_8192x7168_e32")
    base = oracle.route(idx, 0, c.E, c.K, pr)
    mx = int(base["counts"].max())
    for cap in [mx, oracle.capacity_from_rows(mx, 1.5), oracle.capacity_from_rows(mx, 2.0), mx - 1, mx // 2]:
        log("route capacity", cap)
        g, _ = gpu_route(idx, 0, c.E, c.K, pr, 1, cap)
        o = oracle.route(idx, 0, c.E, c.K, pr, 1, cap, g["R"])
        assert_route_equal(g, o, f"cap {cap}")
        assert bool(g["flag"] & oracle.FLAG_CAPACITY) == (cap < mx)


@pytest.mark.parametrize("T", [0, 1, 16, 63, 64, 65, 100, 256])
def test_decode_sizes_with_live_trim(T):
    c = S.CONFIGS["decode_fp8_7168_e256"]
    bucket = S.next_pow2_bucket(T)
    idx, pr = S.route_sigmoid_topk(bucket, c.E, c.K, c.seed + T)
    log("route decode", T, bucket)
    g, _ = gpu_route(idx, 0, c.E, c.K, pr, c.pad, -1, None, T)
    o = oracle.route(idx, 0, c.E, c.K, pr, c.pad, -1, g["R"], T)
    assert_route_equal(g, o, f"T {T}")


def test_large_token_count_and_max_experts():
    r = np.random.default_rng(77)
    T, E, K = 40_000, 1024, 6
    idx = np.argsort(r.random((T, 64)), axis=1)[:, :K] * 16 + r.integers(0, 16, (T, 1))
    idx = idx.astype(np.int32)
    log("route large", T, E, K)
    g, _ = gpu_route(idx, oracle.FMT_DENSE_I32, E, K, None, 8, 300)
    o = oracle.route(idx, oracle.FMT_DENSE_I32, E, K, None, 8, 300, g["R"])
    assert_route_equal(g, o, "large")


def test_repeated_preprocess_is_deterministic():
    c, (idx, pr) = _workload("dsv3_layer_8192x7168_e256")
    g1, d = gpu_route(idx, 0, c.E, c.K, pr, c.pad)
    import torch
    from gpu_util import dev
    for cycle in range(3):
        log("route repeat", cycle)
        d.preprocess(dev(idx), dev(pr))
        torch.cuda.synchronize()
        assert np.array_equal(d.row_id.cpu().numpy(), g1["row_id"])
        assert np.array_equal(d.tokens_per_expert.cpu().numpy(), g1["counts"])
        assert int(d.flag.item()) == 0
