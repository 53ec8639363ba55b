"""Pins for the oracle's routing metadata (counts, capacity, padding,
offsets, row map, flag): an independent sort-by-expert brute force on
exhaustive tiny inputs, invariants on larger seeded inputs, the pages'
printed values and the pages' capacity checks.  CPU only."""
import itertools
import json
import math
import os

import numpy as np
import pytest

import moe_synth as S
import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))


def brute_route(routing, fmt, E, K, probs=None, pad=1, cap=-1, R=None, T_live=None):
    """Second formulation of the routing definition: collect the valid
    copies, group them by expert, order each group by token, keep a prefix of
    each group, lay the padded groups out one after another."""
    T = routing.shape[0]
    T_live = T if T_live is None else T_live
    flag = 0
    copies = []                            # (t, j, e, prob)
    for t in range(T_live):
        if fmt == oracle.FMT_SPARSE_U8:
            es = [e for e in range(E) if routing[t, e]]
            if len(es) > K:
                flag |= oracle.FLAG_DUPLICATE
            for j, e in enumerate(es[:K]):
                copies.append((t, j, e, 1.0 if probs is None else float(probs[t, e])))
        else:
            used = set()
            for j in range(K):
                e = int(routing[t, j])
                if e == -1:
                    continue
                if e < -1 or e >= E:
                    flag |= oracle.FLAG_BAD_EXPERT
                    continue
                if e in used:
                    flag |= oracle.FLAG_DUPLICATE
                    continue
                used.add(e)
                copies.append((t, j, e, 1.0 if probs is None else float(probs[t, j])))
    groups = {e: sorted([c for c in copies if c[2] == e], key=lambda c: c[0]) for e in range(E)}
    counts = [len(groups[e]) for e in range(E)]
    if cap >= 0 and any(c > cap for c in counts):
        flag |= oracle.FLAG_CAPACITY
    kept = [c if cap < 0 else min(c, cap) for c in counts]
    sizes = [math.ceil(k / pad) * pad for k in kept]
    seg = [0] + list(itertools.accumulate(sizes))
    if R is None:
        R = oracle.out_rows_bound(T, E, K, pad, cap)
    if seg[-1] > R:
        flag |= oracle.FLAG_OUT_ROWS
    row_id = -np.ones((T, K), np.int64)
    src = -np.ones(R, np.int64)
    pp = np.zeros(R, np.float32)
    for e in range(E):
        for rank, (t, j, _, p) in enumerate(groups[e][:kept[e]]):
            row = seg[e] + rank
            if row < R:
                row_id[t, j] = row
                src[row] = t
                pp[row] = p
    return dict(counts=np.array(counts), seg_off=np.array(seg), row_id=row_id, src_row=src,
                perm_prob=pp, rows_needed=seg[-1], flag=flag)


def _same(o, b):
    assert np.array_equal(o["counts"], b["counts"])
    assert np.array_equal(o["seg_off"], b["seg_off"])
    assert np.array_equal(o["row_id"], b["row_id"])
    assert np.array_equal(o["src_row"], b["src_row"])
    assert np.array_equal(o["perm_prob"], b["perm_prob"])
    assert o["rows_needed"] == b["rows_needed"]
    assert o["flag"] == b["flag"]


def test_exhaustive_dense_tiny():
    """Every dense table over T=2, K=2 with entries in {-2,-1,0,1,2} (E=2, so
    -2 and 2 are invalid), every padding multiple 1..3, capacity -1..2 and a
    range of output row counts."""
    E, K, T = 2, 2, 2
    vals = [-2, -1, 0, 1, 2]
    n = 0
    for cells in itertools.product(vals, repeat=T * K):
        idx = np.array(cells, np.int16).reshape(T, K)
        probs = (np.arange(T * K, dtype=np.float32).reshape(T, K) + 1) / 8
        for pad in (1, 2, 3):
            for cap in (-1, 0, 1, 2):
                bound = oracle.out_rows_bound(T, E, K, pad, cap)
                for R in sorted({0, 1, 3, bound}):
                    o = oracle.route(idx, oracle.FMT_DENSE_I16, E, K, probs, pad, cap, R)
                    _same(o, brute_route(idx, oracle.FMT_DENSE_I16, E, K, probs, pad, cap, R))
                    n += 1
    assert n > 10000


def test_exhaustive_sparse_tiny():
    E, T = 3, 2
    for bits in range(1 << (T * E)):
        m = np.array([(bits >> i) & 1 for i in range(T * E)], np.uint8).reshape(T, E)
        probs = (np.arange(T * E, dtype=np.float32).reshape(T, E) + 1) / 16
        for K in (1, 2, 3):
            for pad in (1, 2):
                for cap in (-1, 0, 1):
                    for R in (2, oracle.out_rows_bound(T, E, K, pad, cap)):
                        o = oracle.route(m, oracle.FMT_SPARSE_U8, E, K, probs, pad, cap, R)
                        _same(o, brute_route(m, oracle.FMT_SPARSE_U8, E, K, probs, pad, cap, R))


@pytest.mark.parametrize("seed", range(40))
def test_random_small_against_brute_force(seed):
    r = np.random.default_rng(seed)
    T = int(r.integers(0, 40))
    E = int(r.integers(1, 9))
    K = int(r.integers(1, E + 1))
    pad = int(r.integers(1, 6))
    cap = int(r.integers(-1, 8))
    T_live = int(r.integers(0, T + 1))
    fmt = int(r.integers(0, 3))
    if fmt == oracle.FMT_SPARSE_U8:
        routing = (r.random((T, E)) < 0.4).astype(np.uint8)
        probs = r.random((T, E)).astype(np.float32)
    else:
        routing = r.integers(-2, E + 1, (T, K)).astype(np.int16 if fmt == 0 else np.int32)
        probs = r.random((T, K)).astype(np.float32)
    bound = oracle.out_rows_bound(T, E, K, pad, cap)
    R = int(r.integers(0, bound + 1))
    o = oracle.route(routing, fmt, E, K, probs, pad, cap, R, T_live)
    _same(o, brute_route(routing, fmt, E, K, probs, pad, cap, R, T_live))


def _invariants(rt, T, K, pad, cap):
    rid = rt["row_id"]
    kept_rows = rid[rid >= 0]
    # each kept copy lands on its own row, and src_row is the exact inverse
    assert len(np.unique(kept_rows)) == len(kept_rows)
    tt = np.repeat(np.arange(T), K).reshape(T, K)
    assert np.array_equal(rt["src_row"][kept_rows], tt[rid >= 0])
    assert np.count_nonzero(rt["src_row"] >= 0) == len(kept_rows)
    seg = rt["seg_off"]
    assert np.all(seg % pad == 0)
    E = len(rt["counts"])
    for e in range(E):
        k = rt["counts"][e] if cap < 0 else min(rt["counts"][e], cap)
        assert seg[e + 1] - seg[e] == -(-k // pad) * pad
        s = rt["src_row"][seg[e]:seg[e] + k]
        assert np.all(np.diff(s) > 0)          # token order inside a segment
        assert np.all(rt["src_row"][seg[e] + k:seg[e + 1]] == -1)
    assert bool(rt["flag"] & oracle.FLAG_CAPACITY) == (cap >= 0 and rt["counts"].max(initial=0) > cap)


@pytest.mark.parametrize("name", ["small_layer_512x1024", "permute_combine_8192x7168_e32", "dsv3_layer_8192x7168_e256"])
def test_invariants_on_workload_routing(name):
    c = S.CONFIGS[name]
    if name == "small_layer_512x1024":
        idx, pr = S.route_softmax_topk(c.T, c.E, c.K, c.seed)
    elif name == "permute_combine_8192x7168_e32":
        idx, pr = S.route_uniform_distinct(c.T, c.E, c.K, c.seed)
    else:
        idx, pr = S.route_sigmoid_topk(c.T, c.E, c.K, c.seed)
    rt = oracle.route(idx, oracle.FMT_DENSE_I16, c.E, c.K, pr, c.pad)
    # full top-k routing: the counts add up to T*K
    assert rt["counts"].sum() == c.T * c.K
    assert rt["flag"] == 0
    _invariants(rt, c.T, c.K, c.pad, -1)
    assert np.allclose(rt["perm_prob"][rt["row_id"][rt["row_id"] >= 0]], pr[rt["row_id"] >= 0])


def test_dense_and_sparse_encodings_agree_on_stress_routing():
    """Dense int16 and Boolean encodings of the same routing give identical
    counts, offsets, row sources and permuted probabilities (the pages report
    bitwise-equal dispatch for both formats)."""
    g = GOLD["stress_shape"]
    T, E, K = 1024, g["experts"], g["topk"]          # token count reduced for CPU time
    idx, pr = S.route_zipf_gumbel(T, E, K, 1003)
    m, pe = S.dense_to_sparse(idx, E, pr)
    d = oracle.route(idx, oracle.FMT_DENSE_I16, E, K, pr)
    s = oracle.route(m, oracle.FMT_SPARSE_U8, E, K, pe)
    for k in ("counts", "seg_off", "src_row", "perm_prob"):
        assert np.array_equal(d[k], s[k]), k
    assert d["flag"] == s["flag"] == 0
    _invariants(d, T, K, 1, -1)


def test_capacity_checks_from_the_pages():
    """Capacity 1x, 1.5x, 2x the largest count: identical to the uncapped
    dispatch, flag clear; capacity at half: flag set, kept copies are each
    expert's earliest tokens.  One below the largest count also overflows."""
    c = S.CONFIGS["permute_combine_8192x7168_e32"]
    T = 2048
    idx, pr = S.route_uniform_distinct(T, c.E, c.K, c.seed)
    base = oracle.route(idx, oracle.FMT_DENSE_I16, c.E, c.K, pr)
    mx = int(base["counts"].max())
    R = base["rows_needed"]
    for f in GOLD["capacity_checks"]["equal_factors"]:
        cap = oracle.capacity_from_rows(mx, f) if f != 1.0 else mx
        rt = oracle.route(idx, oracle.FMT_DENSE_I16, c.E, c.K, pr, 1, cap, R)
        assert rt["flag"] == 0
        for k in ("counts", "seg_off", "row_id", "src_row", "perm_prob"):
            assert np.array_equal(rt[k], base[k]), (f, k)
    for cap in (mx - 1, mx // 2):
        rt = oracle.route(idx, oracle.FMT_DENSE_I16, c.E, c.K, pr, 1, cap)
        assert rt["flag"] & oracle.FLAG_CAPACITY
        assert np.array_equal(rt["counts"], base["counts"])       # counts stay raw
        _invariants(rt, T, c.K, 1, cap)
        for e in range(c.E):
            toks = np.nonzero((base["copy_expert"] == e).any(axis=1))[0]
            got = rt["src_row"][rt["seg_off"][e]:rt["seg_off"][e + 1]]
            assert np.array_equal(got, toks[:cap])


def test_out_rows_flag_and_drop():
    idx = np.array([[0, 1], [1, 0], [0, 1]], np.int16)
    full = oracle.route(idx, 0, 2, 2, pad=4)
    assert full["rows_needed"] == 8 and full["flag"] == 0
    rt = oracle.route(idx, 0, 2, 2, pad=4, R=5)
    assert rt["flag"] == oracle.FLAG_OUT_ROWS
    # expert 0 keeps rows 0..2, expert 1 starts at 4 and only its first copy fits
    assert list(rt["src_row"]) == [0, 1, 2, -1, 0]
    assert rt["row_id"].tolist() == [[0, 4], [-1, 1], [2, -1]]
    assert rt["copy_prob"].tolist() == [[1, 1], [0, 1], [1, 0]]


def test_flag_bits_for_bad_and_duplicate_entries():
    idx = np.array([[0, 5], [1, 1], [-1, -1]], np.int16)
    rt = oracle.route(idx, 0, 3, 2)
    assert rt["flag"] == oracle.FLAG_BAD_EXPERT | oracle.FLAG_DUPLICATE
    assert rt["row_id"].tolist() == [[0, -1], [1, -1], [-1, -1]]
    m = np.array([[1, 1, 1]], np.uint8)
    rt = oracle.route(m, 2, 3, 2)
    assert rt["flag"] == oracle.FLAG_DUPLICATE
    assert rt["copy_expert"].tolist() == [[0, 1]]


def test_empty_and_degenerate():
    rt = oracle.route(np.zeros((0, 4), np.int16), 0, 8, 4, pad=16)
    assert rt["rows_needed"] == 0 and rt["flag"] == 0 and rt["counts"].sum() == 0
    # one expert, every token routed to it
    rt = oracle.route(np.zeros((5, 1), np.int16), 0, 1, 1, pad=4)
    assert rt["seg_off"].tolist() == [0, 8] and list(rt["src_row"][:5]) == [0, 1, 2, 3, 4]
    # K == E: every token goes everywhere
    idx = np.tile(np.arange(4, dtype=np.int16), (3, 1))
    rt = oracle.route(idx, 0, 4, 4)
    assert rt["counts"].tolist() == [3, 3, 3, 3]
    # capacity 0 drops everything
    rt = oracle.route(idx, 0, 4, 4, cap=0)
    assert rt["rows_needed"] == 0 and np.all(rt["row_id"] == -1) and rt["flag"] == oracle.FLAG_CAPACITY
    # live-token trim: tokens at or beyond T_live are unrouted
    rt = oracle.route(idx, 0, 4, 4, T_live=1)
    assert rt["counts"].tolist() == [1, 1, 1, 1] and np.all(rt["row_id"][1:] == -1)


def test_page_value_routing_bytes():
    g = GOLD["routing_bytes"]
    tok = g["tokens_per_rank"] * g["world_size"]          # the gathered routing on each rank
    assert oracle.routing_bytes(tok, g["experts"], g["topk"], oracle.FMT_SPARSE_U8) == g["sparse_bool_bytes_per_rank"]
    assert oracle.routing_bytes(tok, g["experts"], g["topk"], oracle.FMT_DENSE_I16) == g["dense_int16_bytes_per_rank"]
    assert g["world_size"] * g["sparse_bool_bytes_per_rank"] == g["sparse_bool_bytes_group"]
    assert g["world_size"] * g["dense_int16_bytes_per_rank"] == g["dense_int16_bytes_group"]


def test_page_value_capacity_calibration():
    g = GOLD["capacity_calibration"]
    assert oracle.capacity_from_rows(g["rows"], g["factor"]) == g["capacity"]
    assert oracle.capacity_from_rows(10, 1.5) == 16        # 15 -> next multiple of 4
    assert oracle.capacity_from_rows(8, 1.0) == 8


def _routing_with_counts(counts, T, K):
    """Dense routing [T,K] in which expert e appears counts[e] times, each at
    most once per token (requires counts[e] <= T and sum(counts) <= T*K;
    unused slots are -1).  The copies are laid out slot-major in expert
    order: position j*T + t of the flat list is slot j of token t, and a run
    of at most T equal experts never reaches the same token twice."""
    flat = np.full(T * K, -1, np.int64)
    ids = np.repeat(np.arange(len(counts)), counts)
    flat[:len(ids)] = ids
    idx = flat.reshape(K, T).T.astype(np.int16)
    for t in range(T):
        row = idx[t][idx[t] >= 0]
        assert len(set(row.tolist())) == len(row)
    return idx


def test_out_rows_bound_reached_by_each_term():
    """The bound is reached exactly, through each of its two terms, by
    routings built for it; together with the safety checks below this pins
    it from both sides (a bound that is too large, e.g. padding E*p rows or
    a capacity not rounded up to the padding multiple, fails here)."""
    cases = 0
    for E in range(1, 7):
        for K in range(1, E + 1):
            for pad in range(1, 5):
                for T in range(1, 13):
                    # copies term T*K + E*(pad-1): every expert holds a count
                    # of 1 mod pad, so each segment carries pad-1 padding rows
                    N = T * K
                    if N >= E and (N - E) % pad == 0:
                        counts = np.ones(E, np.int64)
                        extra, e = (N - E) // pad, 0
                        while extra and e < E:        # top experts up by pad, keeping counts <= T
                            take = min(extra, (T - 1) // pad)
                            counts[e] += take * pad
                            extra -= take
                            e += 1
                        if extra == 0:
                            idx = _routing_with_counts(counts, T, K)
                            rt = oracle.route(idx, 0, E, K, pad=pad, R=10 ** 6)
                            bound = oracle.out_rows_bound(T, E, K, pad, -1)
                            assert rt["rows_needed"] == bound == N + E * (pad - 1), (T, E, K, pad)
                            cases += 1
                    # capacity term E*roundup(C, pad): every expert over capacity
                    for C in range(0, T + 1):
                        if E * T > N:
                            continue          # not every expert can receive T copies
                        counts = np.full(E, T, np.int64)
                        idx = _routing_with_counts(counts, T, K)
                        rt = oracle.route(idx, 0, E, K, pad=pad, cap=C, R=10 ** 6)
                        bound = oracle.out_rows_bound(T, E, K, pad, C)
                        if E * (-(-C // pad) * pad) <= N + E * (pad - 1):
                            assert rt["rows_needed"] == bound, (T, E, K, pad, C)
                            cases += 1
    assert cases > 300


def test_out_rows_bound_safe_exhaustive_tiny():
    """No dense routing of up to 3 tokens, 3 experts, top-2 (empty slots
    included) needs more rows than the bound, for every padding multiple
    1 and 3 and capacity none, 1 and 2."""
    for T in range(0, 4):
        for E in range(1, 4):
            for K in range(1, min(E, 2) + 1):
                rows = list(itertools.product(range(-1, E), repeat=K))
                rows = [r for r in rows if len({e for e in r if e >= 0}) == sum(e >= 0 for e in r)]
                for pad in (1, 3):
                    for cap in (-1, 1, 2):
                        bound = oracle.out_rows_bound(T, E, K, pad, cap)
                        worst = 0
                        for combo in itertools.product(rows, repeat=T):
                            idx = np.array(combo, np.int16).reshape(T, K)
                            worst = max(worst, oracle.route(idx, 0, E, K, pad=pad, cap=cap, R=10 ** 6)["rows_needed"])
                        assert worst <= bound, (T, E, K, pad, cap, worst, bound)


def test_out_rows_bound_is_tight_and_safe():
    r = np.random.default_rng(7)
    for _ in range(200):
        T, E = int(r.integers(0, 30)), int(r.integers(1, 7))
        K, pad, cap = int(r.integers(1, E + 1)), int(r.integers(1, 5)), int(r.integers(-1, 6))
        idx = np.argsort(r.random((T, E)), axis=1)[:, :K].astype(np.int16)
        rt = oracle.route(idx, 0, E, K, pad=pad, cap=cap)
        assert rt["rows_needed"] <= rt["R"] and rt["flag"] == (oracle.FLAG_CAPACITY if cap >= 0 and rt["counts"].max(initial=0) > cap else 0)
