#!/usr/bin/env python3
"""Benchmark of the MoE layer hot path on one MI355X.

One step = routing metadata preprocessing -> permute -> grouped FC1 + SwiGLU
-> grouped FC2 (into a reused caller-owned buffer) -> combine -> device-side
assert that the overflow flag is clear, over one batch of the
DeepSeek-V3-shaped synthetic workload: 8192 tokens x 7168 bf16, 256 experts
top-8 (sigmoid scores, renormalised), FFN 2048, padding multiple 128.  Inputs
and weights are resident in HBM before timing starts.

Prints one JSON line (stdout).  Per-stage times come from HIP events recorded
on the stream the kernels run on; the roofline entry is for the dominant
kernel (grouped FC1 + SwiGLU).  Beside the headline step the line carries the
other synthetic workloads (small layer per stage, the 32-expert
permute/combine with its overflow case, the fp8 routing stress in both routing
formats, the fp8 decode buckets) and the CPU oracle timed on the host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
METRIC = "permute+combine HBM GB/s (% peak); MoE-layer tokens/s at 8192x7168, 256E top-8"
FC1_PROFILE = os.path.join(ROOT, "profiles", "fc1_dsv3_layer.json")
FC1_SOURCE = os.path.join(ROOT, "combine_routing_preprocess_amd", "csrc", "gemm_bf16.hip")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def source_hash(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def fc1_profile():
    """The committed rocprofv3 figures of the FC1 kernel (HBM bytes per launch
    from FETCH_SIZE/WRITE_SIZE, average duration from the kernel trace), or
    an empty dict when they are missing or were taken on another kernel
    source."""
    try:
        t = json.load(open(FC1_PROFILE))
    except (OSError, ValueError):
        return {}
    if t.get("kernel_source_sha256_16") != source_hash(FC1_SOURCE):
        return {}
    return t


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-tokens", type=int, default=256, help="oracle MLP sample size (0 = no CPU baseline)")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay measurement")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the other synthetic workloads (small layer, 32-expert permute/combine, fp8 "
                         "routing stress, fp8 decode buckets)")
    ap.add_argument("--extra", action="store_true",
                    help="also time the backward and the fp8 formats at the layer shape")
    ap.add_argument("--calib-copy", action="store_true",
                    help="end with one 1 GiB device copy (reference dispatch for hardware byte counters)")
    ap.add_argument("--workload", choices=("dsv3_layer", "decode"), default="dsv3_layer",
                    help="decode: only the fp8 decode layer, eager, for kernel profiling")
    ap.add_argument("--tokens", type=int, default=16, help="decode workload: live tokens (bucket = next pow2)")
    ap.add_argument("--decode-path", choices=("separate", "fused", "persistent"), default="separate",
                    help="decode workload: separate launches, the fused decode layer (two launches) or the "
                         "persistent decode kernel (one launch)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the single-GPU layer: every expert is local to one MI355X and there is no "
              "cross-GPU exchange in this library, so --gpus must be 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import moe_synth as S
    from combine_routing_preprocess_amd import Dispatcher, assert_no_overflow

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = "cuda"
    if args.workload == "decode":
        return run_decode(args)
    c = S.CONFIGS["dsv3_layer_8192x7168_e256"]
    T, H, E, K, F, pad = c.T, c.H, c.E, c.K, c.F, c.pad

    # ---- inputs, resident in HBM -------------------------------------------
    idx, pr = S.route_sigmoid_topk(T, E, K, c.seed)
    x_np = S.bf16_normal((T, H), c.seed)
    x = torch.from_numpy(x_np.view(np.int16)).to(dev).view(torch.bfloat16)
    routing = torch.from_numpy(idx).to(dev)
    probs = torch.from_numpy(pr).to(dev)
    log("drawing weights on the device")
    w1 = S.weights_bf16(E, 2 * F, H, c.seed + 1, device=dev)
    w2 = S.weights_bf16(E, H, F, c.seed + 2, device=dev)
    d = Dispatcher(T, H, E, K, pad_multiple=pad)
    perm = torch.empty((d.R, H), dtype=torch.bfloat16, device=dev)
    scratch = d.alloc_mlp_scratch(F)
    expert_out = torch.empty((d.R, H), dtype=torch.bfloat16, device=dev)
    y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        d.preprocess(routing, probs)
        if ev is not None:
            ev[1].record()
        d.permute(x, out=perm)
        if ev is not None:
            ev[2].record()
        d.fc1(perm, w1, scratch)
        if ev is not None:
            ev[3].record()
        d.fc2(w2, scratch, expert_out)
        if ev is not None:
            ev[4].record()
        d.combine(expert_out, out=y)
        if ev is not None:
            ev[5].record()
        assert_no_overflow(d.flag)      # on the device; the host does not wait

    # the step ends with a device-side assert on the overflow flag (a failing
    # device assert aborts the queue on this ROCm build): check the flag on
    # the host first, on the same inputs
    _require_clear_flag(d, routing, probs)
    log("layer step: warm-up")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert int(d.flag.item()) == 0, "routing flag set"
    kept = d.kept.cpu().numpy().astype(np.int64)
    n_copies = int(kept.sum())
    touched = int((kept > 0).sum())

    # ---- timed region ------------------------------------------------------------
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    tokens_per_s = T * args.steps / (t1 - t0)
    log(f"layer step: {ms_per_step:.3f} ms")

    names = ["preprocess", "permute", "fc1_swiglu", "fc2", "combine"]
    stage_ms = {n: [evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(args.steps)] for j, n in enumerate(names)}
    mean = {n: statistics.fmean(v) for n, v in stage_ms.items()}
    mins = {n: min(v) for n, v in stage_ms.items()}

    # ---- algorithmic work per launch (kept copies only, no padding rows) ------
    b = 2  # bf16 bytes
    work = {
        "permute": dict(bytes=T * H * b + n_copies * H * b),
        "combine": dict(bytes=n_copies * H * b + T * H * b),
        "fc1_swiglu": dict(bytes=touched * 2 * F * H * b + n_copies * H * b + n_copies * F * b,
                           flops=2 * n_copies * H * 2 * F),
        "fc2": dict(bytes=touched * H * F * b + n_copies * F * b + n_copies * H * b, flops=2 * n_copies * F * H),
    }
    stages = {}
    for n in names:
        s = {"mean_ms": round(mean[n], 4), "min_ms": round(mins[n], 4)}
        if n in work:
            s["alg_bytes"] = work[n]["bytes"]
            s["GB_s"] = round(work[n]["bytes"] / (mean[n] * 1e-3) / 1e9, 1)
            s["hbm_frac"] = round(s["GB_s"] / HBM_PEAK_GBS, 4)
            if "flops" in work[n]:
                s["alg_flops"] = work[n]["flops"]
                s["TFLOP_s"] = round(work[n]["flops"] / (mean[n] * 1e-3) / 1e12, 1)
                s["mfma_frac"] = round(s["TFLOP_s"] / BF16_PEAK_TFLOPS, 4)
        stages[n] = s

    fc1 = work["fc1_swiglu"]
    t_fc1 = mean["fc1_swiglu"] * 1e-3
    hbm_time = fc1["bytes"] / (HBM_PEAK_GBS * 1e9)
    mfma_time = fc1["flops"] / (BF16_PEAK_TFLOPS * 1e12)
    prof = fc1_profile()
    if hbm_time >= mfma_time:
        roof = {"bound": "hbm", "achieved": round(fc1["bytes"] / t_fc1 / 1e9, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
        per_s = lambda sec: fc1["bytes"] / sec / 1e9
    else:
        roof = {"bound": "mfma", "achieved": round(fc1["flops"] / t_fc1 / 1e12, 1), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
        per_s = lambda sec: fc1["flops"] / sec / 1e12
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = prof.get("bytes_per_launch")
    roof["kernel"] = "k_gemm_bf16<0> (grouped FC1 + SwiGLU)"
    roof["timing"] = "HIP events around the launch on its stream, mean over the timed steps"
    roof["mean_us_events"] = round(mean["fc1_swiglu"] * 1e3, 1)
    roof["rocprof_avg_us"] = prof.get("rocprof_avg_us")
    roof["frac_rocprof"] = (round(per_s(prof["rocprof_avg_us"] * 1e-6) / roof["peak"], 4)
                            if prof.get("rocprof_avg_us") else None)
    roof["alg_bytes_per_launch"] = fc1["bytes"]
    roof["alg_flops_per_launch"] = fc1["flops"]
    roof["mfma_frac"] = stages["fc1_swiglu"]["mfma_frac"]

    pc_bytes = work["permute"]["bytes"] + work["combine"]["bytes"]
    pc_ms = mean["permute"] + mean["combine"]
    permute_combine = {"GB_s": round(pc_bytes / (pc_ms * 1e-3) / 1e9, 1),
                       "frac_of_peak": round(pc_bytes / (pc_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                       "permute_GB_s": stages["permute"]["GB_s"], "combine_GB_s": stages["combine"]["GB_s"]}
    # practical HBM ceilings measured beside them (outside the timed region):
    # a 1 GiB device copy (half reads, half writes) and a 1 GiB fill (writes
    # only; the permute is 89 % writes, the combine 89 % reads)
    ca = torch.empty(2 ** 29, dtype=torch.int16, device=dev)
    cb = torch.empty_like(ca)
    cmin, _ = _event_times(lambda: cb.copy_(ca))
    fmin, _ = _event_times(lambda: cb.fill_(1))
    permute_combine["copy_1GiB_GB_s"] = round(2 * 2 ** 30 / (cmin * 1e-3) / 1e9, 1)
    permute_combine["fill_1GiB_GB_s"] = round(2 ** 30 / (fmin * 1e-3) / 1e9, 1)
    permute_combine["permute_frac_of_fill"] = round(stages["permute"]["GB_s"] / permute_combine["fill_1GiB_GB_s"], 4)
    del ca, cb

    # ---- HIP-graph replay of the whole step ------------------------------------
    graph = None
    if not args.no_graph:
        log("layer step: graph replay")
        gmin, gmed = _graph_times(step, reps=20)
        graph = {"min_ms": round(gmin, 4), "median_ms": round(gmed, 4),
                 "tokens_per_s_at_min": round(T / (gmin * 1e-3), 1)}

    # ---- CPU baseline: the oracle on the host's cores ----------------------------
    cpu = None
    if args.cpu_tokens > 0:
        cpu = cpu_baseline(args, c, idx, pr, x_np, w1, w2, y, expert_out, d)
    del w1, w2, perm, scratch, expert_out
    torch.cuda.empty_cache()

    workloads = None if args.no_workloads else run_workloads()
    extra = run_extra(args) if args.extra else None
    if args.calib_copy:
        _calib_copy()

    out = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "dsv3_layer: 8192 tokens x 7168 bf16, 256 experts top-8 (sigmoid, renormalised), "
                               "SwiGLU FFN 2048, padding multiple 128, dense int16 routing",
                   "T": T, "H": H, "E": E, "K": K, "F": F, "pad_multiple": pad, "out_rows": d.R,
                   "kept_rows": n_copies, "experts_touched": touched, "parallelism": "1 GPU, all experts local"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "permute_combine": permute_combine,
        "stages": stages,
        "graph_replay": graph,
        "workloads": workloads,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)
    return 0


def cpu_baseline(args, c, idx, pr, x_np, w1, w2, y, expert_out, d):
    """The oracle as it stands, on the host's cores.

    All threads, on the layer batch: routing metadata, permute and combine
    over the whole batch; the expert MLPs (fp64 loops) for the first
    ``--cpu-tokens`` tokens, scaled to the batch.  One thread: the small
    layer, the 32-expert permute/combine and the 16-token fp8 decode layer,
    each with its MLP on a token sample.  Host copies of weights and expert
    outputs are made outside the timed calls."""
    import numpy as np
    import torch

    import moe_synth as S
    import oracle
    T, H, E, K, F, pad = c.T, c.H, c.E, c.K, c.F, c.pad
    threads = oracle.get_threads()
    log(f"CPU baseline: oracle on {threads} threads")
    t_start = time.perf_counter()

    def timed(fn):
        t0 = time.perf_counter()
        r = fn()
        return r, time.perf_counter() - t0

    rt, t_route = timed(lambda: oracle.route(idx, oracle.FMT_DENSE_I16, E, K, pr, pad))
    P, t_perm = timed(lambda: oracle.permute_rows(x_np, rt["row_id"], rt["R"]))
    del P
    Yh = expert_out.view(torch.int16).cpu().numpy().view(np.uint16)
    _, t_comb = timed(lambda: oracle.combine_bf16(Yh, rt["row_id"], rt["copy_prob"]))
    del Yh
    n = min(args.cpu_tokens, T)
    toks = np.arange(n)
    t_mlp = [0.0]
    rows_done = [0]

    def expert(e, rows):
        w1h = w1[e].view(torch.int16).cpu().numpy().view(np.uint16)
        w2h = w2[e].view(torch.int16).cpu().numpy().view(np.uint16)
        out, t = timed(lambda: oracle.expert_mlp_bf16(rows, w1h, w2h))
        t_mlp[0] += t
        rows_done[0] += len(rows)
        return out

    yo = oracle.layer_tokens(toks, x_np, rt, expert)
    got = y[:n].view(torch.int16).cpu().numpy().view(np.uint16)
    gf, of = S.bf16_to_float(got).astype(np.float64), S.bf16_to_float(yo).astype(np.float64)
    rel = float(np.linalg.norm(gf - of) / np.linalg.norm(of))
    mlp_est = t_mlp[0] * T / n
    total = t_route + t_perm + mlp_est + t_comb
    cpu = {"value": round(T / total, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
           "sample": f"layer batch ({T} tokens): routing, permute and combine timed over the whole batch; expert "
                     f"MLPs timed for the first {n} tokens ({rows_done[0]} expert rows, fp64 loops) and scaled "
                     f"to {T} tokens",
           "stages_s": {"preprocess": round(t_route, 4), "permute": round(t_perm, 4),
                        "mlp_sample": round(t_mlp[0], 3), "mlp_batch_est": round(mlp_est, 2),
                        "combine": round(t_comb, 4)},
           "gpu_vs_oracle_rel_l2": rel}

    # one thread: the small layer, the 32-expert permute/combine, fp8 decode
    oracle.set_threads(1)
    try:
        one = {}
        cs = S.CONFIGS["small_layer_512x1024"]
        i1, p1 = S.route_softmax_topk(cs.T, cs.E, cs.K, cs.seed)
        x1 = S.bf16_normal((cs.T, cs.H), cs.seed)
        a1 = S.bf16_normal((cs.E, 2 * cs.F, cs.H), cs.seed + 1, std=0.02)
        b1 = S.bf16_normal((cs.E, cs.H, cs.F), cs.seed + 2, std=0.02)
        r1, tr = timed(lambda: oracle.route(i1, 0, cs.E, cs.K, p1, cs.pad))
        P1, tp = timed(lambda: oracle.permute_rows(x1, r1["row_id"], r1["R"]))
        ns = 64
        _, tm = timed(lambda: oracle.layer_tokens(np.arange(ns), x1, r1,
                                                  lambda e, rows: oracle.expert_mlp_bf16(rows, a1[e], b1[e])))
        _, tc = timed(lambda: oracle.combine_bf16(P1, r1["row_id"], r1["copy_prob"]))
        t_small = tr + tp + tm * cs.T / ns + tc
        one["small_layer_512x1024"] = {
            "tokens_per_s": round(cs.T / t_small, 1), "preprocess_s": round(tr, 4), "permute_s": round(tp, 4),
            "mlp_s_est": round(tm * cs.T / ns, 3), "combine_s": round(tc, 4),
            "sample": f"routing, permute, combine on all {cs.T} tokens; MLP on {ns} tokens, scaled"}
        del P1
        c2 = S.CONFIGS["permute_combine_8192x7168_e32"]
        i2, p2 = S.route_uniform_distinct(c2.T, c2.E, c2.K, c2.seed)
        x2 = S.bf16_normal((c2.T, c2.H), c2.seed)
        cap = oracle.capacity_from_rows(int(oracle.route(i2, 0, c2.E, c2.K, p2)["counts"].max()), 1.5)
        r2, tr = timed(lambda: oracle.route(i2, 0, c2.E, c2.K, p2, 1, cap))
        P2, tp = timed(lambda: oracle.permute_rows(x2, r2["row_id"], r2["R"]))
        _, tc = timed(lambda: oracle.combine_bf16(P2, r2["row_id"], r2["copy_prob"]))
        nb = (c2.T + c2.T * c2.K) * c2.H * 2
        one["permute_combine_8192x7168_e32"] = {
            "preprocess_s": round(tr, 4), "permute_s": round(tp, 4), "combine_s": round(tc, 4),
            "permute_GB_s": round(nb / tp / 1e9, 2), "combine_GB_s": round(nb / tc / 1e9, 2),
            "sample": "whole batch, capacity 1.5x, identity experts"}
        del P2, x2
        c5 = S.CONFIGS["decode_fp8_7168_e256"]
        i5, p5 = S.route_sigmoid_topk(16, c5.E, c5.K, c5.seed + 16)
        x5 = S.bf16_normal((16, c5.H), c5.seed + 16)
        r5, tr = timed(lambda: oracle.route(i5, 0, c5.E, c5.K, p5, c5.pad))
        P5, tp = timed(lambda: oracle.permute_rows(x5, r5["row_id"], r5["R"]))
        ns5 = 4
        need = sorted({int(e) for e in r5["copy_expert"][:ns5].reshape(-1) if e >= 0})
        wa, wb = _decode_weights_host(c5, need)
        tm5 = 0.0
        for e in need:
            rows = [t for t in range(ns5) for j in range(c5.K) if r5["row_id"][t, j] >= 0
                    and int(r5["copy_expert"][t, j]) == e]
            _, t = timed(lambda: oracle.expert_mlp_fp8(x5[rows], *wa[e], *wb[e]))
            tm5 += t
        _, tc = timed(lambda: oracle.combine_bf16(P5, r5["row_id"], r5["copy_prob"]))
        t_dec = tr + tp + tm5 * 16 / ns5 + tc
        one["decode_fp8_16_tokens"] = {
            "tokens_per_s": round(16 / t_dec, 2), "mlp_s_est": round(tm5 * 16 / ns5, 3),
            "sample": f"16-token bucket: routing, permute, combine on all tokens; fp8 MLP (dequantised fp64 "
                      f"loops) on {ns5} tokens, scaled"}
        cpu["single_thread"] = one
    finally:
        oracle.set_threads(threads)
    cpu["wall_s"] = round(time.perf_counter() - t_start, 1)
    return cpu


def _decode_weights_host(c5, experts):
    """Host copies of the decode workload's fp8 expert weights for the listed
    experts: the same draws as ``weights_fp8_blocks`` on the device, read back
    expert by expert.  Returns ({e: (w1q, w1s)}, {e: (w2q, w2s)}) with the
    tuples ordered as ``oracle.expert_mlp_fp8`` takes them."""
    import torch

    import moe_synth as S
    w1q, w1s = S.weights_fp8_blocks(c5.E, 2 * c5.F, c5.H, c5.seed + 1, device="cuda")
    w2q, w2s = S.weights_fp8_blocks(c5.E, c5.H, c5.F, c5.seed + 2, device="cuda")
    a = {e: (w1q[e].cpu().numpy(), w1s[e].cpu().numpy()) for e in experts}
    b = {e: (w2q[e].cpu().numpy(), w2s[e].cpu().numpy()) for e in experts}
    del w1q, w1s, w2q, w2s
    torch.cuda.empty_cache()
    return a, b


def _require_clear_flag(d, routing, probs=None, T_live=None):
    """Eager routing preprocessing with a host check that the overflow flag is
    clear, before any step that enqueues the device-side assert on it."""
    import torch
    d.preprocess(routing, probs, T_live)
    torch.cuda.synchronize()
    flag = int(d.flag.item())
    if flag != 0:
        raise RuntimeError(f"routing sets the overflow flag ({flag})")


def _graph_times(step, reps=30):
    """Capture `step` in a HIP graph, replay it; min / median ms per replay."""
    import statistics as st
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(5):
        g.replay()
    torch.cuda.synchronize()
    t = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        b.synchronize()
        t.append(a.elapsed_time(b))
    return min(t), st.median(t)


_FLUSH = []


def _flush_caches():
    """Evict the last-level caches (256 MB memory-side cache, 4 MB L2 per
    XCD): a 512 MB device copy, enqueued outside any timed region."""
    import torch
    if not _FLUSH:
        _FLUSH.append(torch.empty(2 ** 29, dtype=torch.uint8, device="cuda"))
        _FLUSH.append(torch.empty(2 ** 29, dtype=torch.uint8, device="cuda"))
    _FLUSH[1].copy_(_FLUSH[0])


def _event_times(fn, reps=30, warm=5, flush=False):
    """min / median ms of `fn` over `reps` runs; with `flush`, caches are
    evicted before every run so inputs come from HBM (cold)."""
    import statistics as st
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    t = []
    for _ in range(reps):
        if flush:
            _flush_caches()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        b.synchronize()
        t.append(a.elapsed_time(b))
    return min(t), st.median(t)


def _calib_copy():
    """One device-to-device copy of exactly 1 GiB: the reference dispatch that
    scales hardware byte counters to bytes."""
    import torch
    a = torch.empty(2 ** 29, dtype=torch.int16, device="cuda")
    a.fill_(1)
    bq = torch.empty_like(a)
    torch.cuda.synchronize()
    bq.copy_(a)
    torch.cuda.synchronize()


def run_decode(args):
    """Decode-sized layer with fp8 weights, eager launches: routing metadata,
    permute, FC1 + SwiGLU, FC2, combine for `--tokens` live tokens in the
    next power-of-two bucket.  One JSON line (milliseconds per layer)."""
    import numpy as np
    import torch

    import moe_synth as S
    from combine_routing_preprocess_amd import Dispatcher
    dev = "cuda"
    c = S.CONFIGS["decode_fp8_7168_e256"]
    T_live = args.tokens
    T = S.next_pow2_bucket(T_live)
    log(f"drawing fp8 weights; {T_live} live tokens in bucket {T}")
    w1q, w1s = S.weights_fp8_blocks(c.E, 2 * c.F, c.H, c.seed + 1, device=dev)
    w2q, w2s = S.weights_fp8_blocks(c.E, c.H, c.F, c.seed + 2, device=dev)
    idx, pr = S.route_sigmoid_topk(T, c.E, c.K, c.seed + T)
    x = torch.from_numpy(S.bf16_normal((T, c.H), c.seed + T).view(np.int16)).to(dev).view(torch.bfloat16)
    d = Dispatcher(T, c.H, c.E, c.K, pad_multiple=c.pad)
    rt, pt = torch.from_numpy(idx).to(dev), torch.from_numpy(pr).to(dev)
    tl = torch.tensor([T_live], dtype=torch.int32, device=dev)
    perm = torch.empty((d.R, c.H), dtype=torch.bfloat16, device=dev)
    scr = d.alloc_mlp_scratch(c.F, "fp8")
    eo = torch.empty((d.R, c.H), dtype=torch.bfloat16, device=dev)
    y = torch.empty((T, c.H), dtype=torch.bfloat16, device=dev)

    status = torch.zeros((1,), dtype=torch.int32, device=dev)
    if args.decode_path == "fused":
        scr = torch.empty(d.decode_fused_scratch_bytes(c.F), dtype=torch.uint8, device=dev)

        def step():
            d.preprocess(rt, pt, tl)
            d.decode_fused_fp8(x, w1q, w2q, w1s, w2s, scratch=scr, expert_out=eo, out=y)
    elif args.decode_path == "persistent":
        scr = torch.empty(d.decode_layer_scratch_bytes(c.F), dtype=torch.uint8, device=dev)

        def step():
            d.preprocess(rt, pt, tl)
            d.decode_layer_fp8(x, w1q, w2q, w1s, w2s, scratch=scr, expert_out=eo, out=y, status=status)
    else:
        # routing, quantise-on-dispatch, FC1, row quantiser, FC2, combine
        d = Dispatcher(T, c.H, c.E, c.K, pad_multiple=c.pad, payload="fp8")
        perm = torch.empty((d.R, c.H), dtype=torch.uint8, device=dev)
        perm_s = torch.empty((d.R, c.H // 128), dtype=torch.float32, device=dev)

        def step():
            d.layer(x, rt, pt, w1q, w2q, w1_scales=w1s, w2_scales=w2s, perm=perm, perm_scales=perm_s, scratch=scr,
                    expert_out=eo, out=y, T_live=tl, check_overflow=True)

    _require_clear_flag(d, rt, pt, tl)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    st = int(status.item())
    if args.calib_copy:
        _calib_copy()
    print(json.dumps({"workload": f"decode_fp8: {T_live} live tokens (bucket {T}) x {c.H}, {c.E} experts top-{c.K}, "
                                  f"FFN {c.F}, fp8 e4m3 weights", "path": args.decode_path,
                      "ms_per_layer_eager": round(ms, 4), "status": st,
                      "steps": args.steps}), flush=True)
    return 0 if st == 0 else 1


def run_workloads():
    """The other synthetic workloads, each timed on its own: the small layer
    per stage, the 32-expert permute/combine at capacity 1.5x and at the
    overflow capacity (max - 1), the fp8 routing stress in both routing
    formats, and the fp8 decode buckets (graph replay)."""
    import numpy as np
    import torch

    import moe_synth as S
    import oracle
    from combine_routing_preprocess_amd import Dispatcher, assert_no_overflow
    dev = "cuda"
    res = {}

    # ---- small layer: 512 x 1024, 16 experts top-4, padding 32, FFN 512 ------
    log("workload: small layer")
    c = S.CONFIGS["small_layer_512x1024"]
    idx, pr = S.route_softmax_topk(c.T, c.E, c.K, c.seed)
    x = torch.from_numpy(S.bf16_normal((c.T, c.H), c.seed).view(np.int16)).to(dev).view(torch.bfloat16)
    w1 = S.weights_bf16(c.E, 2 * c.F, c.H, c.seed + 1, device=dev)
    w2 = S.weights_bf16(c.E, c.H, c.F, c.seed + 2, device=dev)
    d = Dispatcher(c.T, c.H, c.E, c.K, pad_multiple=c.pad)
    rt, pt = torch.from_numpy(idx).to(dev), torch.from_numpy(pr).to(dev)
    perm = torch.empty((d.R, c.H), dtype=torch.bfloat16, device=dev)
    scr = d.alloc_mlp_scratch(c.F)
    eo = torch.empty((d.R, c.H), dtype=torch.bfloat16, device=dev)
    y = torch.empty((c.T, c.H), dtype=torch.bfloat16, device=dev)
    _require_clear_flag(d, rt, pt)
    d.permute(x, out=perm)
    d.fc1(perm, w1, scr)
    st = {}
    for name, fn in (("preprocess", lambda: d.preprocess(rt, pt)), ("permute", lambda: d.permute(x, out=perm)),
                     ("fc1_swiglu", lambda: d.fc1(perm, w1, scr)), ("fc2", lambda: d.fc2(w2, scr, eo)),
                     ("combine", lambda: d.combine(eo, out=y))):
        mn, md = _event_times(fn, reps=50)
        st[name] = {"min_us": round(mn * 1e3, 1), "median_us": round(md * 1e3, 1)}
    gm, gmed = _graph_times(lambda: d.layer(x, rt, pt, w1, w2, perm=perm, scratch=scr, expert_out=eo, out=y,
                                            check_overflow=True), reps=50)
    res["small_layer_512x1024"] = {"stages": st, "graph_layer_min_us": round(gm * 1e3, 1),
                                   "graph_layer_median_us": round(gmed * 1e3, 1),
                                   "tokens_per_s": round(c.T / (gm * 1e-3), 1)}
    del d, perm, scr, eo, y, w1, w2, x

    # ---- permute + combine: 8192 x 7168 bf16, 32 experts top-8 ---------------
    log("workload: 32-expert permute/combine")
    c = S.CONFIGS["permute_combine_8192x7168_e32"]
    idx, pr = S.route_uniform_distinct(c.T, c.E, c.K, c.seed)
    counts = oracle.route(idx, 0, c.E, c.K, pr)["counts"]
    mx = int(counts.max())
    x = torch.from_numpy(S.bf16_normal((c.T, c.H), c.seed).view(np.int16)).to(dev).view(torch.bfloat16)
    rt, pt = torch.from_numpy(idx).to(dev), torch.from_numpy(pr).to(dev)
    out2 = {}
    for name, cap, want_flag in (("capacity_1.5x", oracle.capacity_from_rows(mx, 1.5), 0),
                                 ("overflow_capacity_max_minus_1", mx - 1, 1)):
        d = Dispatcher(c.T, c.H, c.E, c.K, capacity=cap)
        perm = torch.empty((d.R, c.H), dtype=torch.bfloat16, device=dev)
        y = torch.empty((c.T, c.H), dtype=torch.bfloat16, device=dev)
        d.preprocess(rt, pt)
        torch.cuda.synchronize()
        flag = int(d.flag.item())
        assert flag == want_flag, (name, flag)
        kept = int(np.minimum(counts, cap).sum())
        nbytes = (c.T + kept) * c.H * 2
        pm, _ = _event_times(lambda: d.permute(x, out=perm), flush=True)
        cm, _ = _event_times(lambda: d.combine(perm, out=y), flush=True)
        pw, _ = _event_times(lambda: d.permute(x, out=perm))
        cw, _ = _event_times(lambda: d.combine(perm, out=y))
        km, _ = _event_times(lambda: d.preprocess(rt, pt), flush=True)
        r = {"capacity": cap, "max_count": mx, "kept_copies": kept, "flag": flag,
             "preprocess_min_us": round(km * 1e3, 1),
             "permute_min_ms": round(pm, 4), "combine_min_ms": round(cm, 4),
             "permute_GB_s": round(nbytes / (pm * 1e-3) / 1e9, 1), "combine_GB_s": round(nbytes / (cm * 1e-3) / 1e9, 1),
             "permute_frac_of_peak": round(nbytes / (pm * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
             "combine_frac_of_peak": round(nbytes / (cm * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
             "permute_warm_GB_s": round(nbytes / (pw * 1e-3) / 1e9, 1),
             "combine_warm_GB_s": round(nbytes / (cw * 1e-3) / 1e9, 1)}
        if want_flag == 0:
            gm, gmed = _graph_times(lambda: (d.dispatch(x, rt, pt, out=perm), d.combine(perm, out=y),
                                             assert_no_overflow(d.flag)))
            r.update({"graph_dispatch_combine_min_ms": round(gm, 4), "graph_median_ms": round(gmed, 4)})
        out2[name] = r
        del d, perm, y
    out2["timing"] = "cold caches (512 MB copy before each run); warm = repeated runs"
    res["permute_combine_8192x7168_e32"] = out2
    del x

    # ---- routing stress: 256 experts top-36 Zipf, fp8 payload ------------------
    log("workload: fp8 routing stress")
    c = S.CONFIGS["route_stress_fp8_8192x7168_e256"]
    idx, _ = S.route_zipf_gumbel(c.T, c.E, c.K, c.seed)
    m, _ = S.dense_to_sparse(idx, c.E)
    xq, xs = S.quantize_rows_fp8_torch(S.bf16_normal((c.T, c.H), c.seed))
    xq, xs = torch.from_numpy(xq).to(dev), torch.from_numpy(xs).to(dev)
    out3 = {}
    for name, routing, fmt in (("dense_i16", idx, "dense_i16"), ("sparse_bool", m, "sparse_bool")):
        d = Dispatcher(c.T, c.H, c.E, c.K, route_fmt=fmt, payload="fp8")
        r = torch.from_numpy(routing).to(dev)
        po = torch.empty((d.R, c.H), dtype=torch.uint8, device=dev)
        so = torch.empty((d.R, c.H // 128), dtype=torch.float32, device=dev)
        km, kmed = _event_times(lambda: d.preprocess(r), flush=True)
        pmn, _ = _event_times(lambda: d.permute(xq, xs, out=po, out_scales=so), flush=True)
        nb = (c.T + c.T * c.K) * (c.H + 4 * c.H // 128)
        out3[name] = {"routing_bytes": int(routing.nbytes), "preprocess_min_us": round(km * 1e3, 1),
                      "preprocess_median_us": round(kmed * 1e3, 1), "permute_min_ms": round(pmn, 4),
                      "permute_GB_s": round(nb / (pmn * 1e-3) / 1e9, 1),
                      "permute_frac_of_peak": round(nb / (pmn * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del d, po, so
    out3["timing"] = "cold caches"
    res["route_stress_fp8_8192x7168_e256"] = out3
    del xq, xs

    # ---- decode buckets, fp8 weights, graph replay ------------------------------
    log("workload: fp8 decode buckets")
    c = S.CONFIGS["decode_fp8_7168_e256"]
    w1q, w1s = S.weights_fp8_blocks(c.E, 2 * c.F, c.H, c.seed + 1, device=dev)
    w2q, w2s = S.weights_fp8_blocks(c.E, c.H, c.F, c.seed + 2, device=dev)
    per_expert = (2 * c.F * c.H + c.H * c.F) + 4 * (2 * c.F // 128 * c.H // 128 + c.H // 128 * c.F // 128)
    out5 = {}
    for T in (16, 64, 256):
        idx, pr = S.route_sigmoid_topk(T, c.E, c.K, c.seed + T)
        x = torch.from_numpy(S.bf16_normal((T, c.H), c.seed + T).view(np.int16)).to(dev).view(torch.bfloat16)
        # separate launches: routing, quantise-on-dispatch, FC1, row quantiser, FC2, combine
        d = Dispatcher(T, c.H, c.E, c.K, pad_multiple=c.pad, payload="fp8")
        rt, pt = torch.from_numpy(idx).to(dev), torch.from_numpy(pr).to(dev)
        perm = torch.empty((d.R, c.H), dtype=torch.uint8, device=dev)
        perm_s = torch.empty((d.R, c.H // 128), dtype=torch.float32, device=dev)
        scr = d.alloc_mlp_scratch(c.F, "fp8")
        eo = torch.empty((d.R, c.H), dtype=torch.bfloat16, device=dev)
        y = torch.empty((T, c.H), dtype=torch.bfloat16, device=dev)
        step = lambda: d.layer(x, rt, pt, w1q, w2q, w1_scales=w1s, w2_scales=w2s, perm=perm, perm_scales=perm_s,
                               scratch=scr, expert_out=eo, out=y, check_overflow=True)
        _require_clear_flag(d, rt, pt)
        gm, gmed = _graph_times(step)
        touched = int((oracle.route(idx, 0, c.E, c.K, pr, c.pad)["counts"] > 0).sum())
        wbytes = touched * per_expert
        # the fused decode layer: preprocess + quantise-on-dispatch + one persistent kernel
        df = Dispatcher(T, c.H, c.E, c.K, pad_multiple=c.pad)
        fscr = torch.empty(df.decode_fused_scratch_bytes(c.F), dtype=torch.uint8, device=dev)
        feo = torch.empty((df.R, c.H), dtype=torch.bfloat16, device=dev)
        fy = torch.empty((T, c.H), dtype=torch.bfloat16, device=dev)

        def fstep():
            df.preprocess(rt, pt)
            df.decode_fused_fp8(x, w1q, w2q, w1s, w2s, scratch=fscr, expert_out=feo, out=fy)

        fm, fmed = _graph_times(fstep)
        torch.cuda.synchronize()
        same = bool(torch.equal(fy.view(torch.int16), y.view(torch.int16)))
        # the persistent decode kernel: preprocess + one launch (dispatch, FC1, FC2, combine)
        dp = Dispatcher(T, c.H, c.E, c.K, pad_multiple=c.pad)
        pscr = torch.empty(dp.decode_layer_scratch_bytes(c.F), dtype=torch.uint8, device=dev)
        peo = torch.empty((dp.R, c.H), dtype=torch.bfloat16, device=dev)
        py = torch.empty((T, c.H), dtype=torch.bfloat16, device=dev)
        pst = torch.zeros((1,), dtype=torch.int32, device=dev)

        def pstep():
            dp.preprocess(rt, pt)
            dp.decode_layer_fp8(x, w1q, w2q, w1s, w2s, scratch=pscr, expert_out=peo, out=py, status=pst)

        pm, pmed = _graph_times(pstep)
        torch.cuda.synchronize()
        psame = bool(torch.equal(py.view(torch.int16), y.view(torch.int16)))
        pstatus = int(pst.item())
        out5[f"T{T}"] = {"graph_min_ms": round(gm, 4), "graph_median_ms": round(gmed, 4),
                         "tokens_per_s": round(T / (gm * 1e-3), 1), "experts_touched": touched,
                         "weight_bytes": wbytes, "weight_GB_s": round(wbytes / (gm * 1e-3) / 1e9, 1),
                         "frac_of_hbm_roofline": round(wbytes / (gm * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "fused": {"graph_min_ms": round(fm, 4), "graph_median_ms": round(fmed, 4),
                                   "tokens_per_s": round(T / (fm * 1e-3), 1),
                                   "weight_GB_s": round(wbytes / (fm * 1e-3) / 1e9, 1),
                                   "frac_of_hbm_roofline": round(wbytes / (fm * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                   "bit_identical_to_separate": same},
                         "persistent": {"graph_min_ms": round(pm, 4), "graph_median_ms": round(pmed, 4),
                                        "tokens_per_s": round(T / (pm * 1e-3), 1),
                                        "weight_GB_s": round(wbytes / (pm * 1e-3) / 1e9, 1),
                                        "frac_of_hbm_roofline": round(wbytes / (pm * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                        "bit_identical_to_separate": psame, "status": pstatus}}
        del d, perm, perm_s, scr, eo, y, df, fscr, feo, fy, dp, pscr, peo, py, pst
    res["decode_fp8_7168_e256"] = out5
    del w1q, w1s, w2q, w2s
    torch.cuda.empty_cache()
    return res


def run_extra(args):
    """The next-row features at the layer shape: the backward of dispatch and
    combine, and the fp8 formats (quantise-on-dispatch, FC2 into the fp8
    combine format, the fp8 combine) against their bf16 counterparts."""
    import numpy as np
    import torch

    import moe_synth as S
    from combine_routing_preprocess_amd import Dispatcher
    dev = "cuda"
    res = {}

    # backward of dispatch and combine at the layer shape, cold caches
    log("extra: backward")
    c = S.CONFIGS["dsv3_layer_8192x7168_e256"]
    idx, pr = S.route_sigmoid_topk(c.T, c.E, c.K, c.seed)
    d = Dispatcher(c.T, c.H, c.E, c.K, pad_multiple=c.pad)
    d.preprocess(torch.from_numpy(idx).to(dev), torch.from_numpy(pr).to(dev))
    gen = torch.Generator(device=dev)
    gen.manual_seed(c.seed + 50)
    G = torch.randn((d.R, c.H), generator=gen, device=dev).to(torch.bfloat16)
    Yb = torch.randn((d.R, c.H), generator=gen, device=dev).to(torch.bfloat16)
    gy = torch.randn((c.T, c.H), generator=gen, device=dev).to(torch.bfloat16)
    gop = torch.randn(d.R, generator=gen, device=dev)
    gx = torch.empty((c.T, c.H), dtype=torch.bfloat16, device=dev)
    gY = torch.empty_like(G)
    gp = torch.empty((c.T, c.K), dtype=torch.float32, device=dev)
    gq = torch.empty((c.T, c.K), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    n_copies = int(d.kept.sum().item())
    db, _ = _event_times(lambda: d.dispatch_backward(G, gop, out=gx, grad_probs=gp), flush=True)
    cb, _ = _event_times(lambda: d.combine_backward(gy, Yb, True, out=gY, grad_probs=gq), flush=True)
    db_bytes = n_copies * c.H * 2 + c.T * c.H * 2 + n_copies * 4 + c.T * c.K * 4
    cb_bytes = c.T * c.H * 2 + 2 * n_copies * c.H * 2 + c.T * c.K * 4
    res["backward_dsv3_shape"] = {
        "copies": n_copies, "timing": "cold caches",
        "dispatch_backward_min_ms": round(db, 4), "dispatch_backward_GB_s": round(db_bytes / (db * 1e-3) / 1e9, 1),
        "combine_backward_min_ms": round(cb, 4), "combine_backward_GB_s": round(cb_bytes / (cb * 1e-3) / 1e9, 1),
        "alg_bytes": {"dispatch_backward": db_bytes, "combine_backward": cb_bytes}}
    del d, G, Yb, gy, gop, gx, gY, gp, gq

    # fp8 formats at the layer shape
    log("extra: fp8 formats")
    x = torch.from_numpy(S.bf16_normal((c.T, c.H), c.seed).view(np.int16)).to(dev).view(torch.bfloat16)
    rt, pt = torch.from_numpy(idx).to(dev), torch.from_numpy(pr).to(dev)
    w1 = S.weights_bf16(c.E, 2 * c.F, c.H, c.seed + 1, device=dev)
    w2 = S.weights_bf16(c.E, c.H, c.F, c.seed + 2, device=dev)
    dq = Dispatcher(c.T, c.H, c.E, c.K, payload="fp8", pad_multiple=c.pad)
    dq.preprocess(rt, pt)
    pq = torch.empty((dq.R, c.H), dtype=torch.uint8, device=dev)
    ps = torch.empty((dq.R, c.H // 128), dtype=torch.float32, device=dev)
    d = Dispatcher(c.T, c.H, c.E, c.K, pad_multiple=c.pad)
    perm = torch.empty((d.R, c.H), dtype=torch.bfloat16, device=dev)
    d.dispatch(x, rt, pt, out=perm)
    scr = d.alloc_mlp_scratch(c.F)
    eo = torch.empty((d.R, c.H), dtype=torch.bfloat16, device=dev)
    eq = torch.empty((d.R, c.H), dtype=torch.uint8, device=dev)
    es = torch.empty((d.R, c.H // 128), dtype=torch.float32, device=dev)
    y = torch.empty((c.T, c.H), dtype=torch.bfloat16, device=dev)
    d.fc1(perm, w1, scr)
    torch.cuda.synchronize()
    n_copies = int(d.kept.sum().item())
    row8 = c.H + 4 * c.H // 128
    pqm, _ = _event_times(lambda: dq.permute_quantize(x, out=pq, out_scales=ps), flush=True)
    f2b, _ = _event_times(lambda: d.fc2(w2, scr, eo), reps=10, warm=2)
    f2q, _ = _event_times(lambda: d.fc2_fp8out(w2, scr, out=eq, out_scales=es), reps=10, warm=2)
    cbm, _ = _event_times(lambda: d.combine(eo, out=y), flush=True)
    cqm, _ = _event_times(lambda: d.combine_fp8(eq, es, out=y), flush=True)

    def layer_q():
        d.dispatch(x, rt, pt, out=perm)
        d.fc1(perm, w1, scr)
        d.fc2_fp8out(w2, scr, out=eq, out_scales=es)
        d.combine_fp8(eq, es, out=y)

    def layer_b():
        d.dispatch(x, rt, pt, out=perm)
        d.fc1(perm, w1, scr)
        d.fc2(w2, scr, eo)
        d.combine(eo, out=y)

    lq, _ = _event_times(layer_q, reps=8, warm=2)
    lb, _ = _event_times(layer_b, reps=8, warm=2)
    qb = c.T * c.H * 2 + n_copies * row8
    cb8 = n_copies * row8 + c.T * c.H * 2
    res["fp8_formats_dsv3_shape"] = {
        "timing": "row copies with cold caches; GEMMs and layers warm (25 GB of weights stream anyway)",
        "permute_quantize_min_ms": round(pqm, 4), "permute_quantize_GB_s": round(qb / (pqm * 1e-3) / 1e9, 1),
        "fc2_bf16_out_min_ms": round(f2b, 4), "fc2_fp8_out_min_ms": round(f2q, 4),
        "combine_bf16_min_ms": round(cbm, 4), "combine_fp8_min_ms": round(cqm, 4),
        "combine_fp8_GB_s": round(cb8 / (cqm * 1e-3) / 1e9, 1),
        "layer_bf16_combine_min_ms": round(lb, 4), "layer_fp8_combine_min_ms": round(lq, 4),
        "alg_bytes": {"permute_quantize": qb, "combine_fp8": cb8}}
    del dq, pq, ps, d, perm, scr, eo, eq, es, y, w1, w2, x
    torch.cuda.empty_cache()
    return res


if __name__ == "__main__":
    sys.exit(main())
