"""Seeded synthetic inputs for the MoE dispatch -> grouped MLP -> combine path.

This module is shared by the CPU oracle tests, the GPU parity tests and the
benchmark.  It only draws random numbers and shapes them into routing tables,
token rows and expert weights; it contains none of the dispatch, MLP or
combine arithmetic (that lives, independently, in ``oracle/`` and in the HIP
library).

Workload shapes follow the pages:
  * 512 tokens/rank, hidden 1024, padding multiple 32 -- DeepEP PR #716
    ("perf: reuse HybridEP routing allgather buffer"), section
    "Full HybridEP reference validation" (expert count / top-k scaled to 16 / 4);
  * 8192 x 7168 tokens, 32 local experts, top-8, random routing, capacity
    1x / 1.5x / 2x -- NeMo-Automodel PR #3931 ("sync-free HybridEP dispatch"),
    section "Validation";
  * 8192 x 7168, 256 experts, top-36, sparse Boolean and dense int16 routing
    -- DeepEP PR #716, sections "Memory impact" and "Harry Zhou's standalone
    allgather stress test";
  * DeepSeek-V3-shaped layer (7168 hidden, 256 experts, top-8) -- Megatron-LM
    PR #6800 ("Reuse caller-owned HybridEP dispatch and expert output
    buffers"), section "Motivation";
  * decode buckets with fp8 weights -- TensorRT-LLM PR #16190 ("Update CuTeDSL
    MegaMoE kernels"), first commit message (adaptive max-tokens bucketing).

Conventions: bf16 tensors are numpy ``uint16`` bit patterns, fp8 e4m3 tensors
are ``uint8`` codes, scales are ``float32``.  Dense routing is ``int16``
``[T, K]`` (``-1`` = empty slot); sparse routing is ``uint8`` ``[T, E]``
(nonzero = routed).  Probabilities are ``float32`` with the routing's shape.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

__all__ = [
    "Config", "CONFIGS", "rng", "bf16_normal", "bf16_to_float",
    "route_softmax_topk", "route_uniform_distinct", "route_zipf_gumbel",
    "route_sigmoid_topk", "dense_to_sparse", "quantize_rows_fp8_torch",
    "weights_bf16", "weights_fp8_blocks", "next_pow2_bucket",
]


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    T: int
    H: int
    E: int
    K: int
    F: int            # expert FFN width (0 = identity experts / no MLP)
    pad: int          # padding multiple
    seed: int


# The five synthetic workloads.  ``seed`` is 1000 + index.
CONFIGS = {
    "small_layer_512x1024": Config("small_layer_512x1024", T=512, H=1024, E=16, K=4, F=512, pad=32, seed=1001),
    "permute_combine_8192x7168_e32": Config("permute_combine_8192x7168_e32", T=8192, H=7168, E=32, K=8, F=0, pad=1, seed=1002),
    "route_stress_fp8_8192x7168_e256": Config("route_stress_fp8_8192x7168_e256", T=8192, H=7168, E=256, K=36, F=0, pad=1, seed=1003),
    "dsv3_layer_8192x7168_e256": Config("dsv3_layer_8192x7168_e256", T=8192, H=7168, E=256, K=8, F=2048, pad=128, seed=1004),
    "decode_fp8_7168_e256": Config("decode_fp8_7168_e256", T=256, H=7168, E=256, K=8, F=2048, pad=16, seed=1005),
}


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def _torch_gen(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def bf16_normal(shape, seed: int, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) values rounded to bf16 (torch's round-to-nearest-even cast);
    returned as uint16 bit patterns."""
    t = torch.randn(*shape, generator=_torch_gen(seed), dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_to_float(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _topk_desc(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest scores per row, in descending score order;
    ties go to the lower expert id (stable sort on the negated score)."""
    order = np.argsort(-scores, axis=1, kind="stable")
    return order[:, :k]


def route_softmax_topk(T: int, E: int, K: int, seed: int):
    """Router of the small layer: N(0,1) logits, softmax over all experts,
    top-K; probabilities are the selected softmax values (not renormalised)."""
    r = rng(seed)
    logits = r.standard_normal((T, E)).astype(np.float64)
    sm = np.exp(logits - logits.max(axis=1, keepdims=True))
    sm /= sm.sum(axis=1, keepdims=True)
    idx = _topk_desc(sm, K)
    probs = np.take_along_axis(sm, idx, axis=1).astype(np.float32)
    return idx.astype(np.int16), probs


def route_uniform_distinct(T: int, E: int, K: int, seed: int):
    """K distinct experts per token, uniformly at random (order = draw order);
    probabilities = softmax of K N(0,1) logits (they sum to 1)."""
    r = rng(seed)
    keys = r.random((T, E))
    idx = np.argsort(keys, axis=1, kind="stable")[:, :K]
    lg = r.standard_normal((T, K))
    p = np.exp(lg - lg.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    return idx.astype(np.int16), p.astype(np.float32)


def route_zipf_gumbel(T: int, E: int, K: int, seed: int, s: float = 1.2):
    """Skewed routing: expert popularity w_e = (pi(e)+1)^-s for a seeded
    permutation pi; K distinct experts per token by Gumbel-top-K on log w_e.
    Probabilities = softmax of the selected perturbed keys."""
    r = rng(seed)
    perm = r.permutation(E)
    logw = -s * np.log(perm.astype(np.float64) + 1.0)
    g = r.gumbel(size=(T, E))
    keys = logw[None, :] + g
    idx = _topk_desc(keys, K)
    sel = np.take_along_axis(keys, idx, axis=1)
    p = np.exp(sel - sel.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    return idx.astype(np.int16), p.astype(np.float32)


def route_sigmoid_topk(T: int, E: int, K: int, seed: int):
    """DeepSeek-V3-style router: N(0,1) logits, sigmoid scores, top-K,
    probabilities = selected scores / their sum."""
    r = rng(seed)
    logits = r.standard_normal((T, E))
    s = 1.0 / (1.0 + np.exp(-logits))
    idx = _topk_desc(s, K)
    sel = np.take_along_axis(s, idx, axis=1)
    p = sel / sel.sum(axis=1, keepdims=True)
    return idx.astype(np.int16), p.astype(np.float32)


def dense_to_sparse(idx: np.ndarray, E: int, probs: Optional[np.ndarray] = None):
    """Re-encode dense top-k indices as a Boolean map [T,E] (and probs as a
    [T,E] table with zeros off the routed entries).  Entries equal to -1 are
    skipped."""
    T, K = idx.shape
    m = np.zeros((T, E), dtype=np.uint8)
    pe = np.zeros((T, E), dtype=np.float32) if probs is not None else None
    rows = np.repeat(np.arange(T), K)
    cols = idx.reshape(-1).astype(np.int64)
    ok = cols >= 0
    m[rows[ok], cols[ok]] = 1
    if probs is not None:
        pe[rows[ok], cols[ok]] = probs.reshape(-1)[ok]
    return m, pe


def quantize_rows_fp8_torch(x_bits: np.ndarray, block: int = 128):
    """Input synthesis for fp8 payload rows: bf16 rows -> (e4m3 codes, fp32
    scale per (row, 128 columns)), scale = amax/448 (1 when the block is all
    zero), codes by torch's float8_e4m3fn cast of x/scale."""
    x = torch.from_numpy(bf16_to_float(x_bits).copy())
    T, H = x.shape
    xb = x.view(T, H // block, block)
    amax = xb.abs().amax(dim=2)
    sc = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (xb / sc[:, :, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).reshape(T, H).numpy(), sc.numpy().astype(np.float32)


def weights_bf16(E: int, rows: int, cols: int, seed: int, std: float = 0.02, device="cpu"):
    """Expert weights [E, rows, cols] ~ N(0, std^2) as a bf16 torch tensor on
    ``device`` (seeded torch generator on that device)."""
    g = _torch_gen(seed, device)
    w = torch.empty((E, rows, cols), dtype=torch.bfloat16, device=device)
    chunk = max(1, (1 << 27) // max(1, rows * cols))
    for e0 in range(0, E, chunk):
        e1 = min(E, e0 + chunk)
        w[e0:e1] = (torch.randn((e1 - e0, rows, cols), generator=g, device=device) * std).to(torch.bfloat16)
    return w


def weights_fp8_blocks(E: int, rows: int, cols: int, seed: int, std: float = 0.02, device="cpu", block: int = 128):
    """Expert weights [E, rows, cols] drawn N(0, std^2) and stored as e4m3
    codes (uint8 torch tensor) with one fp32 scale per 128x128 block
    ([E, rows/128, cols/128]); scale = block amax / 448."""
    assert rows % block == 0 and cols % block == 0
    g = _torch_gen(seed, device)
    q = torch.empty((E, rows, cols), dtype=torch.uint8, device=device)
    sc = torch.empty((E, rows // block, cols // block), dtype=torch.float32, device=device)
    for e in range(E):
        w = torch.randn((rows, cols), generator=g, device=device) * std
        wb = w.view(rows // block, block, cols // block, block)
        amax = wb.abs().amax(dim=(1, 3))
        s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
        qq = (wb / s[:, None, :, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
        q[e] = qq.view(torch.uint8).reshape(rows, cols)
        sc[e] = s
    return q, sc


def next_pow2_bucket(T: int, floor: int = 16) -> int:
    """Decode bucket for T live tokens: the next power of two >= T (at least
    ``floor``); T = 0 keeps the smallest bucket."""
    b = floor
    while b < T:
        b *= 2
    return b

