"""Helpers for the GPU parity tests: moving seeded numpy inputs to the GPU,
running the HIP path through the C ABI, reading results back."""
import sys

import numpy as np
import torch

import oracle
from combine_routing_preprocess_amd import Dispatcher

DEV = "cuda"
FMT_NAME = {oracle.FMT_DENSE_I16: "dense_i16", oracle.FMT_DENSE_I32: "dense_i32", oracle.FMT_SPARSE_U8: "sparse_bool"}


def log(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


def host_bf16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def gpu_route(routing, fmt, E, K, probs=None, pad=1, cap=-1, R=None, T_live=None, H=64):
    T = routing.shape[0]
    d = Dispatcher(T, H, E, K, route_fmt=FMT_NAME[fmt], pad_multiple=pad, capacity=None if cap < 0 else cap,
                   out_rows=0 if R is None else R)
    rt = dev(routing)
    pt = None if probs is None else dev(probs.astype(np.float32))
    tl = None if T_live is None else torch.tensor([T_live], dtype=torch.int32, device=DEV)
    out_probs = torch.full((max(d.R, 1),), float("nan"), dtype=torch.float32, device=DEV)
    d.preprocess(rt, pt, tl, out_probs if d.R else None)
    torch.cuda.synchronize()
    res = dict(counts=d.tokens_per_expert.cpu().numpy(), seg_off=d.seg_off.cpu().numpy(),
               row_id=d.row_id.cpu().numpy(), copy_prob=d.copy_prob.cpu().numpy(),
               src_row=d.src_row.cpu().numpy(), perm_prob=out_probs[:d.R].cpu().numpy(),
               rows_needed=int(d.rows_needed.item()), flag=int(d.flag.item()), R=d.R)
    return res, d


def assert_route_equal(g, o, what=""):
    assert g["R"] == o["R"], what
    for k in ("counts", "seg_off", "row_id", "copy_prob", "src_row", "perm_prob"):
        a, b = np.asarray(g[k]), np.asarray(o[k])
        assert a.shape == b.shape, (what, k, a.shape, b.shape)
        if a.dtype.kind == "f":
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), (what, k)
        else:
            assert np.array_equal(a, b), (what, k, np.nonzero(a != b)[0][:10])
    assert g["rows_needed"] == o["rows_needed"], what
    assert g["flag"] == o["flag"], (what, g["flag"], o["flag"])


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def row_rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    num = np.linalg.norm(a - b, axis=1)
    den = np.maximum(np.linalg.norm(b, axis=1), 1e-30)
    return num / den


def require_clear_flag(d, routing, probs=None, T_live=None):
    """Run the routing preprocessing eagerly and check on the host that the
    overflow flag is clear.  Call this before any step that enqueues the
    device-side overflow assert on these inputs: on this ROCm build a failing
    device assert aborts the queue, so the tests only assert where the flag
    is known to be clear."""
    d.preprocess(routing, probs, T_live)
    torch.cuda.synchronize()
    flag = int(d.flag.item())
    assert flag == 0, f"routing sets the overflow flag ({flag}); the device assert must not run on it"
