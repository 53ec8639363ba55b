"""CPU oracle for the MoE dispatch-permute -> grouped SwiGLU MLP -> combine path.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``, never by the product package.  The
arithmetic lives in ``moe_oracle.c`` (plain C loops, double precision); this
file only marshals numpy arrays.  See the C file for the definitions, the page
citations and the readings taken where the pages are silent.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "moe_oracle.c")

FLAG_CAPACITY = 1
FLAG_OUT_ROWS = 2
FLAG_BAD_EXPERT = 4
FLAG_DUPLICATE = 8

FMT_DENSE_I16 = 0
FMT_DENSE_I32 = 1
FMT_SPARSE_U8 = 2


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C11 + OpenMP).  The helpers are
    exported symbols; -fno-semantic-interposition lets gcc inline them into
    the loops that call them (same arithmetic, about 3x faster)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-fno-semantic-interposition", "-shared", "-std=c11",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _SO)
    return _SO


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = C.CDLL(_SO)
        P = C.c_void_p
        L.orc_bf16_from_double.restype = C.c_uint16
        L.orc_bf16_from_double.argtypes = [C.c_double]
        L.orc_bf16_to_double.restype = C.c_double
        L.orc_bf16_to_double.argtypes = [C.c_uint16]
        L.orc_e4m3_to_double.restype = C.c_double
        L.orc_e4m3_to_double.argtypes = [C.c_uint8]
        L.orc_e4m3_from_double_sat.restype = C.c_uint8
        L.orc_e4m3_from_double_sat.argtypes = [C.c_double]
        L.orc_routing_bytes.restype = C.c_int64
        L.orc_routing_bytes.argtypes = [C.c_int64, C.c_int64, C.c_int64, C.c_int32]
        L.orc_capacity_from_rows.restype = C.c_int64
        L.orc_capacity_from_rows.argtypes = [C.c_int64, C.c_double]
        L.orc_out_rows_bound.restype = C.c_int64
        L.orc_out_rows_bound.argtypes = [C.c_int32] * 5
        L.orc_route.restype = C.c_int
        L.orc_route.argtypes = [C.c_int32, C.c_int32, C.c_int32, C.c_int32, P, P, C.c_int32,
                                C.c_int32, C.c_int64, C.c_int32] + [P] * 9
        L.orc_permute_rows.restype = None
        L.orc_permute_rows.argtypes = [C.c_int32, C.c_int32, C.c_int64, P, P, P]
        L.orc_combine_bf16.restype = None
        L.orc_combine_bf16.argtypes = [C.c_int32, C.c_int32, C.c_int32, P, P, C.c_int32, P, P]
        L.orc_expert_mlp_bf16.restype = None
        L.orc_expert_mlp_bf16.argtypes = [C.c_int32, C.c_int32, C.c_int32, P, P, P, P, P, P]
        L.orc_combine_fp8.restype = None
        L.orc_combine_fp8.argtypes = [C.c_int32, C.c_int32, C.c_int32, P, P, C.c_int32, P, P, P]
        L.orc_quant_rows_e4m3_f32.restype = None
        L.orc_quant_rows_e4m3_f32.argtypes = [C.c_int32, C.c_int32, P, P, P]
        L.orc_expert_mlp_fp8.restype = None
        L.orc_expert_mlp_fp8.argtypes = [C.c_int32, C.c_int32, C.c_int32] + [P] * 6
        L.orc_dispatch_backward.restype = None
        L.orc_dispatch_backward.argtypes = [C.c_int32] * 5 + [P] * 6
        L.orc_combine_backward.restype = None
        L.orc_combine_backward.argtypes = [C.c_int32] * 5 + [P] * 3 + [C.c_int32] + [P] * 4
        L.orc_set_threads.restype = None
        L.orc_set_threads.argtypes = [C.c_int]
        L.orc_get_threads.restype = C.c_int
        L.orc_get_threads.argtypes = []
        _lib = L
    return _lib


def _p(a):
    return None if a is None else C.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))


def get_threads() -> int:
    return int(lib().orc_get_threads())


# ---- number formats ------------------------------------------------------
def bf16_from_double(v: float) -> int:
    return int(lib().orc_bf16_from_double(float(v)))


def bf16_to_double(b: int) -> float:
    return float(lib().orc_bf16_to_double(int(b)))


def e4m3_to_double(c: int) -> float:
    return float(lib().orc_e4m3_to_double(int(c)))


def e4m3_from_double(v: float) -> int:
    return int(lib().orc_e4m3_from_double_sat(float(v)))


def bf16_round_array(v: np.ndarray) -> np.ndarray:
    f = lib().orc_bf16_from_double
    flat = np.asarray(v, dtype=np.float64).reshape(-1)
    return np.fromiter((f(float(x)) for x in flat), dtype=np.uint16, count=flat.size).reshape(np.shape(v))


# ---- host helpers ----------------------------------------------------------
def routing_bytes(tokens: int, experts: int, topk: int, fmt: int) -> int:
    return int(lib().orc_routing_bytes(tokens, experts, topk, fmt))


def capacity_from_rows(rows: int, factor: float) -> int:
    return int(lib().orc_capacity_from_rows(int(rows), float(factor)))


def out_rows_bound(T: int, E: int, K: int, pad: int, cap: int) -> int:
    return int(lib().orc_out_rows_bound(T, E, K, pad, cap))


# ---- routing ---------------------------------------------------------------
def route(routing: np.ndarray, fmt: int, E: int, K: int, probs=None, pad: int = 1,
          cap: int = -1, R: int | None = None, T_live: int | None = None) -> dict:
    """Routing metadata for one dispatch; returns a dict of numpy arrays."""
    if fmt == FMT_DENSE_I16:
        routing = _c(routing, np.int16)
    elif fmt == FMT_DENSE_I32:
        routing = _c(routing, np.int32)
    else:
        routing = _c(routing, np.uint8)
    T = routing.shape[0]
    if R is None:
        R = out_rows_bound(T, E, K, pad, cap)
    if T_live is None:
        T_live = T
    pr = None if probs is None else _c(probs, np.float32)
    counts = np.zeros(E, np.int32)
    seg_off = np.zeros(E + 1, np.int64)
    row_id = np.zeros((T, K), np.int32)
    copy_prob = np.zeros((T, K), np.float32)
    copy_expert = np.zeros((T, K), np.int32)
    src_row = np.zeros(max(R, 1), np.int32)[:R]
    perm_prob = np.zeros(max(R, 1), np.float32)[:R]
    rows_needed = np.zeros(1, np.int64)
    flag = np.zeros(1, np.int32)
    rc = lib().orc_route(T, E, K, fmt, _p(routing), _p(pr), pad, cap, R, T_live,
                         _p(counts), _p(seg_off), _p(row_id), _p(copy_prob), _p(copy_expert),
                         _p(src_row), _p(perm_prob), _p(rows_needed), _p(flag))
    if rc != 0:
        raise ValueError(f"orc_route rejected its arguments (rc={rc})")
    return dict(counts=counts, seg_off=seg_off, row_id=row_id, copy_prob=copy_prob,
                copy_expert=copy_expert, src_row=src_row, perm_prob=perm_prob,
                rows_needed=int(rows_needed[0]), flag=int(flag[0]), R=int(R))


def permute_rows(x: np.ndarray, row_id: np.ndarray, R: int, fill: int = 0) -> np.ndarray:
    """out[row_id[t,j]] = x[t] for every kept copy; other rows keep ``fill``."""
    x = np.ascontiguousarray(x)
    T = x.shape[0]
    K = row_id.shape[1]
    row_bytes = x.nbytes // max(T, 1) if T else 0
    out = np.full((R,) + x.shape[1:], fill, dtype=x.dtype)
    rid = _c(row_id, np.int32)
    if T and R:
        lib().orc_permute_rows(T, K, row_bytes, _p(x), _p(rid), _p(out))
    return out


def combine_bf16(Y: np.ndarray, row_id: np.ndarray, copy_prob: np.ndarray, apply_probs: bool = True) -> np.ndarray:
    Y = _c(Y, np.uint16)
    T, K = row_id.shape
    H = Y.shape[1]
    y = np.zeros((T, H), np.uint16)
    if T:
        lib().orc_combine_bf16(T, K, H, _p(_c(row_id, np.int32)), _p(_c(copy_prob, np.float32)),
                               1 if apply_probs else 0, _p(Y), _p(y))
    return y


def dispatch_backward(grad_out: np.ndarray, rt: dict, E: int, sparse: bool, grad_out_probs=None):
    """Gradients of a dispatch: (grad_x [T,H] bf16 bits, grad_probs or None).
    grad_probs has the routing's shape ([T,K] dense, [T,E] sparse)."""
    rid = _c(rt["row_id"], np.int32)
    T, K = rid.shape
    grad_out = _c(grad_out, np.uint16)
    H = grad_out.shape[1]
    gx = np.zeros((T, H), np.uint16)
    gop = None if grad_out_probs is None else _c(grad_out_probs, np.float32)
    gp = None if gop is None else np.zeros((T, E if sparse else K), np.float32)
    if T:
        lib().orc_dispatch_backward(T, K, E, H, 1 if sparse else 0, _p(rid), _p(_c(rt["copy_expert"], np.int32)),
                                    _p(grad_out), _p(gop), _p(gx), _p(gp))
    return gx, gp


def combine_backward(grad_y: np.ndarray, Y: np.ndarray, rt: dict, E: int, sparse: bool,
                     apply_probs: bool = True, want_probs: bool = True, fill: int = 0):
    """Gradients of a combine: (grad_Y [R,H] bf16 bits, rows holding no kept
    copy keep ``fill``; grad_probs in the routing's shape, or None)."""
    rid = _c(rt["row_id"], np.int32)
    T, K = rid.shape
    grad_y = _c(grad_y, np.uint16)
    Y = _c(Y, np.uint16)
    H = grad_y.shape[1]
    R = Y.shape[0]
    gY = np.full((R, H), fill, np.uint16)
    gp = np.zeros((T, E if sparse else K), np.float32) if want_probs else None
    if T:
        lib().orc_combine_backward(T, K, E, H, 1 if sparse else 0, _p(rid), _p(_c(rt["copy_expert"], np.int32)),
                                   _p(_c(rt["copy_prob"], np.float32)), 1 if apply_probs else 0,
                                   _p(grad_y), _p(Y), _p(gY), _p(gp))
    return gY, gp


def expert_mlp_bf16(x: np.ndarray, w1: np.ndarray, w2: np.ndarray, return_a: bool = False,
                    return_y32: bool = False):
    """One expert's SwiGLU MLP over rows x [n,H] (bf16 bits); w1 [2F,H], w2 [H,F].
    Returns y (bf16 bits), plus the activations a and/or the FC2 sums rounded
    to float32 when asked."""
    x = _c(x, np.uint16)
    w1 = _c(w1, np.uint16)
    w2 = _c(w2, np.uint16)
    n, H = x.shape
    F = w1.shape[0] // 2
    y = np.zeros((n, H), np.uint16)
    a = np.zeros((n, F), np.uint16) if return_a else None
    y32 = np.zeros((n, H), np.float32) if return_y32 else None
    if n:
        lib().orc_expert_mlp_bf16(n, H, F, _p(x), _p(w1), _p(w2), _p(y), _p(a), _p(y32))
    out = (y,) + ((a,) if return_a else ()) + ((y32,) if return_y32 else ())
    return out if len(out) > 1 else y


def combine_fp8(Yq: np.ndarray, Ys: np.ndarray, row_id: np.ndarray, copy_prob: np.ndarray,
                apply_probs: bool = True) -> np.ndarray:
    """Combine from fp8 expert-output rows (e4m3 codes [R,H], scales [R,H/128])."""
    Yq = _c(Yq, np.uint8)
    Ys = _c(Ys, np.float32)
    T, K = row_id.shape
    H = Yq.shape[1]
    y = np.zeros((T, H), np.uint16)
    if T:
        lib().orc_combine_fp8(T, K, H, _p(_c(row_id, np.int32)), _p(_c(copy_prob, np.float32)),
                              1 if apply_probs else 0, _p(Yq), _p(Ys), _p(y))
    return y


def quant_rows_e4m3(x: np.ndarray):
    x = _c(x, np.float32)
    n, cols = x.shape
    q = np.zeros((n, cols), np.uint8)
    s = np.zeros((n, cols // 128), np.float32)
    if n:
        lib().orc_quant_rows_e4m3_f32(n, cols, _p(x), _p(q), _p(s))
    return q, s


def expert_mlp_fp8(x: np.ndarray, w1q, w1s, w2q, w2s) -> np.ndarray:
    x = _c(x, np.uint16)
    w1q = _c(w1q, np.uint8)
    w1s = _c(w1s, np.float32)
    w2q = _c(w2q, np.uint8)
    w2s = _c(w2s, np.float32)
    n, H = x.shape
    F = w1q.shape[0] // 2
    y = np.zeros((n, H), np.uint16)
    if n:
        lib().orc_expert_mlp_fp8(n, H, F, _p(x), _p(w1q), _p(w1s), _p(w2q), _p(w2s), _p(y))
    return y


def layer_tokens(tokens, x, rt: dict, expert_fn, apply_probs: bool = True) -> np.ndarray:
    """Full-layer output rows for the listed tokens: each kept copy (t, j) runs
    through its expert (``expert_fn(e, rows) -> bf16 rows``), then the
    token's copies are combined.  Each output row depends only on its own
    token, so a sample of tokens can be checked at any problem size."""
    tokens = np.asarray(tokens, dtype=np.int64)
    K = rt["row_id"].shape[1]
    H = x.shape[1]
    need = {}
    for t in tokens:
        for j in range(K):
            if rt["row_id"][t, j] >= 0:
                need.setdefault(int(rt["copy_expert"][t, j]), []).append(int(t))
    Yrows = {}
    for e, ts in need.items():
        ys = expert_fn(e, x[np.asarray(ts)])
        for t, yr in zip(ts, ys):
            Yrows[(t, e)] = yr
    # one pseudo expert-output table with K rows per sampled token
    n = len(tokens)
    Y = np.zeros((max(n * K, 1), H), np.uint16)
    rid = np.full((n, K), -1, np.int32)
    cp = np.zeros((n, K), np.float32)
    for i, t in enumerate(tokens):
        for j in range(K):
            if rt["row_id"][t, j] >= 0:
                Y[i * K + j] = Yrows[(int(t), int(rt["copy_expert"][t, j]))]
                rid[i, j] = i * K + j
                cp[i, j] = rt["copy_prob"][t, j]
    return combine_bf16(Y, rid, cp, apply_probs)
