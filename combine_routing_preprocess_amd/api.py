"""torch-facing binding of the C ABI (argument marshalling only).

torch supplies device memory and the current HIP stream; every computation
is a kernel of libmoe_route.so.  Shapes are fixed per ``Dispatcher`` (the
handle is initialised once, like a static-shape buffer), and no call reads a
device value back to the host.
"""
from __future__ import annotations

import ctypes as C
from typing import Optional

import torch

from . import _abi as A

_FMT = {"dense_i16": A.ROUTE_DENSE_I16, "dense_i32": A.ROUTE_DENSE_I32, "sparse_bool": A.ROUTE_SPARSE_BOOL}
_FMT_DTYPES = {A.ROUTE_DENSE_I16: (torch.int16,), A.ROUTE_DENSE_I32: (torch.int32,),
               A.ROUTE_SPARSE_BOOL: (torch.uint8, torch.bool, torch.int8)}
_DT = {"bf16": A.BF16, "fp8": A.FP8E4M3_B128}
_FP8_DTYPES = (torch.uint8, torch.float8_e4m3fn)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def make_desc(T: int, H: int, E: int, K: int, route_fmt: str = "dense_i16", payload: str = "bf16",
              pad_multiple: int = 1, capacity: Optional[int] = None, out_rows: int = 0) -> A.MoeDesc:
    return A.MoeDesc(T=T, H=H, E=E, K=K, route_fmt=_FMT[route_fmt], payload=_DT[payload],
                     pad_multiple=pad_multiple, capacity=-1 if capacity is None else int(capacity),
                     out_rows=int(out_rows))


def out_rows_bound(T: int, H: int, E: int, K: int, pad_multiple: int = 1, capacity: Optional[int] = None,
                   route_fmt: str = "dense_i16", payload: str = "bf16") -> int:
    d = make_desc(T, H, E, K, route_fmt, payload, pad_multiple, capacity)
    return int(A.lib().moe_out_rows_bound(C.byref(d)))


def routing_bytes(T: int, E: int, K: int, route_fmt: str = "dense_i16") -> int:
    d = make_desc(T, 8, E, K, route_fmt)
    return int(A.lib().moe_routing_bytes(C.byref(d)))


def capacity_from_rows(rows: int, factor: float) -> int:
    return int(A.lib().moe_capacity_from_rows(int(rows), float(factor)))


def assert_no_overflow(flag: torch.Tensor) -> None:
    """Device-side assert that the overflow flag is clear; the host does not
    wait for it (the failure surfaces at the next synchronisation)."""
    torch._assert_async(flag[0] == 0)


class Dispatcher:
    """One fixed-shape dispatch/MLP/combine problem with its workspace."""

    def __init__(self, T: int, H: int, E: int, K: int, *, route_fmt: str = "dense_i16",
                 payload: str = "bf16", pad_multiple: int = 1, capacity: Optional[int] = None,
                 out_rows: int = 0, device=None):
        L = A.lib()
        self.device = torch.device(device if device is not None else "cuda")
        self.desc = make_desc(T, H, E, K, route_fmt, payload, pad_multiple, capacity, out_rows)
        ws_bytes = int(L.moe_workspace_bytes(C.byref(self.desc)))
        if ws_bytes == 0:
            raise A.MoeError(A.MOE_ESHAPE, "moe_workspace_bytes")
        self.ws = torch.empty(ws_bytes, dtype=torch.uint8, device=self.device)
        self.h = A.MoeHandle()
        A.check(L.moe_handle_init(C.byref(self.desc), _ptr(self.ws), ws_bytes, C.byref(self.h)), "moe_handle_init")
        self.T, self.H, self.E, self.K = T, H, E, K
        self.R = int(self.h.desc.out_rows)
        self.route_fmt = self.desc.route_fmt
        self.payload = self.desc.payload
        self.tokens_per_expert = torch.empty(E, dtype=torch.int32, device=self.device)
        self.flag = torch.empty(1, dtype=torch.int32, device=self.device)

    # ---- views of the handle's device metadata ------------------------------
    def _view(self, field: str, dtype: torch.dtype, n: int) -> torch.Tensor:
        off = int(getattr(self.h, field)) - int(self.h.ws)
        nb = n * torch.empty(0, dtype=dtype).element_size()
        return self.ws[off:off + nb].view(dtype)

    @property
    def row_id(self):
        return self._view("row_id", torch.int32, self.T * self.K).view(self.T, self.K)

    @property
    def copy_prob(self):
        return self._view("copy_prob", torch.float32, self.T * self.K).view(self.T, self.K)

    @property
    def seg_off(self):
        return self._view("seg_off", torch.int64, self.E + 1)

    @property
    def kept(self):
        return self._view("kept", torch.int32, self.E)

    @property
    def src_row(self):
        return self._view("src_row", torch.int32, self.R)

    @property
    def rows_needed(self):
        return self._view("rows_needed", torch.int64, 1)

    # ---- checks ------------------------------------------------------------------
    def _dev(self, t: torch.Tensor, name: str):
        _need(t.device == self.device or (t.device.type == "cuda" and self.device.type == "cuda"
                                          and t.device.index == torch.cuda.current_device()),
              f"{name} must live on {self.device}")
        _need(t.is_contiguous(), f"{name} must be contiguous")

    def _check_routing(self, routing, probs, T_live):
        self._dev(routing, "routing")
        _need(routing.dtype in _FMT_DTYPES[self.route_fmt], f"routing dtype {routing.dtype} does not match the format")
        shape = (self.T, self.E) if self.route_fmt == A.ROUTE_SPARSE_BOOL else (self.T, self.K)
        _need(tuple(routing.shape) == shape, f"routing shape {tuple(routing.shape)} != {shape}")
        if probs is not None:
            self._dev(probs, "probs")
            _need(probs.dtype == torch.float32 and tuple(probs.shape) == shape, "probs must be float32 shaped like routing")
        if T_live is not None:
            self._dev(T_live, "T_live")
            _need(T_live.dtype == torch.int32 and T_live.numel() == 1, "T_live must be one int32")

    # ---- calls -------------------------------------------------------------------
    def preprocess(self, routing: torch.Tensor, probs: Optional[torch.Tensor] = None,
                   T_live: Optional[torch.Tensor] = None, out_probs: Optional[torch.Tensor] = None):
        self._check_routing(routing, probs, T_live)
        if out_probs is not None:
            self._dev(out_probs, "out_probs")
            _need(out_probs.dtype == torch.float32 and out_probs.numel() >= self.R, "out_probs must hold R floats")
        A.check(A.lib().moe_route_preprocess(C.byref(self.h), _ptr(routing), _ptr(probs), _ptr(T_live),
                                             _ptr(self.tokens_per_expert), _ptr(out_probs), _ptr(self.flag),
                                             _stream()), "moe_route_preprocess")
        return self.tokens_per_expert, self.flag

    def _alloc_out(self, x, out, x_scales, out_scales):
        if out is None:
            out = torch.empty((self.R, self.H), dtype=x.dtype, device=self.device)
        self._dev(out, "out")
        _need(out.dtype == x.dtype and tuple(out.shape) == (self.R, self.H), "out must be [R,H] like x")
        if self.payload == A.FP8E4M3_B128:
            _need(x_scales is not None, "fp8 payload needs x_scales")
            self._dev(x_scales, "x_scales")
            _need(x_scales.dtype == torch.float32 and tuple(x_scales.shape) == (self.T, self.H // 128),
                  "x_scales must be float32 [T, H/128]")
            if out_scales is None:
                out_scales = torch.empty((self.R, self.H // 128), dtype=torch.float32, device=self.device)
            self._dev(out_scales, "out_scales")
            _need(tuple(out_scales.shape) == (self.R, self.H // 128), "out_scales must be [R, H/128]")
        return out, out_scales

    def _check_x(self, x):
        self._dev(x, "x")
        _need(tuple(x.shape) == (self.T, self.H), f"x shape {tuple(x.shape)} != {(self.T, self.H)}")
        if self.payload == A.BF16:
            _need(x.dtype == torch.bfloat16, "bf16 payload expects a bfloat16 x")
        else:
            _need(x.dtype in _FP8_DTYPES, "fp8 payload expects uint8 / float8_e4m3fn codes")

    def permute(self, x: torch.Tensor, x_scales: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None, out_scales: Optional[torch.Tensor] = None):
        self._check_x(x)
        out, out_scales = self._alloc_out(x, out, x_scales, out_scales)
        A.check(A.lib().moe_permute(C.byref(self.h), _ptr(x), _ptr(x_scales), _ptr(out), _ptr(out_scales),
                                    _stream()), "moe_permute")
        return (out, out_scales) if self.payload == A.FP8E4M3_B128 else out

    def permute_quantize(self, x: torch.Tensor, out: Optional[torch.Tensor] = None,
                         out_scales: Optional[torch.Tensor] = None):
        """Quantise-on-dispatch (handle with fp8 payload): bf16 token rows x
        [T,H] -> e4m3 codes [R,H] and 1x128 fp32 scales [R,H/128] at every
        kept copy's row.  Returns (codes, scales)."""
        _need(self.payload == A.FP8E4M3_B128, "quantise-on-dispatch needs a handle with fp8 payload")
        self._dev(x, "x")
        _need(x.dtype == torch.bfloat16 and tuple(x.shape) == (self.T, self.H), "x must be bf16 [T,H]")
        if out is None:
            out = torch.empty((self.R, self.H), dtype=torch.uint8, device=self.device)
        if out_scales is None:
            out_scales = torch.empty((self.R, self.H // 128), dtype=torch.float32, device=self.device)
        self._dev(out, "out")
        self._dev(out_scales, "out_scales")
        _need(out.dtype in _FP8_DTYPES and tuple(out.shape) == (self.R, self.H), "out must be e4m3 codes [R,H]")
        _need(out_scales.dtype == torch.float32 and tuple(out_scales.shape) == (self.R, self.H // 128),
              "out_scales must be float32 [R, H/128]")
        A.check(A.lib().moe_permute_quantize(C.byref(self.h), _ptr(x), _ptr(out), _ptr(out_scales), _stream()),
                "moe_permute_quantize")
        return out, out_scales

    def dispatch(self, x: torch.Tensor, routing: torch.Tensor, probs: Optional[torch.Tensor] = None, *,
                 x_scales=None, out=None, out_scales=None, out_probs=None, T_live=None):
        """preprocess + permute.  Returns (permuted, tokens_per_expert, flag,
        out_probs, out_scales); out_probs / out_scales are None unless given
        / fp8."""
        self._check_x(x)
        self._check_routing(routing, probs, T_live)
        out, out_scales = self._alloc_out(x, out, x_scales, out_scales)
        if out_probs is not None:
            self._dev(out_probs, "out_probs")
            _need(out_probs.dtype == torch.float32 and out_probs.numel() >= self.R, "out_probs must hold R floats")
        A.check(A.lib().moe_dispatch(C.byref(self.h), _ptr(routing), _ptr(probs), _ptr(T_live), _ptr(x),
                                     _ptr(x_scales), _ptr(out), _ptr(out_scales), _ptr(out_probs),
                                     _ptr(self.tokens_per_expert), _ptr(self.flag), _stream()), "moe_dispatch")
        return out, self.tokens_per_expert, self.flag, out_probs, out_scales

    def mlp_scratch_bytes(self, F: int, wdtype: str = "bf16") -> int:
        return int(A.lib().moe_mlp_scratch_bytes(C.byref(self.h), int(F), _DT[wdtype]))

    def alloc_mlp_scratch(self, F: int, wdtype: str = "bf16") -> torch.Tensor:
        n = self.mlp_scratch_bytes(F, wdtype)
        _need(n > 0, "invalid F / wdtype for the MLP scratch")
        return torch.empty(n, dtype=torch.uint8, device=self.device)

    def _check_perm(self, perm, perm_scales):
        self._dev(perm, "perm")
        if self.payload == A.FP8E4M3_B128:
            _need(perm.dtype in _FP8_DTYPES and tuple(perm.shape) == (self.R, self.H),
                  "perm must be e4m3 codes [R,H] (quantised on dispatch)")
            _need(perm_scales is not None, "fp8 permuted rows need their scales")
            self._dev(perm_scales, "perm_scales")
            _need(perm_scales.dtype == torch.float32 and tuple(perm_scales.shape) == (self.R, self.H // 128),
                  "perm_scales must be float32 [R, H/128]")
        else:
            _need(perm.dtype == torch.bfloat16 and tuple(perm.shape) == (self.R, self.H), "perm must be bf16 [R,H]")
            _need(perm_scales is None, "bf16 permuted rows take no scales")

    def _check_w1(self, w1: torch.Tensor, w1_scales: Optional[torch.Tensor]):
        """FC1 weights [E, 2F, H] (bf16, or e4m3 codes with [E, 2F/128, H/128]
        float32 block scales) on this device; returns (F, wdtype)."""
        self._dev(w1, "w1")
        _need(w1.dim() == 3 and w1.shape[0] == self.E and w1.shape[2] == self.H and w1.shape[1] % 2 == 0
              and w1.shape[1] > 0, f"w1 must be [E, 2F, H] = [{self.E}, 2F, {self.H}], got {tuple(w1.shape)}")
        F = int(w1.shape[1]) // 2
        return F, self._check_wdtype(w1, w1_scales, "w1", (self.E, 2 * F // 128, self.H // 128))

    def _check_w2(self, w2: torch.Tensor, w2_scales: Optional[torch.Tensor]):
        """FC2 weights [E, H, F] (bf16, or e4m3 codes with [E, H/128, F/128]
        float32 block scales) on this device; returns (F, wdtype)."""
        self._dev(w2, "w2")
        _need(w2.dim() == 3 and w2.shape[0] == self.E and w2.shape[1] == self.H and w2.shape[2] > 0,
              f"w2 must be [E, H, F] = [{self.E}, {self.H}, F], got {tuple(w2.shape)}")
        F = int(w2.shape[2])
        return F, self._check_wdtype(w2, w2_scales, "w2", (self.E, self.H // 128, F // 128))

    def _check_wdtype(self, w, scales, name, scale_shape):
        if w.dtype in _FP8_DTYPES:
            _need(self.H % 128 == 0 and w.shape[1] % 128 == 0 and w.shape[2] % 128 == 0,
                  f"fp8 {name} needs dimensions that are multiples of 128")
            _need(scales is not None, f"fp8 {name} needs its 128x128 block scales")
            self._dev(scales, f"{name}_scales")
            _need(scales.dtype == torch.float32 and tuple(scales.shape) == scale_shape,
                  f"{name}_scales must be float32 {scale_shape}, got {scales.dtype} {tuple(scales.shape)}")
            return "fp8"
        _need(w.dtype == torch.bfloat16, f"{name} must be bfloat16 or e4m3 codes, got {w.dtype}")
        _need(scales is None, f"bf16 {name} takes no block scales")
        return "bf16"

    def _check_scratch(self, scratch: torch.Tensor, F: int, wdtype: str):
        self._dev(scratch, "scratch")
        need = self.mlp_scratch_bytes(F, wdtype)
        _need(need > 0, f"invalid FFN width {F} for {wdtype} weights")
        _need(scratch.numel() * scratch.element_size() >= need, f"scratch holds fewer than the {need} bytes needed")

    def _check_expert_out(self, out: torch.Tensor):
        self._dev(out, "out")
        _need(out.dtype == torch.bfloat16 and tuple(out.shape) == (self.R, self.H),
              f"out must be bf16 [R, H] = [{self.R}, {self.H}]")

    def grouped_mlp(self, perm: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor, *,
                    w1_scales: Optional[torch.Tensor] = None, w2_scales: Optional[torch.Tensor] = None,
                    scratch: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                    perm_scales: Optional[torch.Tensor] = None):
        """Grouped SwiGLU MLP over the permuted rows.  w1 [E,2F,H], w2 [E,H,F]
        (bf16, or e4m3 codes with 128x128 block scales).  With a handle of fp8
        payload, perm is e4m3 codes quantised on dispatch plus perm_scales
        (fp8 weights only)."""
        F, wdtype = self._check_w1(w1, w1_scales)
        F2, wdtype2 = self._check_w2(w2, w2_scales)
        _need(F2 == F and wdtype2 == wdtype, "w1 and w2 must share the FFN width and dtype")
        self._check_perm(perm, perm_scales)
        if scratch is None:
            scratch = self.alloc_mlp_scratch(F, wdtype)
        self._check_scratch(scratch, F, wdtype)
        if out is None:
            out = torch.empty((self.R, self.H), dtype=torch.bfloat16, device=self.device)
        self._check_expert_out(out)
        A.check(A.lib().moe_grouped_swiglu_mlp(C.byref(self.h), F, _DT[wdtype], _ptr(perm), _ptr(perm_scales), _ptr(w1),
                                               _ptr(w1_scales), _ptr(w2), _ptr(w2_scales), _ptr(scratch),
                                               scratch.numel(), _ptr(out), _stream()), "moe_grouped_swiglu_mlp")
        return out

    def grouped_mlp_noalloc(self, perm: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor, *,
                            w1_scales: Optional[torch.Tensor] = None, w2_scales: Optional[torch.Tensor] = None,
                            out: torch.Tensor, perm_scales: Optional[torch.Tensor] = None):
        """grouped_mlp without a scratch argument and without any allocation:
        the activations live in the library's fixed device array
        (A.NOALLOC_SCRATCH_BYTES per GPU, shared by every call on that GPU).
        ``out`` is required."""
        F, wdtype = self._check_w1(w1, w1_scales)
        F2, wdtype2 = self._check_w2(w2, w2_scales)
        _need(F2 == F and wdtype2 == wdtype, "w1 and w2 must share the FFN width and dtype")
        self._check_perm(perm, perm_scales)
        self._check_expert_out(out)
        A.check(A.lib().moe_grouped_swiglu_mlp_noalloc(C.byref(self.h), F, _DT[wdtype], _ptr(perm), _ptr(perm_scales),
                                                       _ptr(w1), _ptr(w1_scales), _ptr(w2), _ptr(w2_scales), _ptr(out),
                                                       _stream()), "moe_grouped_swiglu_mlp_noalloc")
        return out

    def fc1(self, perm: torch.Tensor, w1: torch.Tensor, scratch: torch.Tensor, w1_scales=None,
            perm_scales=None) -> None:
        """FC1 + SwiGLU of every kept row into ``scratch`` (the first half of
        grouped_mlp).  The FFN width and weight dtype are remembered: fc2 on
        this scratch must use the same."""
        F, wdtype = self._check_w1(w1, w1_scales)
        self._check_perm(perm, perm_scales)
        self._check_scratch(scratch, F, wdtype)
        A.check(A.lib().moe_grouped_fc1_swiglu(C.byref(self.h), F, _DT[wdtype], _ptr(perm), _ptr(perm_scales), _ptr(w1),
                                               _ptr(w1_scales), _ptr(scratch), scratch.numel(), _stream()),
                "moe_grouped_fc1_swiglu")
        self._fc1_done = (F, wdtype, scratch.data_ptr())

    def _check_after_fc1(self, F: int, wdtype: str, scratch: torch.Tensor):
        prev = getattr(self, "_fc1_done", None)
        _need(prev is not None, "fc2 needs an fc1 on this Dispatcher first")
        _need(prev == (F, wdtype, scratch.data_ptr()),
              f"fc2 with FFN width {F} ({wdtype}) on scratch {scratch.data_ptr():#x} does not match the last fc1 "
              f"(width {prev[0]} ({prev[1]}) on scratch {prev[2]:#x})")

    def fc2(self, w2: torch.Tensor, scratch: torch.Tensor, out: torch.Tensor, w2_scales=None) -> torch.Tensor:
        """FC2 from ``scratch`` into the caller-owned ``out`` (the second half
        of grouped_mlp)."""
        F, wdtype = self._check_w2(w2, w2_scales)
        self._check_scratch(scratch, F, wdtype)
        self._check_after_fc1(F, wdtype, scratch)
        self._check_expert_out(out)
        A.check(A.lib().moe_grouped_fc2(C.byref(self.h), F, _DT[wdtype], _ptr(w2), _ptr(w2_scales), _ptr(scratch),
                                        scratch.numel(), _ptr(out), _stream()), "moe_grouped_fc2")
        return out

    def fc2_fp8out(self, w2: torch.Tensor, scratch: torch.Tensor, out: Optional[torch.Tensor] = None,
                   out_scales: Optional[torch.Tensor] = None):
        """FC2 (bf16 weights) into the fp8 combine format: returns (codes
        [R,H] uint8, scales [R,H/128] float32)."""
        F, wdtype = self._check_w2(w2, None)
        _need(wdtype == "bf16", "the fp8 combine format is written from bf16 weights")
        self._check_scratch(scratch, F, wdtype)
        self._check_after_fc1(F, wdtype, scratch)
        if out is None:
            out = torch.empty((self.R, self.H), dtype=torch.uint8, device=self.device)
        if out_scales is None:
            out_scales = torch.empty((self.R, self.H // 128), dtype=torch.float32, device=self.device)
        self._dev(out, "out")
        self._dev(out_scales, "out_scales")
        _need(out.dtype in _FP8_DTYPES and tuple(out.shape) == (self.R, self.H), "out must be e4m3 codes [R,H]")
        _need(out_scales.dtype == torch.float32 and tuple(out_scales.shape) == (self.R, self.H // 128),
              "out_scales must be float32 [R, H/128]")
        A.check(A.lib().moe_grouped_fc2_fp8out(C.byref(self.h), F, A.BF16, _ptr(w2), None, _ptr(scratch),
                                               scratch.numel(), _ptr(out), _ptr(out_scales), _stream()),
                "moe_grouped_fc2_fp8out")
        return out, out_scales

    def combine_fp8(self, expert_out_q: torch.Tensor, expert_out_scales: torch.Tensor, apply_probs: bool = True,
                    out: Optional[torch.Tensor] = None):
        """Combine from fp8 expert-output rows (codes [R,H], scales [R,H/128])."""
        self._dev(expert_out_q, "expert_out_q")
        self._dev(expert_out_scales, "expert_out_scales")
        _need(expert_out_q.dtype in _FP8_DTYPES and tuple(expert_out_q.shape) == (self.R, self.H),
              "expert_out_q must be e4m3 codes [R,H]")
        _need(expert_out_scales.dtype == torch.float32 and tuple(expert_out_scales.shape) == (self.R, self.H // 128),
              "expert_out_scales must be float32 [R, H/128]")
        if out is None:
            out = torch.empty((self.T, self.H), dtype=torch.bfloat16, device=self.device)
        self._dev(out, "out")
        _need(out.dtype == torch.bfloat16 and tuple(out.shape) == (self.T, self.H), "out must be bf16 [T,H]")
        A.check(A.lib().moe_combine_fp8(C.byref(self.h), _ptr(expert_out_q), _ptr(expert_out_scales),
                                        1 if apply_probs else 0, _ptr(out), _stream()), "moe_combine_fp8")
        return out

    def combine(self, expert_out: torch.Tensor, apply_probs: bool = True, out: Optional[torch.Tensor] = None):
        self._dev(expert_out, "expert_out")
        _need(expert_out.dtype == torch.bfloat16 and tuple(expert_out.shape) == (self.R, self.H),
              "expert_out must be bf16 [R,H]")
        if out is None:
            out = torch.empty((self.T, self.H), dtype=torch.bfloat16, device=self.device)
        self._dev(out, "out")
        _need(out.dtype == torch.bfloat16 and tuple(out.shape) == (self.T, self.H), "out must be bf16 [T,H]")
        A.check(A.lib().moe_combine(C.byref(self.h), _ptr(expert_out), 1 if apply_probs else 0, _ptr(out),
                                    _stream()), "moe_combine")
        return out

    # ---- backward ---------------------------------------------------------------
    def _probs_grad_shape(self):
        return (self.T, self.E) if self.route_fmt == A.ROUTE_SPARSE_BOOL else (self.T, self.K)

    def _grad_probs_out(self, grad_probs):
        if grad_probs is None:
            grad_probs = torch.empty(self._probs_grad_shape(), dtype=torch.float32, device=self.device)
        self._dev(grad_probs, "grad_probs")
        _need(grad_probs.dtype == torch.float32 and tuple(grad_probs.shape) == self._probs_grad_shape(),
              "grad_probs must be float32 in the routing's shape")
        return grad_probs

    def dispatch_backward(self, grad_out: torch.Tensor, grad_out_probs: Optional[torch.Tensor] = None, *,
                          out: Optional[torch.Tensor] = None, grad_probs: Optional[torch.Tensor] = None):
        """Gradients of a dispatch: (grad_x [T,H] bf16, grad_probs or None).
        grad_probs (routing-shaped fp32) is produced when grad_out_probs [R]
        is given."""
        self._dev(grad_out, "grad_out")
        _need(grad_out.dtype == torch.bfloat16 and tuple(grad_out.shape) == (self.R, self.H),
              "grad_out must be bf16 [R,H]")
        if out is None:
            out = torch.empty((self.T, self.H), dtype=torch.bfloat16, device=self.device)
        self._dev(out, "out")
        _need(out.dtype == torch.bfloat16 and tuple(out.shape) == (self.T, self.H), "out must be bf16 [T,H]")
        if grad_out_probs is not None:
            self._dev(grad_out_probs, "grad_out_probs")
            _need(grad_out_probs.dtype == torch.float32 and grad_out_probs.numel() >= self.R,
                  "grad_out_probs must hold R floats")
            grad_probs = self._grad_probs_out(grad_probs)
        else:
            _need(grad_probs is None, "grad_probs needs grad_out_probs")
        A.check(A.lib().moe_dispatch_backward(C.byref(self.h), _ptr(grad_out), _ptr(grad_out_probs), _ptr(out),
                                              _ptr(grad_probs), _stream()), "moe_dispatch_backward")
        return out, grad_probs

    def combine_backward(self, grad_y: torch.Tensor, expert_out: Optional[torch.Tensor] = None,
                         apply_probs: bool = True, *, out: Optional[torch.Tensor] = None,
                         grad_probs: Optional[torch.Tensor] = None, want_probs: bool = True):
        """Gradients of a combine: (grad_expert_out [R,H] bf16, grad_probs or
        None).  The probability gradient needs the forward's expert_out."""
        self._dev(grad_y, "grad_y")
        _need(grad_y.dtype == torch.bfloat16 and tuple(grad_y.shape) == (self.T, self.H), "grad_y must be bf16 [T,H]")
        if out is None:
            out = torch.empty((self.R, self.H), dtype=torch.bfloat16, device=self.device)
        self._dev(out, "out")
        _need(out.dtype == torch.bfloat16 and tuple(out.shape) == (self.R, self.H), "out must be bf16 [R,H]")
        if expert_out is not None:
            self._dev(expert_out, "expert_out")
            _need(expert_out.dtype == torch.bfloat16 and tuple(expert_out.shape) == (self.R, self.H),
                  "expert_out must be bf16 [R,H]")
        if want_probs or grad_probs is not None:
            _need(expert_out is not None or not apply_probs, "the probability gradient needs expert_out")
            grad_probs = self._grad_probs_out(grad_probs)
        A.check(A.lib().moe_combine_backward(C.byref(self.h), _ptr(grad_y), _ptr(expert_out), 1 if apply_probs else 0,
                                             _ptr(out), _ptr(grad_probs), _stream()), "moe_combine_backward")
        return out, grad_probs

    def decode_layer_scratch_bytes(self, F: int) -> int:
        return int(A.lib().moe_decode_layer_scratch_bytes(C.byref(self.h), int(F)))

    def decode_layer_fp8(self, x: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor, w1_scales: torch.Tensor,
                         w2_scales: torch.Tensor, *, scratch: torch.Tensor, expert_out: torch.Tensor,
                         out: torch.Tensor, status: torch.Tensor, apply_probs: bool = True) -> torch.Tensor:
        """The rest of the layer after preprocess(), as one persistent kernel:
        quantise-on-dispatch, FC1 + SwiGLU, activation quantiser, FC2 into
        ``expert_out`` and the combine into ``out``, with fp8 weights.
        ``status`` (one int32 on the device): the call clears bits 0 and 1
        and keeps bit 2, the caller's abort request (every wait returns at
        once).  Afterwards bit 0 means a wait ran past its bound and bit 1 a
        workgroup on an XCD numbered 8 or more; with any bit set the outputs
        are unspecified."""
        _need(self.payload == A.BF16, "the decode layer takes bf16 token rows")
        self._check_x(x)
        F, wdtype = self._check_w1(w1, w1_scales)
        F2, wdtype2 = self._check_w2(w2, w2_scales)
        _need(wdtype == "fp8" and wdtype2 == "fp8" and F2 == F, "the decode layer takes fp8 w1 and w2 of one FFN width")
        self._dev(scratch, "scratch")
        need = self.decode_layer_scratch_bytes(F)
        _need(need > 0 and scratch.numel() * scratch.element_size() >= need,
              f"scratch holds fewer than the {need} bytes needed")
        self._check_expert_out(expert_out)
        self._dev(out, "out")
        _need(out.dtype == torch.bfloat16 and tuple(out.shape) == (self.T, self.H), "out must be bf16 [T,H]")
        self._dev(status, "status")
        _need(status.dtype == torch.int32 and status.numel() == 1, "status must be one int32")
        A.check(A.lib().moe_decode_layer_fp8(C.byref(self.h), F, _ptr(x), _ptr(w1), _ptr(w1_scales), _ptr(w2),
                                             _ptr(w2_scales), _ptr(scratch), scratch.numel(), _ptr(expert_out),
                                             1 if apply_probs else 0, _ptr(out), _ptr(status), _stream()),
                "moe_decode_layer_fp8")
        return out

    def decode_fused_scratch_bytes(self, F: int) -> int:
        return int(A.lib().moe_decode_fused_scratch_bytes(C.byref(self.h), int(F)))

    def decode_fused_fp8(self, x: torch.Tensor, w1: torch.Tensor, w2: torch.Tensor, w1_scales: torch.Tensor,
                         w2_scales: torch.Tensor, *, scratch: torch.Tensor, expert_out: torch.Tensor,
                         out: torch.Tensor, apply_probs: bool = True) -> torch.Tensor:
        """The rest of the layer after preprocess(), with fp8 weights, in two
        launches: quantise-on-dispatch, then one persistent kernel for FC1 +
        SwiGLU, the activation blocks, FC2 into ``expert_out`` and the combine
        into ``out``."""
        _need(self.payload == A.BF16, "the decode layer takes bf16 token rows")
        self._check_x(x)
        F, wdtype = self._check_w1(w1, w1_scales)
        F2, wdtype2 = self._check_w2(w2, w2_scales)
        _need(wdtype == "fp8" and wdtype2 == "fp8" and F2 == F, "the decode layer takes fp8 w1 and w2 of one FFN width")
        self._dev(scratch, "scratch")
        need = self.decode_fused_scratch_bytes(F)
        _need(need > 0, "the fused decode layer needs H, F multiples of 128 and H <= 8192")
        _need(scratch.numel() * scratch.element_size() >= need, f"scratch holds fewer than the {need} bytes needed")
        self._check_expert_out(expert_out)
        self._dev(out, "out")
        _need(out.dtype == torch.bfloat16 and tuple(out.shape) == (self.T, self.H), "out must be bf16 [T,H]")
        A.check(A.lib().moe_decode_fused_fp8(C.byref(self.h), F, _ptr(x), _ptr(w1), _ptr(w1_scales), _ptr(w2),
                                             _ptr(w2_scales), _ptr(scratch), scratch.numel() * scratch.element_size(),
                                             _ptr(expert_out), 1 if apply_probs else 0, _ptr(out), _stream()),
                "moe_decode_fused_fp8")
        return out

    def layer(self, x, routing, probs, w1, w2, *, perm=None, perm_scales=None, scratch=None, expert_out=None,
              out=None, w1_scales=None, w2_scales=None, T_live=None, apply_probs=True, check_overflow=False):
        """dispatch -> grouped MLP -> combine on the current stream.  With a
        handle of fp8 payload and bf16 tokens, dispatch quantises on the way
        (routing metadata, then moe_permute_quantize into e4m3 rows ``perm``
        with 1x128 scales ``perm_scales``).  With ``check_overflow``, a
        device-side assert on the overflow flag is enqueued after the combine
        (no host wait; capturable).  Buffers the caller omits are allocated
        per call."""
        if self.payload == A.FP8E4M3_B128 and x.dtype == torch.bfloat16:
            _, flag = self.preprocess(routing, probs, T_live)
            perm, perm_scales = self.permute_quantize(x, out=perm, out_scales=perm_scales)
        else:
            perm, _, flag, _, perm_scales = self.dispatch(x, routing, probs, out=perm, out_scales=perm_scales,
                                                          T_live=T_live)
        y = self.grouped_mlp(perm, w1, w2, w1_scales=w1_scales, w2_scales=w2_scales, scratch=scratch,
                             out=expert_out, perm_scales=perm_scales)
        y = self.combine(y, apply_probs=apply_probs, out=out)
        if check_overflow:
            assert_no_overflow(flag)
        return y


class BufferRing:
    """Caller-owned ring of persistent device slots (dispatch outputs, FC2
    outputs): ``acquire`` hands the next slot to a producer on the current
    stream, which first waits on the device for the slot's last release;
    ``release`` marks the final consumer's use on its stream.  Reuse before
    release raises (MOE_EBUSY), as does a second release (MOE_ESTATE).  The
    storage is one torch allocation made here; the library only carves it."""

    def __init__(self, n_slots: int, shape, dtype: torch.dtype, device=None):
        self.device = torch.device(device if device is not None else "cuda")
        self.shape = tuple(shape)
        self.dtype = dtype
        n = 1
        for v in self.shape:
            n *= int(v)
        self.nbytes = n * torch.empty(0, dtype=dtype).element_size()
        self.slot_bytes = (self.nbytes + 255) // 256 * 256
        self.storage = torch.empty(n_slots * self.slot_bytes, dtype=torch.uint8, device=self.device)
        self.r = A.MoeRing()
        A.check(A.lib().moe_ring_init(C.byref(self.r), _ptr(self.storage), self.slot_bytes, int(n_slots)),
                "moe_ring_init")
        self.n_slots = n_slots

    def acquire(self, stream=None):
        """(slot index, tensor view of the slot) for a producer on ``stream``
        (default: the current stream)."""
        st = C.c_void_p((stream or torch.cuda.current_stream()).cuda_stream)
        ptr = C.c_void_p()
        idx = C.c_int32()
        A.check(A.lib().moe_ring_acquire(C.byref(self.r), st, C.byref(ptr), C.byref(idx)), "moe_ring_acquire")
        off = int(idx.value) * self.slot_bytes
        view = self.storage[off:off + self.nbytes].view(self.dtype).view(self.shape)
        return int(idx.value), view

    def release(self, slot: int, stream=None):
        st = C.c_void_p((stream or torch.cuda.current_stream()).cuda_stream)
        A.check(A.lib().moe_ring_release(C.byref(self.r), int(slot), st), "moe_ring_release")

    def close(self):
        A.check(A.lib().moe_ring_destroy(C.byref(self.r)), "moe_ring_destroy")
