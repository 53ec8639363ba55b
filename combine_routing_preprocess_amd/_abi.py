"""ctypes declarations mirroring include/moe_route.h.  Loading fails loudly if
the HIP library has not been built: there is no other implementation."""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_route.so")

MOE_OK, MOE_EINVAL, MOE_ESHAPE, MOE_EDTYPE, MOE_EALIGN = 0, -1, -2, -3, -4
MOE_ESTALE, MOE_EHIP, MOE_EUNSUPPORTED, MOE_ENOSPC = -5, -6, -7, -8
MOE_EBUSY, MOE_ESTATE = -9, -10
NOALLOC_SCRATCH_BYTES = 128 << 20      # MOE_NOALLOC_SCRATCH_BYTES
RING_MAX_SLOTS = 32

ROUTE_DENSE_I16, ROUTE_DENSE_I32, ROUTE_SPARSE_BOOL = 0, 1, 2
BF16, FP8E4M3_B128 = 0, 1

FLAG_CAPACITY, FLAG_OUT_ROWS, FLAG_BAD_EXPERT, FLAG_DUPLICATE = 1, 2, 4, 8


class MoeDesc(C.Structure):
    _fields_ = [("T", C.c_int32), ("H", C.c_int32), ("E", C.c_int32), ("K", C.c_int32),
                ("route_fmt", C.c_int32), ("payload", C.c_int32), ("pad_multiple", C.c_int32),
                ("capacity", C.c_int32), ("out_rows", C.c_int64)]


class MoeHandle(C.Structure):
    _fields_ = [("desc", MoeDesc), ("epoch", C.c_uint64), ("n_tiles", C.c_int32), ("state", C.c_int32),
                ("ws", C.c_void_p), ("ws_bytes", C.c_size_t),
                ("tile_mask", C.c_void_p), ("tile_base", C.c_void_p), ("tile_err", C.c_void_p),
                ("seg_off", C.c_void_p), ("kept", C.c_void_p), ("rows_needed", C.c_void_p),
                ("row_id", C.c_void_p), ("copy_prob", C.c_void_p), ("src_row", C.c_void_p)]


class MoeRing(C.Structure):
    _fields_ = [("base", C.c_void_p), ("slot_bytes", C.c_size_t), ("n_slots", C.c_int32), ("next", C.c_int32),
                ("acquisitions", C.c_uint64), ("state", C.c_int32 * RING_MAX_SLOTS),
                ("event_kind", C.c_int32 * RING_MAX_SLOTS), ("event_capture", C.c_ulonglong * RING_MAX_SLOTS),
                ("event", C.c_void_p * RING_MAX_SLOTS)]


# (name, restype, argtypes) for every function the header declares
_P = C.c_void_p
SIGNATURES = [
    ("moe_status_string", C.c_char_p, [C.c_int]),
    ("moe_out_rows_bound", C.c_int64, [C.POINTER(MoeDesc)]),
    ("moe_routing_bytes", C.c_int64, [C.POINTER(MoeDesc)]),
    ("moe_capacity_from_rows", C.c_int64, [C.c_int64, C.c_double]),
    ("moe_workspace_bytes", C.c_size_t, [C.POINTER(MoeDesc)]),
    ("moe_handle_init", C.c_int, [C.POINTER(MoeDesc), _P, C.c_size_t, C.POINTER(MoeHandle)]),
    ("moe_route_preprocess", C.c_int, [C.POINTER(MoeHandle), _P, _P, _P, _P, _P, _P, _P]),
    ("moe_permute", C.c_int, [C.POINTER(MoeHandle), _P, _P, _P, _P, _P]),
    ("moe_permute_quantize", C.c_int, [C.POINTER(MoeHandle), _P, _P, _P, _P]),
    ("moe_dispatch", C.c_int, [C.POINTER(MoeHandle), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    ("moe_mlp_scratch_bytes", C.c_size_t, [C.POINTER(MoeHandle), C.c_int32, C.c_int32]),
    ("moe_grouped_swiglu_mlp", C.c_int, [C.POINTER(MoeHandle), C.c_int32, C.c_int32, _P, _P, _P, _P, _P, _P,
                                         _P, C.c_size_t, _P, _P]),
    ("moe_grouped_swiglu_mlp_noalloc", C.c_int, [C.POINTER(MoeHandle), C.c_int32, C.c_int32, _P, _P, _P, _P, _P,
                                                 _P, _P, _P]),
    ("moe_grouped_fc1_swiglu", C.c_int, [C.POINTER(MoeHandle), C.c_int32, C.c_int32, _P, _P, _P, _P, _P,
                                         C.c_size_t, _P]),
    ("moe_grouped_fc2", C.c_int, [C.POINTER(MoeHandle), C.c_int32, C.c_int32, _P, _P, _P, C.c_size_t, _P, _P]),
    ("moe_combine", C.c_int, [C.POINTER(MoeHandle), _P, C.c_int32, _P, _P]),
    ("moe_grouped_fc2_fp8out", C.c_int, [C.POINTER(MoeHandle), C.c_int32, C.c_int32, _P, _P, _P, C.c_size_t, _P,
                                         _P, _P]),
    ("moe_combine_fp8", C.c_int, [C.POINTER(MoeHandle), _P, _P, C.c_int32, _P, _P]),
    ("moe_ring_init", C.c_int, [C.POINTER(MoeRing), _P, C.c_size_t, C.c_int32]),
    ("moe_ring_acquire", C.c_int, [C.POINTER(MoeRing), _P, C.POINTER(C.c_void_p), C.POINTER(C.c_int32)]),
    ("moe_ring_release", C.c_int, [C.POINTER(MoeRing), C.c_int32, _P]),
    ("moe_ring_destroy", C.c_int, [C.POINTER(MoeRing)]),
    ("moe_decode_layer_scratch_bytes", C.c_size_t, [C.POINTER(MoeHandle), C.c_int32]),
    ("moe_decode_layer_set_wait_bound", None, [C.c_int64]),
    ("moe_decode_layer_fp8", C.c_int, [C.POINTER(MoeHandle), C.c_int32, _P, _P, _P, _P, _P, _P, C.c_size_t, _P,
                                       C.c_int32, _P, _P, _P]),
    ("moe_decode_fused_scratch_bytes", C.c_size_t, [C.POINTER(MoeHandle), C.c_int32]),
    ("moe_decode_fused_fp8", C.c_int, [C.POINTER(MoeHandle), C.c_int32, _P, _P, _P, _P, _P, _P, C.c_size_t, _P,
                                       C.c_int32, _P, _P]),
    ("moe_dispatch_backward", C.c_int, [C.POINTER(MoeHandle), _P, _P, _P, _P, _P]),
    ("moe_combine_backward", C.c_int, [C.POINTER(MoeHandle), _P, _P, C.c_int32, _P, _P, _P]),
]

_lib = None


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = status_string(status) if _lib is not None else str(status)
        super().__init__(f"{where}: {msg} (status {status})")


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m combine_routing_preprocess_amd.build` (there is no fallback path)")
        L = C.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def check(status: int, where: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, where)
