"""MI355X-native MoE layer hot path: routing preprocessing -> dispatch-permute
-> grouped SwiGLU MLP -> combine-unpermute.

Every step runs in the hand-written HIP kernels of ``libmoe_route.so``
(C ABI in ``include/moe_route.h``).  This package only marshals torch tensors
(device memory) and torch's current HIP stream into those calls.
"""
from ._abi import (BF16, FP8E4M3_B128, FLAG_BAD_EXPERT, FLAG_CAPACITY, FLAG_DUPLICATE, FLAG_OUT_ROWS,
                   ROUTE_DENSE_I16, ROUTE_DENSE_I32, ROUTE_SPARSE_BOOL, MoeError, lib)
from .api import (BufferRing, Dispatcher, assert_no_overflow, capacity_from_rows, out_rows_bound, routing_bytes)

__all__ = ["BufferRing", "Dispatcher", "assert_no_overflow", "capacity_from_rows", "out_rows_bound", "routing_bytes",
           "MoeError", "lib", "BF16", "FP8E4M3_B128", "ROUTE_DENSE_I16", "ROUTE_DENSE_I32",
           "ROUTE_SPARSE_BOOL", "FLAG_CAPACITY", "FLAG_OUT_ROWS", "FLAG_BAD_EXPERT", "FLAG_DUPLICATE"]
