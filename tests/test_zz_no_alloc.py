"""The grouped MLP entry point that allocates nothing
(moe_grouped_swiglu_mlp_noalloc), called through the C ABI, against the
scratch-taking entry point (moe_grouped_swiglu_mlp) on the same inputs: two
calls in a row, the second on a smaller problem, for bf16 and fp8 weights.
Both run the same kernels, so the kept rows must agree bit for bit."""
import ctypes as C

import numpy as np
import pytest
import torch

import moe_synth as S
from combine_routing_preprocess_amd import Dispatcher
from combine_routing_preprocess_amd import _abi as A
from gpu_util import DEV, dev, log

pytestmark = pytest.mark.gpu


def _p(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _case(T, H, E, K, F, pad, seed, fp8):
    idx, pr = S.route_softmax_topk(T, E, K, seed)
    x = dev(S.bf16_normal((T, H), seed))
    if fp8:
        w1, w1s = (t.to(DEV) for t in S.weights_fp8_blocks(E, 2 * F, H, seed + 1, std=0.05))
        w2, w2s = (t.to(DEV) for t in S.weights_fp8_blocks(E, H, F, seed + 2, std=0.05))
    else:
        w1 = dev(S.bf16_normal((E, 2 * F, H), seed + 1, std=0.05))
        w2 = dev(S.bf16_normal((E, H, F), seed + 2, std=0.05))
        w1s = w2s = None
    d = Dispatcher(T, H, E, K, pad_multiple=pad)
    perm, *_ = d.dispatch(x, dev(idx), dev(pr))
    return d, perm, w1, w1s, w2, w2s, F


def _both(d, perm, w1, w1s, w2, w2s, F, wdtype):
    L = A.lib()
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    ref = torch.full((d.R, d.H), -1.0, dtype=torch.bfloat16, device=DEV)
    got = torch.full((d.R, d.H), 7.0, dtype=torch.bfloat16, device=DEV)
    need = int(L.moe_mlp_scratch_bytes(C.byref(d.h), F, wdtype))
    scratch = torch.empty(need, dtype=torch.uint8, device=DEV)
    assert L.moe_grouped_swiglu_mlp(C.byref(d.h), F, wdtype, _p(perm), None, _p(w1), _p(w1s), _p(w2), _p(w2s),
                                    _p(scratch), need, _p(ref), stream) == 0
    assert L.moe_grouped_swiglu_mlp_noalloc(C.byref(d.h), F, wdtype, _p(perm), None, _p(w1), _p(w1s), _p(w2),
                                            _p(w2s), _p(got), stream) == 0
    torch.cuda.synchronize()
    rows = d.src_row >= 0
    assert int(rows.sum().item()) > 0
    assert torch.equal(ref[rows].view(torch.int16), got[rows].view(torch.int16))


@pytest.mark.parametrize("fp8", [False, True])
def test_noalloc_mlp_matches_scratch_entry_point_twice(fp8):
    wdtype = A.FP8E4M3_B128 if fp8 else A.BF16
    # first call: 512 tokens x 1024, 16 experts top-4, padding 32
    log("no-alloc MLP", "fp8" if fp8 else "bf16", "large")
    big = _case(512, 1024, 16, 4, 512, 32, 11, fp8)
    _both(*big, wdtype)
    # second call, right after, on a smaller problem: the shared array still
    # holds the first call's activations
    log("no-alloc MLP", "fp8" if fp8 else "bf16", "small")
    small = _case(100, 256, 8, 2, 128, 16, 12, fp8)
    _both(*small, wdtype)

