"""The caller-owned buffer ring on the GPU: a producer stream and a consumer
stream share a two-slot ring of permuted-row buffers; the ring's device-side
wait for the final consumer's release must keep a slot from being
overwritten while the consumer still reads it.  Early reuse and double
release fail explicitly; a captured iteration replays correctly."""
import numpy as np
import pytest
import torch

import moe_synth as S
from combine_routing_preprocess_amd import BufferRing, Dispatcher, MoeError
from combine_routing_preprocess_amd import _abi as A
from gpu_util import DEV, dev, log

pytestmark = pytest.mark.gpu


def _problem(T=2048, H=1024, E=16, K=2):
    idx, _ = S.route_uniform_distinct(T, E, K, 77)
    d = Dispatcher(T, H, E, K)
    d.preprocess(dev(idx))
    return d


def test_ring_orders_producer_after_final_consumer():
    d = _problem()
    ring = BufferRing(2, (d.R, d.H), torch.bfloat16)
    A_s, B_s = torch.cuda.Stream(), torch.cuda.Stream()
    busy = torch.randn((4096, 4096), device=DEV)   # keeps the consumer stream slow
    xs = [dev(S.bf16_normal((d.T, d.H), 500 + i)) for i in range(6)]
    ys = []
    A_s.wait_stream(torch.cuda.current_stream())     # routing metadata and inputs are ready
    B_s.wait_stream(torch.cuda.current_stream())
    log("ring: two streams, 6 iterations over 2 slots")
    for i, x in enumerate(xs):
        with torch.cuda.stream(A_s):
            slot, buf = ring.acquire(A_s)
            d.permute(x, out=buf)
            produced = torch.cuda.Event()
            produced.record(A_s)
        with torch.cuda.stream(B_s):
            B_s.wait_event(produced)
            for _ in range(3):
                busy = busy @ busy.T * 1e-3         # slow final consumer
            ys.append(d.combine(buf, apply_probs=False))
            ring.release(slot, B_s)
    torch.cuda.synchronize()
    for x, y in zip(xs, ys):
        assert torch.equal(y, x * 2)                # top-2 copies, no probabilities: 2x exactly
    ring.close()


def test_ring_explicit_failures():
    d = _problem(T=64)
    ring = BufferRing(2, (d.R, d.H), torch.bfloat16)
    s0, _ = ring.acquire()
    s1, _ = ring.acquire()
    with pytest.raises(MoeError) as e:
        ring.acquire()                               # slot 0 not released yet
    assert e.value.status == A.MOE_EBUSY
    ring.release(s0)
    with pytest.raises(MoeError) as e:
        ring.release(s0)                             # double release
    assert e.value.status == A.MOE_ESTATE
    s2, _ = ring.acquire()                           # slot 0 again, after its release
    assert s2 == s0
    ring.release(s1)
    ring.release(s2)
    torch.cuda.synchronize()
    ring.close()


def test_ring_eager_warmup_then_graph_capture():
    d = _problem(T=512)
    ring = BufferRing(3, (d.R, d.H), torch.bfloat16)
    x = torch.empty((d.T, d.H), dtype=torch.bfloat16, device=DEV)
    y = torch.empty((d.T, d.H), dtype=torch.bfloat16, device=DEV)

    def iteration():
        slot, buf = ring.acquire()
        d.permute(x, out=buf)
        d.combine(buf, apply_probs=False, out=y)
        ring.release(slot)

    log("ring: eager warm-up, capture, replays")
    for i in range(4):                               # eager warm-up, wraps the ring
        x.copy_(dev(S.bf16_normal((d.T, d.H), 600 + i)))
        iteration()
        torch.cuda.synchronize()
        assert torch.equal(y, x * 2)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        iteration()
    for i in range(3):
        x.copy_(dev(S.bf16_normal((d.T, d.H), 700 + i)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, x * 2), i
    iteration()                                      # eager again after the graph
    torch.cuda.synchronize()
    assert torch.equal(y, x * 2)
    ring.close()
