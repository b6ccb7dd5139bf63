"""The decode step (pa_reshape_and_cache of the step's tokens, then pa_decode)
captured once in a HIP graph and replayed: every replay, with new query rows
and new K/V written between replays by the program's own eager work, must
give the same bits as the eager calls on the same inputs.  Neither call
allocates, synchronises or records a memset, so both can be captured; the
workspace is allocated before capture and its contents between calls do not
matter."""
import numpy as np
import pytest
import torch

from paged_kv_cache_72_amd import lib as L
from paged_kv_cache_72_amd import workloads as W
from helpers import DeviceCase, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("part", [-1, 1, 64])
@pytest.mark.parametrize("name,make", [
    ("d128_bs16", lambda: W.custom("g", 90, [1, 17, 300, 1000, 64], 32, 8, 128, 16)),
    ("fp8_d64_bs32", lambda: W.custom("g", 91, [5, 513, 40], 8, 2, 64, 32,
                                      kv_dtype="fp8_e4m3fn")),
])
def test_decode_step_replays_from_a_graph(name, make, part):
    w = make()
    say(f"graph {name} partition={part}")
    dc = DeviceCase(w, poison=True)
    pool = dc.pool
    q = dc.q.clone()
    k_new, v_new, slots = dc.k_new.clone(), dc.v_new.clone(), dc.slot_new.clone()
    out = torch.empty_like(q)
    ws = L.alloc_workspace(pool, w.num_seqs, w.num_q_heads, w.max_seq_len, part)

    def step(o):
        L.pa_reshape_and_cache(pool, k_new, v_new, slots)
        L.pa_decode(pool, o, q, dc.bt, dc.lens, w.max_seq_len, w.scale, part, ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(out)                                # warm-up outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(out)
    torch.cuda.synchronize()

    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    eager = torch.empty_like(out)
    for rep in range(4):
        # new inputs, written eagerly between replays
        q.copy_(torch.randn(q.shape, generator=gen, device="cuda").half())
        k_new.copy_(torch.randn(k_new.shape, generator=gen, device="cuda").half())
        v_new.copy_(torch.randn(v_new.shape, generator=gen, device="cuda").half())
        torch.cuda.synchronize()
        out.fill_(7.0)
        g.replay()
        torch.cuda.synchronize()
        step(eager)                              # same pool state: rewrites the same bits
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        assert bool(torch.isfinite(out).all())
