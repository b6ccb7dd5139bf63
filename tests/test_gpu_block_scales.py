"""GPU parity of fp8 pools with one scale per (block, KV head), kept beside
the pools and written by pa_reshape_and_cache ("KV Cache memory core",
section 4.4: finer scale grains; quantise on write with the scale kept with
the block).  The bytes AND the scales the device writes must equal the
oracle's bit for bit, over the same sequence of calls: whole blocks written
in one run, appends that raise a block's scale (the rows already there are
re-encoded) and appends that do not, a run that starts a block over, runs cut
by skipped slots, non-finite inputs, and copy_blocks carrying the scales.
Decode parity with these pools runs in tests/test_gpu_decode.py (the
per-block shapes there) and tests/test_gpu_grouped.py."""
import numpy as np
import pytest
import torch

import oracle as O
from paged_kv_cache_72_amd import lib as L
from paged_kv_cache_72_amd import workloads as W
from helpers import DeviceCase, oracle_pool, say

pytestmark = pytest.mark.gpu


def _assert_same(pool, hp, what):
    torch.cuda.synchronize()
    assert np.array_equal(pool.k.cpu().numpy(), hp.k), f"{what}: K bytes"
    assert np.array_equal(pool.v.cpu().numpy(), hp.v), f"{what}: V bytes"
    assert np.array_equal(pool.k_block_scales.cpu().numpy().view(np.uint32),
                          hp.k_blk.view(np.uint32)), f"{what}: K scales"
    assert np.array_equal(pool.v_block_scales.cpu().numpy().view(np.uint32),
                          hp.v_blk.view(np.uint32)), f"{what}: V scales"


@pytest.mark.parametrize("name,make", [
    ("e4m3_bs16", lambda: W.custom("b", 81, [1, 15, 16, 17, 100, 700], 8, 2, 128, 16,
                                   kv_dtype="fp8_e4m3fn", scale_grain="block")),
    ("e5m2_bs8", lambda: W.custom("b", 82, [1, 9, 100, 333], 8, 4, 128, 8,
                                  kv_dtype="fp8_e5m2", scale_grain="block")),
    ("e4m3_d64_bs32", lambda: W.custom("b", 83, [17, 40, 95], 8, 8, 64, 32,
                                       kv_dtype="fp8_e4m3fn", scale_grain="block")),
    ("e5m2_d256_bs128", lambda: W.custom("b", 84, [5, 129, 300], 16, 4, 256, 128,
                                         kv_dtype="fp8_e5m2", scale_grain="block")),
    ("e4m3_prefill_bs16", lambda: W.custom_prefill("b", 85, [7, 0, 30], [20, 33, 5], 8, 4, 128,
                                                   16, kv_dtype="fp8_e4m3fn",
                                                   scale_grain="block")),
])
@pytest.mark.parametrize("poison", [False, True])
def test_workload_writes_bit_exact(name, make, poison):
    w = make()
    say(f"block scales {name} poison={poison}")
    dc = DeviceCase(w, poison=poison)
    hp = oracle_pool(w, poison=poison)
    _assert_same(dc.pool, hp, name)
    # the step's twice-as-large rows raised some blocks' scales
    h0 = O.HostPool.for_workload(w, W.poison_pool_bits(w) if poison else 0)
    keep = np.ones(w.tok_slot.size, bool)
    keep[w.new_idx] = False
    O.scatter(h0, w.tok_k, w.tok_v, np.where(keep, w.tok_slot, -1))
    assert (hp.k_blk > h0.k_blk).any()


@pytest.mark.parametrize("kv", ["fp8_e4m3fn", "fp8_e5m2"])
@pytest.mark.parametrize("bs", [8, 16, 128])
def test_call_sequence_bit_exact(kv, bs):
    """The same calls on both sides: a first run from slot 0, a larger append
    (re-encoding), a smaller append, runs cut by a skipped slot and by a block
    change in one call, a run that starts a block over, non-finite values,
    then a copy of the block."""
    rng = np.random.default_rng(86 + bs)
    H, D, nb = 4, 128, 12
    pool = L.KVPool.allocate(nb, bs, H, D, kv, fill_bits=0x7F, block_scales=True)
    hp = O.HostPool(nb, bs, H, D, kv, fill_bits=0x7F, block_scales=True)

    def call(x, slots, what):
        xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
        sd = torch.from_numpy(np.asarray(slots, np.int64)).cuda()
        L.pa_reshape_and_cache(pool, xd, xd * 0.5, sd)
        O.scatter(hp, x, (x.astype(np.float32) * 0.5).astype(np.float16), np.asarray(slots))
        _assert_same(pool, hp, what)

    def rows(n, mag):
        return (rng.standard_normal((n, H, D)).astype(np.float32) * mag).astype(np.float16)

    b = 3
    half = bs // 2
    call(rows(half, 1.0), np.arange(b * bs, b * bs + half), "first run from slot 0")
    call(rows(2, 4.0), np.arange(b * bs + half, b * bs + half + 2), "larger append")
    call(rows(1, 0.1), [b * bs + half + 2], "smaller append")
    # one call: the rest of block b (two runs split by a skipped slot), then
    # slot 0 of block b + 1
    rest = bs - half - 3
    sl = list(range(b * bs + half + 3, b * bs + bs)) + [(b + 1) * bs]
    if rest >= 2:
        sl.insert(1, -1)
    x = rows(len(sl), 2.0)
    x[0, 1, 5] = np.inf
    x[-1, 2, 7] = np.nan
    call(x, sl, "split runs, block change, non-finite values")
    call(rows(3, 0.5), np.arange(b * bs, b * bs + 3), "a run that starts the block over")
    pr = np.array([[b, 9], [b + 1, 10]], np.int64)
    L.pa_copy_blocks(pool, torch.from_numpy(pr).cuda())
    O.copy_blocks(hp, pr)
    _assert_same(pool, hp, "copy_blocks")
