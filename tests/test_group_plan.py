"""The host planner of the grouped decode schedule, pa_decode_group_plan (CPU
only): every sequence is listed once, groups respect the member cap, the
shared length is exactly the longest run of leading table entries all members
list (in whole 16-token tiles, within every member's length), and groups come
longest first.  Checked against a brute-force restatement on seeded batches
with prefix sharing, and on the prefix-sharing workloads (256 groups of 4
forked sequences whose first child owns a copy of the last prompt block)."""
import numpy as np
import pytest

from paged_kv_cache_72_amd import lib as L
from paged_kv_cache_72_amd import workloads as W


def _plan(w):
    return L.pa_decode_group_plan(w.block_tables, w.seq_lens, w.block_size, w.num_q_heads,
                                  w.num_kv_heads, device="cpu")


def _shared_brute(w, s, t):
    """Positions s and t share: their common run of leading table entries,
    within both lengths, in whole 16-token tiles."""
    bs = w.block_size
    ls, lt = int(w.seq_lens[s]), int(w.seq_lens[t])
    n = min(-(-ls // bs), -(-lt // bs))
    k = 0
    while k < n and w.block_tables[s, k] == w.block_tables[t, k]:
        k += 1
    return min(k * bs, ls, lt) // 16 * 16


def _check(w, gr):
    S = w.num_seqs
    cap = 16 // w.gqa
    assert sorted(gr.members.tolist()) == list(range(S))
    st = gr.member_start
    assert st[0] == 0 and st[-1] == S and np.all(np.diff(st) >= 1) and np.all(np.diff(st) <= cap)
    work = []
    for i in range(gr.num_groups):
        mem = gr.members[st[i]:st[i + 1]]
        sh = gr.member_shared[st[i]:st[i + 1]]
        assert sh[0] == 0
        for k in range(1, len(mem)):
            assert sh[k] == _shared_brute(w, mem[k - 1], mem[k]) > 0
        work.append(sum(-(-int(w.seq_lens[m]) // 16) - int(x) // 16 for m, x in zip(mem, sh)))
    assert work == sorted(work, reverse=True)
    return work


@pytest.mark.parametrize("Hq,Hkv,bs", [(32, 8, 16), (28, 4, 8), (8, 4, 32), (4, 4, 16),
                                       (16, 1, 64), (16, 2, 16)])
def test_plan_on_seeded_shared_prefix_batches(Hq, Hkv, bs):
    groups = [(40, [0, 3, 17, 100]), (64, [1, 1, 1, 1, 1]), (5, [10, 20]),
              (300, list(range(50, 140, 10))), (16, [0] * 20), (1000, [7, 7])]
    w = W.shared_prefix_batch("plan", 5, groups, Hq, Hkv, 64, bs)
    _check(w, _plan(w))


@pytest.mark.parametrize("bs", [16, 8])
def test_plan_on_the_prefix_sharing_workload(bs):
    w = W.prefix_share(bs)
    gr = _plan(w)
    _check(w, gr)
    # 256 groups of 4; child 0 owns a copy of the last prompt block: the
    # other three share all 256 prompt tokens, child 0 the 240 before it, and
    # sorting by table rows puts child 0 first or last
    assert gr.num_groups == 256 and np.all(np.diff(gr.member_start) == 4)
    for i in range(256):
        mem = gr.members[4 * i:4 * i + 4]
        assert sorted(mem // 4) == [mem[0] // 4] * 4
        sh = gr.member_shared[4 * i:4 * i + 4].tolist()
        assert sh in ([0, 240, 256, 256], [0, 256, 256, 240])
        # every distinct (tile, block) of the group is read once
        tiles = {(t, int(w.block_tables[m, t * 16 // bs])) for m in mem
                 for t in range(-(-int(w.seq_lens[m]) // 16))}
        if bs == 16:
            assert sum(-(-int(w.seq_lens[m]) // 16) - x // 16 for m, x in zip(mem, sh)) == \
                len(tiles)


def test_plan_without_sharing_gives_singletons():
    w = W.llama3_8b_b64()
    gr = _plan(w)
    _check(w, gr)
    assert gr.num_groups == w.num_seqs and np.all(gr.member_shared == 0)


def test_plan_argument_checks():
    bt = np.zeros((2, 3), np.int32)
    lens = np.array([5, 5], np.int32)
    for hq, hkv in ((20, 8), (136, 8), (4, 8)):        # not a multiple; ratio > 16; fewer q heads
        with pytest.raises(L.PaError):
            L.pa_decode_group_plan(bt, lens, 16, hq, hkv, device="cpu")
    gr = L.pa_decode_group_plan(bt, lens, 16, 24, 8, device="cpu")
    assert gr.num_groups == 2 and list(gr.member_shared) == [0, 0]


def test_grouped_refuses_window_pools_on_the_host():
    """Argument checks that return before anything would launch (no GPU)."""
    import ctypes as C
    lib = L.load()
    pool = L.pa_kv_pool(16, 16, 8, 0, 16, 2, 64, L.PA_KV_F16, 1.0, 1.0, 0, 100, None, None)
    st = lib.pa_decode_grouped(C.byref(pool), 16, 16, 1, 8, 16, 1, 16, 8, C.c_float(0.1), 1, 16,
                               16, 16, 0, None, 0, None)
    assert st == L.PA_ERR_UNSUPPORTED and "sliding" in L.pa_last_error()
    pool.sliding_window = 0
    assert lib.pa_decode_grouped_plan(C.byref(pool), 1000, 8, 600, 250, 0) == L.GROUPED_FLAT
    assert lib.pa_decode_grouped_plan(C.byref(pool), 6000, 8, 600, 250, 0) == L.GROUPED_PER_GROUP
    assert lib.pa_decode_grouped_plan(C.byref(pool), 6000, 8, 600, 250, 1) == L.PA_ERR_UNSUPPORTED
    assert lib.pa_decode_grouped_plan(C.byref(pool), 10, 8, 600, 11, 0) == L.PA_ERR_INVALID_ARG
    assert lib.pa_decode_grouped_workspace_size(C.byref(pool), 1000, 8, 600, 250, 2) == 0
    ws = lib.pa_decode_grouped_workspace_size(C.byref(pool), 1000, 8, 600, 250, 0)
    ranges = min(2048 // 2, 1000 * 38 // 8)              # 4 KiB fp16 tiles at head_dim 64
    assert ws == 1024 + ranges * 2 * 2 * 16 * 66 * 4
