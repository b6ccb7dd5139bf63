"""GPU tests of the device-argument checks (include/pa_check.h): valid inputs
of every workload shape pass, and each kind of bad entry planted on the host
is found and named.  Planted entries are only ever read by the check kernels,
which bound every access by the sizes they are given; the compute calls are
never launched on them (with CHECK_INPUTS the binding raises first)."""
import numpy as np
import pytest
import torch

from paged_kv_cache_72_amd import lib as L
from paged_kv_cache_72_amd import workloads as W
from helpers import DeviceCase, say

pytestmark = pytest.mark.gpu


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _raises(fn, *words):
    with pytest.raises(L.PaError) as e:
        fn()
    assert e.value.status == L.PA_ERR_INVALID_ARG
    for w in words:
        assert w in str(e.value), str(e.value)
    return str(e.value)


@pytest.fixture(scope="module")
def case():
    w = W.custom("chk", 80, [0, 1, 17, 100, 333], 8, 2, 64, 16)
    return w, DeviceCase(w, poison=True)


def _dec(dc, bt=None, lens=None, max_len=None):
    w = dc.w
    bt = dc.bt if bt is None else _dev(bt)
    lens = dc.lens if lens is None else _dev(lens)
    L.pa_check_decode_inputs(dc.pool, bt, lens, int(w.max_seq_len) if max_len is None else max_len)


def test_valid_workloads_pass():
    for make in (W.tiny, lambda: W.custom("a", 81, [5, 64, 700], 32, 8, 128, 32,
                                          kv_dtype="fp8_e4m3fn"),
                 W.llama3_8b_b64):
        w = make()
        say(f"check valid {w.name}")
        dc = DeviceCase(w, poison=True)
        L.pa_check_decode_inputs(dc.pool, dc.bt, dc.lens, int(w.max_seq_len))
        L.pa_check_slot_mapping(dc.pool, _dev(w.tok_slot.astype(np.int64)))


def test_table_entry_out_of_range(case):
    w, dc = case
    bt = w.block_tables.copy()
    bt[3, 2] = w.num_blocks                     # seq 3 (100 tokens) reads block 2
    _raises(lambda: _dec(dc, bt=bt), f"block_tables[3][2] = {w.num_blocks}", "1 problem")
    bt[4, 0] = -1
    bt[4, 20] = -5                              # seq 4 has 21 blocks: read
    msg = _raises(lambda: _dec(dc, bt=bt), "block_tables[3][2]", "3 problems")
    say(msg)


def test_entries_past_the_context_or_before_the_window_are_not_read(case):
    w, dc = case
    bt = w.block_tables.copy()
    bt[2, 5:] = -7                              # seq 2 has 17 tokens: blocks 0, 1
    _dec(dc, bt=bt)
    pool = L.KVPool(dc.pool.k, dc.pool.v, w.block_size, w.num_kv_heads, w.head_dim,
                    sliding_window=64)
    bt[4, :16] = -1                             # 333 tokens, window 64: first block read is 16
    L.pa_check_decode_inputs(pool, _dev(bt), dc.lens, int(w.max_seq_len))
    bt[4, 16] = -1
    _raises(lambda: L.pa_check_decode_inputs(pool, _dev(bt), dc.lens, int(w.max_seq_len)),
            "block_tables[4][16] = -1")


def test_lengths(case):
    w, dc = case
    lens = w.seq_lens.copy()
    lens[1] = -3
    _raises(lambda: _dec(dc, lens=lens), "seq_lens[1] = -3")
    lens = w.seq_lens.copy()
    _raises(lambda: _dec(dc, max_len=200), "seq_lens[4] = 333", "max_seq_len 200")
    lens[2] = w.block_tables.shape[1] * w.block_size + 1
    _raises(lambda: _dec(dc, lens=lens, max_len=1 << 20), "seq_lens[2]", "max_blocks_per_seq")


def test_slot_mapping(case):
    w, dc = case
    nslots = w.num_blocks * w.block_size
    slots = np.array([5, -1, 17, nslots - 1, -1], np.int64)
    L.pa_check_slot_mapping(dc.pool, _dev(slots))
    slots[2] = nslots
    _raises(lambda: L.pa_check_slot_mapping(dc.pool, _dev(slots)),
            f"slot_mapping[2] = {nslots}")
    slots = np.array([9, 40, 9, 41, 40, 40], np.int64)
    _raises(lambda: L.pa_check_slot_mapping(dc.pool, _dev(slots)),
            "slot 9 is listed more than once", "3 problems")


def test_block_mapping(case):
    w, dc = case
    nb = w.num_blocks
    ok = np.array([[0, 5], [0, 6], [1, 7]], np.int64)
    L.pa_check_block_mapping(dc.pool, _dev(ok))
    _raises(lambda: L.pa_check_block_mapping(dc.pool, _dev(np.array([[0, 5], [nb, 6]]))),
            f"block_mapping[1] = ({nb}, 6)")
    _raises(lambda: L.pa_check_block_mapping(dc.pool, _dev(np.array([[0, 5], [1, 5]]))),
            "block 5 is the destination of more than one pair")
    _raises(lambda: L.pa_check_block_mapping(dc.pool, _dev(np.array([[0, 5], [5, 6]]))),
            "block 5 is both a destination and a source")
    _raises(lambda: L.pa_check_block_mapping(dc.pool, _dev(np.array([[3, 3]]))),
            "block 3 is both")


def test_prefill_inputs():
    w = W.PREFILL_CONFIGS["prefill_tiny"]()
    say(f"check prefill {w.name}")
    dc = DeviceCase(w, poison=True)
    qs = w.q_start.astype(np.int32)
    T = int(qs[-1])
    args = lambda q=qs, mq=w.max_q_len: (dc.pool, _dev(q), dc.bt, dc.lens, T,
                                         int(mq))
    L.pa_check_prefill_inputs(*args())
    bad = qs.copy()
    bad[1], bad[2] = bad[2], bad[1]
    if bad[1] != bad[2]:
        _raises(lambda: L.pa_check_prefill_inputs(*args(q=bad)), "q_start[")
    _raises(lambda: L.pa_check_prefill_inputs(*args(mq=0)), "max_q_len 0")


def test_check_inputs_mode_stops_the_compute_call(case, monkeypatch):
    w, dc = case
    monkeypatch.setattr(L, "CHECK_INPUTS", True)
    y = dc.decode(-1)                           # valid: checked, then run
    bt = w.block_tables.copy()
    bt[4, 3] = 1 << 30
    out = torch.full_like(y, 7.0)
    _raises(lambda: L.pa_decode(dc.pool, out, dc.q, _dev(bt), dc.lens, int(w.max_seq_len),
                                w.scale, -1), "block_tables[4][3]")
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())             # nothing was launched
