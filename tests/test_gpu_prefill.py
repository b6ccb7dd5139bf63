"""GPU parity of pa_prefill against the fp64 oracle.

Each case writes the context and this step's new tokens with
pa_reshape_and_cache into a pool whose unused slots and padding block hold
NaN, runs pa_prefill, and compares every output element with the oracle's
causal attention: |y - r| <= 2e-3 + 1e-2 |r| for fp16 KV, |y - r| <= 3e-2 for
fp8 KV.  Shapes cover head_dim 64/128/256, block sizes 8..128, GQA 1..16 (so
tiles of 128 / gqa tokens with ragged tails, and at head_dim 128 also of 192 /
gqa: PA_PREFILL_GROUPS=3), fp8 e4m3fn and e5m2 pools, one-token and
cache-free prompts, empty sequences, and the full-size prefill workloads on
sampled rows with the library's choice of row groups and the other one."""
import dataclasses
import zlib

import numpy as np
import pytest
import torch

import oracle as O
from paged_kv_cache_72_amd import lib as L
from paged_kv_cache_72_amd import workloads as W
from helpers import (DeviceCase, check_close, oracle_pool, prefill_row_index,
                     sample_prefill_rows, say, seq_token_indices)

pytestmark = pytest.mark.gpu

_RS = np.random.RandomState(94)      # lengths of the many-pairs shape (drawn once, at import)

SHAPES = {
    "tiny": W.prefill_tiny,
    "d128_bs16_g4": lambda: W.custom_prefill("pf", 81, [0, 5, 33, 300], [70, 31, 32, 129],
                                             32, 8, 128, 16),
    "d128_bs8_g7": lambda: W.custom_prefill("pf", 82, [0, 17, 64], [19, 37, 100], 28, 4, 128, 8),
    "d128_bs32_g1": lambda: W.custom_prefill("pf", 83, [0, 200], [130, 257], 4, 4, 128, 32),
    "d64_bs16_g16": lambda: W.custom_prefill("pf", 84, [1, 40], [9, 24], 16, 1, 64, 16),
    "d64_bs64_g3": lambda: W.custom_prefill("pf", 85, [0, 100, 63], [50, 43, 1], 6, 2, 64, 64),
    "d128_bs128_g8": lambda: W.custom_prefill("pf", 86, [120, 0], [33, 16], 16, 2, 128, 128),
    "d128_bs16_g4_e4m3": lambda: W.custom_prefill("pf", 87, [0, 40, 7], [64, 25, 90], 32, 8,
                                                  128, 16, kv_dtype="fp8_e4m3fn"),
    "d64_bs8_g2_e5m2": lambda: W.custom_prefill("pf", 88, [3, 0], [61, 47], 8, 4, 64, 8,
                                                kv_dtype="fp8_e5m2"),
    "decode_like": lambda: W.custom_prefill("pf", 89, [0, 1, 15, 16, 500], [1, 1, 1, 1, 1],
                                            32, 8, 128, 16),
    "empty_seq": lambda: W.custom_prefill("pf", 90, [10, 20, 5], [12, 0, 7], 8, 2, 128, 16),
    "d128_bs16_g4_e4m3_head": lambda: W.custom_prefill("pf", 91, [0, 40], [64, 25], 32, 8, 128,
                                                       16, kv_dtype="fp8_e4m3fn",
                                                       scale_grain="head"),
    # head_dim 256: the hybrid example's full-attention shape
    "d256_bs16_g4": lambda: W.custom_prefill("pf", 92, [0, 5, 33, 300], [70, 31, 32, 129],
                                             16, 4, 256, 16),
    "d256_bs64_g8": lambda: W.custom_prefill("pf", 93, [0, 100], [45, 96], 16, 2, 256, 64),
    # 128 query rows per workgroup at head_dim 256: groups that do not divide
    # it (3: 42 tokens, 126 rows) and the largest group (16: 8 tokens)
    "d256_bs32_g3": lambda: W.custom_prefill("pf", 95, [0, 50, 7], [70, 22, 43], 6, 2, 256, 32),
    "d256_bs8_g16": lambda: W.custom_prefill("pf", 96, [3, 0], [9, 30], 16, 1, 256, 8),
    "d256_bs16_g4_e4m3": lambda: W.custom_prefill("pf", 100, [0, 5, 33, 300], [70, 31, 32, 129],
                                                  16, 4, 256, 16, kv_dtype="fp8_e4m3fn"),
    "d256_bs32_g2_e5m2_head": lambda: W.custom_prefill("pf", 101, [0, 64], [45, 20], 8, 4, 256,
                                                       32, kv_dtype="fp8_e5m2",
                                                       scale_grain="head"),
    # fp8 pools at head_dim 128 (staged as bytes, widened in LDS) at other
    # block sizes, gqa and scale granularities
    "d128_bs8_g4_e5m2": lambda: W.custom_prefill("pf", 97, [0, 30, 5], [40, 17, 70], 32, 8,
                                                 128, 8, kv_dtype="fp8_e5m2"),
    "d128_bs64_g7_e4m3": lambda: W.custom_prefill("pf", 98, [0, 100], [90, 33], 28, 4, 128,
                                                  64, kv_dtype="fp8_e4m3fn"),
    "d128_bs128_g2_e4m3_head": lambda: W.custom_prefill("pf", 99, [130, 0], [20, 50], 8, 4,
                                                        128, 128, kv_dtype="fp8_e4m3fn",
                                                        scale_grain="head"),
    # one fp8 scale per (block, KV head), written by reshape_and_cache
    "d128_bs16_g4_e4m3_block": lambda: W.custom_prefill("pf", 102, [0, 40, 7], [64, 25, 90], 32,
                                                        8, 128, 16, kv_dtype="fp8_e4m3fn",
                                                        scale_grain="block"),
    "d128_bs8_g7_e5m2_block": lambda: W.custom_prefill("pf", 103, [0, 17, 64], [19, 37, 100],
                                                       28, 4, 128, 8, kv_dtype="fp8_e5m2",
                                                       scale_grain="block"),
    "d256_bs16_g4_e5m2_block": lambda: W.custom_prefill("pf", 104, [0, 5, 33, 300],
                                                        [70, 31, 32, 129], 16, 4, 256, 16,
                                                        kv_dtype="fp8_e5m2", scale_grain="block"),
    "d256_bs128_g2_e4m3_block": lambda: W.custom_prefill("pf", 105, [130, 0], [20, 50], 8, 4,
                                                         256, 128, kv_dtype="fp8_e4m3fn",
                                                         scale_grain="block"),
    "d128_bs64_g4_e4m3_block": lambda: W.custom_prefill("pf", 106, [0, 100], [90, 33], 32, 8,
                                                        128, 64, kv_dtype="fp8_e4m3fn",
                                                        scale_grain="block"),
    # 2,600 (sequence, KV head) pairs: more than 256 per XCD, so the workgroups
    # take the pairs in index order instead of ranking them by length
    "many_pairs": lambda: W.custom_prefill("pf", 94, _RS.randint(0, 48, 325).tolist(),
                                           _RS.randint(1, 12, 325).tolist(), 32, 8, 128, 16),
}


D128 = [n for n in SHAPES if n.startswith("d128") or n in ("decode_like", "empty_seq",
                                                             "many_pairs")]
CASES = [(n, "auto") for n in SHAPES] + [(n, g) for n in D128 for g in ("2", "3")]


def set_groups(monkeypatch, groups):
    """Fix the head_dim-128 row groups per wave ("2", "3") or leave the
    library's choice ("auto")."""
    if groups == "auto":
        monkeypatch.delenv("PA_PREFILL_GROUPS", raising=False)
    else:
        monkeypatch.setenv("PA_PREFILL_GROUPS", groups)


@pytest.mark.parametrize("name,groups", CASES, ids=[f"{n}-{g}" for n, g in CASES])
def test_prefill_matches_oracle(name, groups, monkeypatch):
    set_groups(monkeypatch, groups)
    w = SHAPES[name]()
    say(f"prefill {name} groups={groups} q_lens={w.q_lens.tolist()} lens={w.seq_lens.tolist()}")
    dc = DeviceCase(w, poison=True)
    y = dc.prefill().cpu().numpy()
    r = O.prefill(oracle_pool(w, poison=True), w.q, w.q_start, w.block_tables, w.seq_lens,
                  w.scale)
    st = check_close(w, y, r, name)
    say(f"  {st}")


def test_prefill_v_offset_gate():
    """Values offset by +1: outputs sit near 1, so an all-zero output fails."""
    w = W.with_v_offset(SHAPES["d128_bs16_g4"](), 1.0)
    y = DeviceCase(w, poison=True).prefill().cpu().numpy()
    r = O.prefill(oracle_pool(w, poison=True), w.q, w.q_start, w.block_tables, w.seq_lens,
                  w.scale)
    check_close(w, y, r, "v_offset")
    with pytest.raises(AssertionError):
        check_close(w, np.zeros_like(y), r)


def _relabel(w, seed):
    perm = np.random.default_rng(seed).permutation(w.num_blocks)
    bs = w.block_size
    slot = perm[w.tok_slot // bs] * bs + w.tok_slot % bs
    return dataclasses.replace(w, block_tables=perm[w.block_tables].astype(np.int32),
                               tok_slot=slot.astype(np.int64), pad_block=int(perm[w.pad_block]))


@pytest.mark.parametrize("name", ["d128_bs16_g4", "d128_bs8_g7", "d64_bs8_g2_e5m2",
                                  "d128_bs64_g7_e4m3"])
@pytest.mark.parametrize("groups", ["2", "3"])
def test_prefill_relabelling_and_reruns_are_bitwise_equal(name, groups, monkeypatch):
    set_groups(monkeypatch, groups)
    w = SHAPES[name]()
    dc = DeviceCase(w, poison=True)
    a = dc.prefill().clone()
    b = dc.prefill(out=torch.empty_like(a))
    c = DeviceCase(_relabel(w, 5), poison=True).prefill()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))


def test_prefill_rows_beyond_total_q_are_not_written():
    """q_start past total_q: those rows are skipped, the rest still computed."""
    w = SHAPES["d128_bs16_g4"]()
    dc = DeviceCase(w, poison=True)
    T = int(w.q_start[-1])
    cut = int(w.q_start[2]) + 5          # sequence 2 keeps 5 of its rows
    out = torch.full((T + 8,) + tuple(w.q.shape[1:]), 7.0, dtype=torch.float16, device="cuda")
    qs = torch.from_numpy(w.q_start).cuda()
    L.pa_prefill(dc.pool, out[:cut], dc.q[:cut], qs, dc.bt, dc.lens, w.max_q_len, w.scale)
    torch.cuda.synchronize()
    y = out.cpu().numpy().astype(np.float64)
    r = O.prefill(oracle_pool(w, poison=True), w.q, w.q_start, w.block_tables, w.seq_lens,
                  w.scale)
    check_close(w, y[:cut], r[:cut], "kept rows")
    assert np.all(y[cut:] == 7.0)


# (workload, generator, sampled rows, row groups): at head_dim 128 the
# library takes 3 groups on the chunked and cold batches and 2 on the
# prefix-hit one; the other choice of each is run as well
FULL = [
    ("prefill_cold_2000", W.prefill_cold_2000, 24, "auto"),
    ("prefill_chunked_8k", W.prefill_chunked_8k, 24, "auto"),
    ("prefill_chunked_8k", W.prefill_chunked_8k, 24, "2"),
    ("prefill_prefix_hit", W.prefill_prefix_hit, 24, "auto"),
    ("prefill_prefix_hit", W.prefill_prefix_hit, 24, "3"),
    ("prefill_chunked_8k_fp8", W.prefill_chunked_8k_fp8, 24, "auto"),
    ("prefill_chunked_8k_fp8", W.prefill_chunked_8k_fp8, 24, "2"),
    ("prefill_chunked_8k_d256", W.prefill_chunked_8k_d256, 24, "auto"),
    ("prefill_chunked_8k_d256_fp8", W.prefill_chunked_8k_d256_fp8, 24, "auto"),
]


@pytest.mark.parametrize("name,make,nrows,groups", FULL, ids=[f"{c[0]}-{c[3]}" for c in FULL])
def test_prefill_full_size_sampled(name, make, nrows, groups, monkeypatch):
    set_groups(monkeypatch, groups)
    say(f"prefill config {name} groups={groups}: generating")
    w = make()
    rows = sample_prefill_rows(w, nrows, seed=zlib.crc32(name.encode()))
    say(f"prefill config {name}: device run")
    dc = DeviceCase(w, poison=True)
    y = dc.prefill().cpu().numpy()
    assert np.all(np.isfinite(y))
    seqs = sorted({s for s, _, _ in rows})
    tok = seq_token_indices(w, seqs)
    say(f"prefill config {name}: oracle on {len(rows)} rows")
    hp = oracle_pool(w, poison=True, token_idx=tok)
    r = O.prefill(hp, w.q, w.q_start, w.block_tables, w.seq_lens, w.scale, rows=rows)
    idx = prefill_row_index(w, rows)
    st = check_close(w, y[idx], r[idx], name)
    say(f"  {st}")


WINDOW_SHAPES = ["d128_bs16_g4", "d128_bs8_g7", "d64_bs16_g16", "d128_bs16_g4_e4m3",
                 "d128_bs8_g4_e5m2", "d256_bs16_g4", "d128_bs8_g7_e5m2_block"]
# row groups are chosen at head_dim 128 only: both there, the library's elsewhere
WINDOW_CASES = [(n, g) for n in WINDOW_SHAPES
                for g in (("2", "3") if n.startswith("d128") else ("auto",))]


@pytest.mark.parametrize("name,groups", WINDOW_CASES, ids=[f"{n}-{g}" for n, g in WINDOW_CASES])
@pytest.mark.parametrize("win", [1, 31, 32, 33, 100])
def test_sliding_window_prefill(name, groups, win, monkeypatch):
    set_groups(monkeypatch, groups)
    w0 = SHAPES[name]()
    w = dataclasses.replace(w0, window=win, block_tables=w0.block_tables.copy())
    # blocks wholly before the window of a sequence's first new token are
    # never read: point them at the NaN padding block
    bs = w.block_size
    for s in range(w.num_seqs):
        first = max(0, int(w.seq_lens[s]) - int(w.q_lens[s]) - win + 1)
        w.block_tables[s, :first // bs] = w.pad_block
    say(f"prefill window {win} {name}")
    y = DeviceCase(w, poison=True).prefill().cpu().numpy()
    r = O.prefill(oracle_pool(w, poison=True), w.q, w.q_start, w.block_tables, w.seq_lens,
                  w.scale)
    check_close(w, y, r, f"prefill window{win}/{name}")
