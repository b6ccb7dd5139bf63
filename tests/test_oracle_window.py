"""Pins for the oracle's sliding-window attention (CPU only).

A query at position p sees positions p - W + 1 .. p ("Paging saves no KV
bytes", section 5: sliding-window layers whose out-of-window blocks are
released).  Checked against torch SDPA in float64 with an explicit band mask on
K/V from the per-position token arrays, against the closed form W = 1 (the
query's own V), and against full attention when W covers everything."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
from paged_kv_cache_72_amd import workloads as W


def _kv(w, s):
    idx = np.array([w.token_index(s, t) for t in range(int(w.seq_lens[s]))])
    return w.tok_k[idx].astype(np.float64), w.tok_v[idx].astype(np.float64)


def _sdpa(q, K, V, mask, scale, g):
    k = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(g, dim=0)[None]
    v = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(g, dim=0)[None]
    return torch.nn.functional.scaled_dot_product_attention(
        q.contiguous(), k.contiguous(), v.contiguous(), attn_mask=torch.from_numpy(mask),
        scale=scale)[0]


@pytest.mark.parametrize("win", [1, 5, 16, 37, 100])
def test_decode_window_matches_band_sdpa(win):
    w = dataclasses.replace(W.custom("w", 51, [1, 17, 40, 130], 8, 2, 64, 16), window=win)
    r = O.decode(O.pool_for_workload(w), w.q, w.block_tables, w.seq_lens, w.scale)
    for s in range(w.num_seqs):
        n = int(w.seq_lens[s])
        K, V = _kv(w, s)
        mask = (np.arange(n) >= n - win)[None, :]
        q = torch.from_numpy(w.q[s].astype(np.float64))[None, :, None, :]
        o = _sdpa(q, K, V, mask, float(w.scale), w.gqa)[:, 0]
        np.testing.assert_allclose(r[s], o.numpy(), rtol=0, atol=1e-12)
        if win == 1:
            assert np.array_equal(r[s], np.repeat(V[n - 1], w.gqa, axis=0))


@pytest.mark.parametrize("win", [1, 9, 32, 50])
def test_prefill_window_matches_band_sdpa(win):
    w = dataclasses.replace(W.custom_prefill("w", 52, [0, 20, 70], [30, 17, 45], 8, 2, 64, 16),
                            window=win)
    r = O.prefill(O.pool_for_workload(w), w.q, w.q_start, w.block_tables, w.seq_lens, w.scale)
    qs = w.q_start
    for s in range(w.num_seqs):
        n, ql = int(w.seq_lens[s]), int(w.q_lens[s])
        K, V = _kv(w, s)
        pos = np.arange(n - ql, n)[:, None]
        key = np.arange(n)[None, :]
        mask = (key <= pos) & (key > pos - win)
        q = torch.from_numpy(w.q[qs[s]:qs[s + 1]].astype(np.float64)).permute(1, 0, 2)[None]
        o = _sdpa(q, K, V, mask, float(w.scale), w.gqa).permute(1, 0, 2)
        np.testing.assert_allclose(r[qs[s]:qs[s + 1]], o.numpy(), rtol=0, atol=1e-12)


def test_window_covering_everything_is_full_attention():
    w = W.custom("w", 53, [3, 64, 200], 8, 2, 64, 16)
    full = O.decode(O.pool_for_workload(w), w.q, w.block_tables, w.seq_lens, w.scale)
    ww = dataclasses.replace(w, window=200)
    win = O.decode(O.pool_for_workload(ww), w.q, w.block_tables, w.seq_lens, w.scale)
    assert np.array_equal(full, win)
