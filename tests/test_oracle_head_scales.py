"""Pins for the oracle with one fp8 scale per KV head (CPU only).

Every head's bytes are checked against torch's float8 conversion of x / scale
of that head, and decode and prefill against torch SDPA in float64 on values
dequantised by torch (byte value times the head's scale), on workloads whose
heads differ in magnitude so that a single scale would not reproduce them."""
import numpy as np
import pytest
import torch

import oracle as O
from paged_kv_cache_72_amd import workloads as W


def _torch_codes(x32, scale, dtype):
    return (torch.from_numpy(x32) / torch.tensor(np.float32(scale))).to(dtype).view(torch.uint8).numpy()


def _dt(kv):
    return torch.float8_e4m3fn if kv == "fp8_e4m3fn" else torch.float8_e5m2


@pytest.mark.parametrize("kv", ["fp8_e4m3fn", "fp8_e5m2"])
def test_scatter_uses_each_heads_scale(kv):
    w = W.custom("h", 41, [9, 33], 8, 4, 64, 16, kv_dtype=kv, scale_grain="head")
    assert len(set(np.round(w.k_head_scales, 6))) > 1
    hp = O.pool_for_workload(w)
    bs = w.block_size
    blk, off = w.tok_slot // bs, w.tok_slot % bs
    for h in range(w.num_kv_heads):
        kc = _torch_codes(w.tok_k[:, h].astype(np.float32), w.k_head_scales[h], _dt(kv))
        vc = _torch_codes(w.tok_v[:, h].astype(np.float32), w.v_head_scales[h], _dt(kv))
        assert np.array_equal(hp.k[blk, off, h], kc)
        assert np.array_equal(hp.v[blk, off, h], vc)


def _deq(w, which):
    a = w.tok_k if which == "k" else w.tok_v
    sc = w.k_head_scales if which == "k" else w.v_head_scales
    out = np.empty(a.shape, np.float64)
    for h in range(a.shape[1]):
        codes = _torch_codes(a[:, h].astype(np.float32), sc[h], _dt(w.kv_dtype))
        vals = torch.from_numpy(codes).view(_dt(w.kv_dtype)).to(torch.float32).double().numpy()
        out[:, h] = vals * np.float64(np.float32(sc[h]))
    return out


@pytest.mark.parametrize("kv", ["fp8_e4m3fn", "fp8_e5m2"])
def test_decode_with_head_scales_matches_sdpa(kv):
    w = W.custom("h", 42, [1, 17, 100], 8, 4, 64, 16, kv_dtype=kv, scale_grain="head")
    r = O.decode(O.pool_for_workload(w), w.q, w.block_tables, w.seq_lens, w.scale)
    K, V = _deq(w, "k"), _deq(w, "v")
    g = w.gqa
    for s in range(w.num_seqs):
        idx = np.array([w.token_index(s, t) for t in range(int(w.seq_lens[s]))])
        q = torch.from_numpy(w.q[s].astype(np.float64))[None, :, None, :]
        k = torch.from_numpy(K[idx]).permute(1, 0, 2).repeat_interleave(g, dim=0)[None]
        v = torch.from_numpy(V[idx]).permute(1, 0, 2).repeat_interleave(g, dim=0)[None]
        o = torch.nn.functional.scaled_dot_product_attention(q, k.contiguous(), v.contiguous(),
                                                             scale=float(w.scale))
        np.testing.assert_allclose(r[s], o[0, :, 0].numpy(), rtol=0, atol=1e-12)


def test_prefill_with_head_scales_matches_sdpa():
    w = W.custom_prefill("h", 43, [7, 0], [20, 33], 8, 4, 64, 16, kv_dtype="fp8_e4m3fn",
                         scale_grain="head")
    r = O.prefill(O.pool_for_workload(w), w.q, w.q_start, w.block_tables, w.seq_lens, w.scale)
    K, V = _deq(w, "k"), _deq(w, "v")
    g, qs = w.gqa, w.q_start
    for s in range(w.num_seqs):
        n, ql = int(w.seq_lens[s]), int(w.q_lens[s])
        idx = np.array([w.token_index(s, t) for t in range(n)])
        q = torch.from_numpy(w.q[qs[s]:qs[s + 1]].astype(np.float64)).permute(1, 0, 2)[None]
        k = torch.from_numpy(K[idx]).permute(1, 0, 2).repeat_interleave(g, dim=0)[None]
        v = torch.from_numpy(V[idx]).permute(1, 0, 2).repeat_interleave(g, dim=0)[None]
        mask = torch.from_numpy(np.arange(n)[None, :] <= np.arange(n - ql, n)[:, None])
        o = torch.nn.functional.scaled_dot_product_attention(q.contiguous(), k.contiguous(),
                                                             v.contiguous(), attn_mask=mask,
                                                             scale=float(w.scale))
        np.testing.assert_allclose(r[qs[s]:qs[s + 1]], o[0].permute(1, 0, 2).numpy(), rtol=0,
                                   atol=1e-12)
