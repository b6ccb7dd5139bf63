"""Seeded synthetic decode workloads (input construction only).

This module draws everything a paged-attention decode step consumes and nothing
it computes: per-sequence context lengths, physical block ids handed out from a
seeded shuffled free list, the pool slot of every token, and fp16 q/K/V values.
It holds no attention, softmax or fp8-coding arithmetic, so the GPU path and the
CPU oracle can both take their inputs from here without sharing any of the
method.

Shapes follow the pages' workloads:
  * the block pool of one layer is ``[num_blocks, block_size, num_kv_heads,
    head_dim]`` ("KV Cache memory core", section 2.2 code sketch);
  * a sequence's ``block_table`` maps logical block j to a physical id, stacked
    into a 2-D ``[num_seqs, max_num_blocks]`` tensor, and ``slot_mapping`` gives
    each new token's absolute slot ``block_id * block_size + offset``
    ("vLLM intro part 2", section 3.2);
  * the number of blocks a sequence holds is ``cdiv(num_tokens, block_size)``
    ("Paging saves no KV bytes", section 3).

Random streams: ``SeedSequence(seed).spawn(6)`` gives, in this order, the
children for lengths, free-list permutation, q, K, V and needles.  Large K/V
draws are split into fixed 16K-token chunks, each with its own grandchild seed,
so the bytes do not depend on how many threads fill them.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os
from typing import Optional

import numpy as np

F16_NAN_BITS = np.uint16(0x7E00)   # quiet NaN in IEEE binary16
E4M3_NAN_BYTE = np.uint8(0x7F)     # S.1111.111 is NaN in OCP e4m3fn
E4M3_MAX = np.float32(448.0)       # largest finite OCP e4m3fn magnitude
E5M2_MAX = np.float32(57344.0)     # largest finite OCP e5m2 magnitude
E5M2_NAN_BYTE = np.uint8(0x7F)     # S.11111.11 is a NaN in OCP e5m2
FP8_DTYPES = ("fp8_e4m3fn", "fp8_e5m2")


def fp8_max(kv_dtype: str) -> np.float32:
    """Largest finite magnitude of a pool's fp8 format (sets the per-pool scale)."""
    return E5M2_MAX if kv_dtype == "fp8_e5m2" else E4M3_MAX

_CHUNK_TOKENS = 16384


def cdiv(a: int, b: int) -> int:
    """Ceiling division: blocks needed for ``a`` tokens at ``b`` tokens/block."""
    return -(-int(a) // int(b))


@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    kv_dtype: str                    # "f16", "fp8_e4m3fn" or "fp8_e5m2"
    scale: float                     # softmax scale (fp32 value)
    k_scale: float                   # per-tensor fp8 scale (1.0 for f16)
    v_scale: float
    seq_lens: np.ndarray             # int32 [S]
    block_tables: np.ndarray         # int32 [S, max_blocks]; padding -> pad_block
    pad_block: int                   # physical id table padding points at
    used_blocks: np.ndarray          # int32 ids holding at least one token
    tok_k: np.ndarray                # float16 [T, Hkv, D] every context token's K
    tok_v: np.ndarray                # float16 [T, Hkv, D]
    tok_slot: np.ndarray             # int64 [T] absolute pool slot of each token
    new_idx: np.ndarray              # int64 indices into tok_* written this step
    q: np.ndarray                    # float16 [S, Hq, D]
    partition_size: int = 0          # partition the workload names (0: none)
    cow_pairs: Optional[np.ndarray] = None      # int64 [N, 2] (src, dst)
    block_tables_before_cow: Optional[np.ndarray] = None
    group_size: int = 1              # sequences forked from one prompt
    prefix_tokens: int = 0
    variant: str = "plain"
    # where each sequence's tokens sit in tok_*: positions t < own_from[s] are a
    # shared prompt starting at shared_start[s]; the rest start at own_start[s]
    own_from: Optional[np.ndarray] = None
    own_start: Optional[np.ndarray] = None
    shared_start: Optional[np.ndarray] = None
    # prefill: sequence s brings q_lens[s] new tokens (the last q_lens[s] of its
    # seq_lens[s] positions); q is then [sum(q_lens), Hq, D], sequence after
    # sequence.  None for decode (one query token per sequence).
    q_lens: Optional[np.ndarray] = None
    # fp8 pools with one scale per KV head (float32 [Hkv]); None: per-tensor scales
    k_head_scales: Optional[np.ndarray] = None
    v_head_scales: Optional[np.ndarray] = None
    # sliding-window layer: a query at position p sees positions p - window + 1 .. p
    window: int = 0
    # fp8 pools with one scale per (block, KV head), kept beside the pools and
    # written by reshape_and_cache (k_scale / v_scale are then unused)
    block_scales: bool = False

    @property
    def is_prefill(self) -> bool:
        return self.q_lens is not None

    @property
    def q_start(self) -> np.ndarray:
        """int32 [S + 1]: sequence s owns q rows [q_start[s], q_start[s + 1])."""
        ql = self.q_lens if self.q_lens is not None else np.ones(self.num_seqs, np.int32)
        return np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max()) if self.q_lens is not None and self.q_lens.size else 1

    def token_index(self, s: int, t: int) -> int:
        if t < int(self.own_from[s]):
            return int(self.shared_start[s]) + t
        return int(self.own_start[s]) + t - int(self.own_from[s])

    @property
    def max_blocks(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.seq_lens.size else 0

    @property
    def gqa(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def kv_elem_bytes(self) -> int:
        return 1 if self.kv_dtype in FP8_DTYPES else 2

    @property
    def new_slots(self) -> np.ndarray:
        return self.tok_slot[self.new_idx]

    @property
    def has_shared_blocks(self) -> bool:
        """True when some physical block is listed by more than one sequence."""
        nb = (self.seq_lens.astype(np.int64) + self.block_size - 1) // self.block_size
        ids = np.concatenate([self.block_tables[s, :nb[s]] for s in range(self.num_seqs)])
        return bool(np.unique(ids).size < ids.size)


# --------------------------------------------------------------------------
# drawing helpers


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal_f16(seed_seq: np.random.SeedSequence, shape, parallel_axis_len: int) -> np.ndarray:
    """N(0,1) drawn in fp32 and rounded to fp16, filled in fixed token chunks."""
    out = np.empty(shape, dtype=np.float16)
    n = parallel_axis_len
    nchunks = max(1, cdiv(n, _CHUNK_TOKENS))
    kids = seed_seq.spawn(nchunks)
    row = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    flat = out.reshape(n, row)

    def fill(i: int) -> None:
        lo, hi = i * _CHUNK_TOKENS, min(n, (i + 1) * _CHUNK_TOKENS)
        g = np.random.default_rng(kids[i])
        flat[lo:hi] = g.standard_normal((hi - lo, row), dtype=np.float32).astype(np.float16)

    if nchunks == 1:
        fill(0)
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def _amax_per_head_f32(a: np.ndarray) -> np.ndarray:
    """max |a| over tokens and dims for each KV head of [T, Hkv, D], as fp32."""
    n = a.shape[0]
    out = np.zeros(a.shape[1], np.float32)
    for lo in range(0, n, _CHUNK_TOKENS):
        part = np.abs(a[lo:lo + _CHUNK_TOKENS]).max(axis=(0, 2)).astype(np.float32)
        out = np.maximum(out, part)
    return out


def fp8_scales(kv_dtype: str, tok_k: np.ndarray, tok_v: np.ndarray, grain: str = "tensor"):
    """(k_scale, v_scale, k_head_scales, v_head_scales): amax / fp8 max, per
    tensor, or per KV head when grain == "head" (then the tensor scales are 1)."""
    if kv_dtype not in FP8_DTYPES:
        return 1.0, 1.0, None, None
    mx = fp8_max(kv_dtype)
    if grain == "head":
        kh = (_amax_per_head_f32(tok_k) / mx).astype(np.float32)
        vh = (_amax_per_head_f32(tok_v) / mx).astype(np.float32)
        return 1.0, 1.0, kh, vh
    return (float(_amax_f32(tok_k) / mx), float(_amax_f32(tok_v) / mx), None, None)


def _amax_f32(a: np.ndarray) -> np.float32:
    """max |a| over an fp16 array, as fp32 (exact: fp16 values are fp32 values)."""
    n = a.shape[0]
    nchunks = max(1, cdiv(n, _CHUNK_TOKENS))

    def part(i: int) -> float:
        lo, hi = i * _CHUNK_TOKENS, min(n, (i + 1) * _CHUNK_TOKENS)
        return float(np.abs(a[lo:hi]).max())

    with _cf.ThreadPoolExecutor(_threads()) as ex:
        return np.float32(max(ex.map(part, range(nchunks))))


class _FreeList:
    """Physical ids popped in the order of a seeded permutation."""

    def __init__(self, num_blocks: int, rng: np.random.Generator):
        self.order = rng.permutation(num_blocks).astype(np.int64)
        self.pos = 0

    def take(self, n: int) -> np.ndarray:
        if self.pos + n > self.order.size:
            raise ValueError(f"pool exhausted: need {n}, have {self.order.size - self.pos}")
        ids = self.order[self.pos:self.pos + n]
        self.pos += n
        return ids.copy()


def _slots_for(table_row: np.ndarray, ntok: int, bs: int, start: int = 0) -> np.ndarray:
    t = np.arange(start, start + ntok, dtype=np.int64)
    return table_row[t // bs].astype(np.int64) * bs + (t % bs)


def _finish(name, seed, S, Hq, Hkv, D, bs, num_blocks, kv_dtype, lens, tables, pad_block,
            tok_slot, new_idx, ss, partition_size=0, q_rows=None, scale_grain="tensor",
            **extra) -> Workload:
    T = int(tok_slot.size)
    nq = S if q_rows is None else int(q_rows)
    q = _normal_f16(ss[2], (nq, Hq, D), nq)
    tok_k = _normal_f16(ss[3], (T, Hkv, D), T)
    tok_v = _normal_f16(ss[4], (T, Hkv, D), T)
    if scale_grain == "head":
        # heads of different magnitude, so that one scale per tensor would not fit all
        mult = (2.0 ** np.arange(Hkv) % 7 + 0.25).astype(np.float32)[None, :, None]
        tok_k = (tok_k.astype(np.float32) * mult).astype(np.float16)
        tok_v = (tok_v.astype(np.float32) * mult[:, ::-1]).astype(np.float16)
    if scale_grain == "block":
        # blocks of different magnitude (2^-3 .. 2^0 by physical id: values of
        # the size the fp8 gate is derived for), and this step's writes twice
        # as large, so that appending to a block raises its scale and
        # re-encodes the rows already there
        e = ((tok_slot // bs) * 5 % 4 - 3).astype(np.float32)
        mult = (2.0 ** e)[:, None, None].astype(np.float32)
        mult[np.asarray(new_idx, np.int64)] *= 2.0
        tok_k = (tok_k.astype(np.float32) * mult).astype(np.float16)
        tok_v = (tok_v.astype(np.float32) * mult[:, :, ::-1]).astype(np.float16)
        extra["block_scales"] = True
        k_scale = v_scale = 1.0
        k_head = v_head = None
    else:
        k_scale, v_scale, k_head, v_head = fp8_scales(kv_dtype, tok_k, tok_v, scale_grain)
    extra.setdefault("k_head_scales", k_head)
    extra.setdefault("v_head_scales", v_head)
    used = np.unique(tok_slot // bs).astype(np.int32)
    return Workload(name=name, seed=seed, num_seqs=S, num_q_heads=Hq, num_kv_heads=Hkv,
                    head_dim=D, block_size=bs, num_blocks=num_blocks, kv_dtype=kv_dtype,
                    scale=float(np.float32(1.0) / np.sqrt(np.float32(D))),
                    k_scale=k_scale, v_scale=v_scale, seq_lens=lens.astype(np.int32),
                    block_tables=tables.astype(np.int32), pad_block=int(pad_block),
                    used_blocks=used, tok_k=tok_k, tok_v=tok_v,
                    tok_slot=tok_slot.astype(np.int64), new_idx=new_idx.astype(np.int64), q=q,
                    partition_size=partition_size, **extra)


def _independent(name, seed, lens, Hq, Hkv, D, bs, num_blocks, kv_dtype="f16",
                 partition_size=0, scale_grain="tensor") -> Workload:
    """Sequences with private blocks; the last token of each is this step's write."""
    ss = np.random.SeedSequence(seed).spawn(6)
    S = len(lens)
    free = _FreeList(num_blocks, np.random.default_rng(ss[1]))
    nb = [cdiv(n, bs) for n in lens]
    max_blocks = max(1, max(nb))
    blocks = [free.take(n) for n in nb]
    pad_block = int(free.take(1)[0])          # table padding target (never a real block)
    tables = np.full((S, max_blocks), pad_block, dtype=np.int64)
    slots, new_idx, pos = [], [], 0
    own_start = np.zeros(S, np.int64)
    for s in range(S):
        tables[s, :nb[s]] = blocks[s]
        slots.append(_slots_for(tables[s], int(lens[s]), bs))
        own_start[s] = pos
        pos += int(lens[s])
        if lens[s] > 0:
            new_idx.append(pos - 1)
    tok_slot = np.concatenate(slots) if slots else np.zeros(0, np.int64)
    return _finish(name, seed, S, Hq, Hkv, D, bs, num_blocks, kv_dtype, np.asarray(lens),
                   tables, pad_block, tok_slot, np.asarray(new_idx, np.int64), ss,
                   partition_size=partition_size, scale_grain=scale_grain,
                   own_from=np.zeros(S, np.int64),
                   own_start=own_start, shared_start=np.full(S, -1, np.int64))


def _prefill_independent(name, seed, ctx_lens, q_lens, Hq, Hkv, D, bs, num_blocks,
                         kv_dtype="f16", scale_grain="tensor") -> Workload:
    """Sequences with private blocks: ctx_lens[s] cached tokens followed by
    q_lens[s] new ones, which are this step's writes and queries."""
    ss = np.random.SeedSequence(seed).spawn(6)
    ctx = np.asarray(ctx_lens, np.int64)
    ql = np.asarray(q_lens, np.int64)
    lens = ctx + ql
    S = len(lens)
    free = _FreeList(num_blocks, np.random.default_rng(ss[1]))
    nb = [cdiv(int(n), bs) for n in lens]
    max_blocks = max(1, max(nb))
    blocks = [free.take(n) for n in nb]
    pad_block = int(free.take(1)[0])
    tables = np.full((S, max_blocks), pad_block, dtype=np.int64)
    slots, new_idx, pos = [], [], 0
    own_start = np.zeros(S, np.int64)
    for s in range(S):
        tables[s, :nb[s]] = blocks[s]
        slots.append(_slots_for(tables[s], int(lens[s]), bs))
        own_start[s] = pos
        new_idx.append(np.arange(pos + ctx[s], pos + lens[s], dtype=np.int64))
        pos += int(lens[s])
    tok_slot = np.concatenate(slots) if slots else np.zeros(0, np.int64)
    return _finish(name, seed, S, Hq, Hkv, D, bs, num_blocks, kv_dtype, lens, tables, pad_block,
                   tok_slot, np.concatenate(new_idx), ss, q_rows=int(ql.sum()),
                   q_lens=ql.astype(np.int32), scale_grain=scale_grain,
                   own_from=np.zeros(S, np.int64),
                   own_start=own_start, shared_start=np.full(S, -1, np.int64))


# --------------------------------------------------------------------------
# the five workloads


def tiny(seed: int = 7201) -> Workload:
    """4 sequences of lengths {1,17,33,100}; 8 query / 2 KV heads, head_dim 64,
    block_size 16, a 64-block fp16 pool whose ids are a seeded permutation."""
    return _independent("tiny", seed, [1, 17, 33, 100], 8, 2, 64, 16, 64)


def llama3_8b_b64(seed: int = 7202) -> Workload:
    """Llama-3-8B-shaped single-layer decode: 64 sequences, lengths uniform in
    [512, 4096]; 32 query / 8 KV heads, head_dim 128, block_size 16; a
    20,000-block fp16 pool from a shuffled free list; 64 new tokens written."""
    ss = np.random.SeedSequence(seed).spawn(6)
    lens = np.random.default_rng(ss[0]).integers(512, 4096, size=64, endpoint=True)
    return _independent("llama3_8b_b64", seed, lens.tolist(), 32, 8, 128, 16, 20000)


def llama3_8b_b64_w1024(seed: int = 7202) -> Workload:
    """The Llama-3-8B-shaped batch of 64 as a sliding-window layer with a
    1,024-token window: each query reads only its last 1,024 positions."""
    return dataclasses.replace(llama3_8b_b64(seed), name="llama3_8b_b64_w1024", window=1024)


def llama3_8b_b64_bs(block_size: int, seed: int = 7202) -> Workload:
    """The Llama-3-8B-shaped batch of 64 (same lengths and heads as
    llama3_8b_b64) in blocks of 64 or 128 tokens, the top of the pages' block
    size range; the pool holds the same 320,000 token slots."""
    ss = np.random.SeedSequence(seed).spawn(6)
    lens = np.random.default_rng(ss[0]).integers(512, 4096, size=64, endpoint=True)
    return _independent(f"llama3_8b_b64_bs{block_size}", seed, lens.tolist(), 32, 8, 128,
                        block_size, 320000 // block_size)


def b64_d64(seed: int = 7209) -> Workload:
    """The batch shape of llama3_8b_b64 (64 sequences, lengths uniform in
    [512, 4096], 32 query / 8 KV heads, block_size 16, fp16) at head_dim 64:
    2 KiB of K and V per token, half of the head_dim 128 case."""
    ss = np.random.SeedSequence(seed).spawn(6)
    lens = np.random.default_rng(ss[0]).integers(512, 4096, size=64, endpoint=True)
    return _independent("b64_d64", seed, lens.tolist(), 32, 8, 64, 16, 20000)


def hybrid_d256_b64(seed: int = 7208) -> Workload:
    """A full-attention layer of a hybrid model with head_dim 256 and 4 KV
    heads, the shape of the pages' hybrid example ("Paging saves no KV bytes",
    section 5), at the batch of llama3_8b_b64: 64 sequences, lengths uniform in
    [512, 4096]; 16 query heads (GQA 4: the pages give no query-head count),
    block_size 16, fp16, 20,000-block pool.  4 KiB of K and V per token, as
    for Llama-3-8B."""
    ss = np.random.SeedSequence(seed).spawn(6)
    lens = np.random.default_rng(ss[0]).integers(512, 4096, size=64, endpoint=True)
    return _independent("hybrid_d256_b64", seed, lens.tolist(), 16, 4, 256, 16, 20000)


def qwen25_7b_8k(seed: int = 7203) -> Workload:
    """Qwen2.5-7B-shaped decode at full context: 13 sequences x 8192 tokens
    (512 blocks each); 28 query / 4 KV heads (GQA 7), head_dim 128, block_size
    16, fp16; non-contiguous physical blocks; one slot write per sequence."""
    return _independent("qwen25_7b_8k", seed, [8192] * 13, 28, 4, 128, 16, 8192)


def long_fp8(seed: int = 7206) -> Workload:
    """Long-context split-KV: 8 sequences x 131,072 tokens; 32 query / 8 KV
    heads, head_dim 128, block_size 32; KV stored as OCP fp8 e4m3fn with a
    per-tensor fp32 scale (K/V ~ N(0,1) before quantisation); 512-token
    partitions followed by a log-sum-exp reduce; fp16 output."""
    return _independent("long_fp8", seed, [131072] * 8, 32, 8, 128, 32, 36864,
                        kv_dtype="fp8_e4m3fn", partition_size=512)


def long_fp8_block(seed: int = 7206) -> Workload:
    """The long-context batch of long_fp8 (same lengths, blocks and values)
    with one e4m3fn scale per (block, KV head), written by reshape_and_cache
    as the blocks fill (amax of the block's rows / 448, raised and re-encoded
    as later rows exceed it)."""
    return _independent("long_fp8_block", seed, [131072] * 8, 32, 8, 128, 32, 36864,
                        kv_dtype="fp8_e4m3fn", partition_size=512, scale_grain="block")


def long_e5m2(seed: int = 7207) -> Workload:
    """The long-context split-KV shape of long_fp8 (8 x 131,072 tokens, 32 / 8
    heads, head_dim 128, block_size 32, 512-token partitions) with the KV
    stored as OCP fp8 e5m2 (per-tensor fp32 scale = amax / 57344)."""
    return _independent("long_e5m2", seed, [131072] * 8, 32, 8, 128, 32, 36864,
                        kv_dtype="fp8_e5m2", partition_size=512)


def prefix_share(block_size: int = 16, seed: Optional[int] = None) -> Workload:
    """Short requests with parallel-sampling prefix sharing: 1,024 sequences in
    groups of 4 that share a 256-token prompt; tails of 1-40 tokens (717 of
    them, 70%) or 100-300 tokens (307, 30%), assigned by a seeded shuffle;
    32 query / 8 KV heads, head_dim 128, fp16.  On fork, child 0 of every group
    takes a copy-on-write copy of the group's last prompt block (one
    copy_blocks call with 256 pairs) and its table is retargeted to the copy."""
    if seed is None:
        seed = 7204 if block_size == 16 else 7205
    ss = np.random.SeedSequence(seed).spawn(6)
    rl = np.random.default_rng(ss[0])
    n_groups, gsz, prefix = 256, 4, 256
    S = n_groups * gsz
    n_short = 717
    tails = np.concatenate([rl.integers(1, 40, size=n_short, endpoint=True),
                            rl.integers(100, 300, size=S - n_short, endpoint=True)])
    tails = tails[rl.permutation(S)]
    lens = prefix + tails
    num_blocks = 12288 if block_size == 16 else 24576
    free = _FreeList(num_blocks, np.random.default_rng(ss[1]))
    npb = cdiv(prefix, block_size)
    max_blocks = int(max(cdiv(int(n), block_size) for n in lens))
    tables = np.zeros((S, max_blocks), dtype=np.int64)
    slots, new_idx, pos = [], [], 0
    prefix_blocks = []
    own_start = np.zeros(S, np.int64)
    shared_start = np.zeros(S, np.int64)
    for gi in range(n_groups):
        pb = free.take(npb)
        prefix_blocks.append(pb)
        slots.append(_slots_for(pb, prefix, block_size))
        shared_start[gi * gsz:(gi + 1) * gsz] = pos
        pos += prefix
        for c in range(gsz):
            s = gi * gsz + c
            tail = int(tails[s])
            own_start[s] = pos
            first_tail_blk = prefix // block_size      # prompt is block aligned
            ntail_blk = cdiv(int(lens[s]), block_size) - first_tail_blk
            tables[s, :npb] = pb
            tables[s, first_tail_blk:first_tail_blk + ntail_blk] = free.take(ntail_blk)
            slots.append(_slots_for(tables[s], tail, block_size, start=prefix))
            pos += tail
            new_idx.append(pos - 1)
    cow_dst = free.take(n_groups)
    pad_block = int(free.take(1)[0])
    for s in range(S):
        nb = cdiv(int(lens[s]), block_size)
        tables[s, nb:] = pad_block
    before = tables.copy()
    cow = np.zeros((n_groups, 2), dtype=np.int64)
    for gi in range(n_groups):
        src = int(prefix_blocks[gi][-1])
        cow[gi] = (src, int(cow_dst[gi]))
        tables[gi * gsz, npb - 1] = cow_dst[gi]
    tok_slot = np.concatenate(slots)
    return _finish(f"prefix_share_bs{block_size}", seed, S, 32, 8, 128, block_size, num_blocks,
                   "f16", lens, tables, pad_block, tok_slot, np.asarray(new_idx, np.int64), ss,
                   cow_pairs=cow, block_tables_before_cow=before.astype(np.int32),
                   group_size=gsz, prefix_tokens=prefix,
                   own_from=np.full(S, prefix, np.int64), own_start=own_start,
                   shared_start=shared_start)


def shared_prefix_batch(name: str, seed: int, groups, Hq: int, Hkv: int, D: int, bs: int,
                        num_blocks: Optional[int] = None, kv_dtype: str = "f16",
                        scale_grain: str = "tensor") -> Workload:
    """Sequences that reuse a cached prompt prefix, as prefix-cache hits do:
    ``groups`` lists (prompt_tokens, [tail lengths]) pairs, one sequence per
    tail; the members of a group list the same physical blocks for the
    prompt's FULL blocks (written once: the blocks a prefix cache can hit),
    while the rest of the prompt (a partial block) and each member's tail sit
    in the member's own blocks.  The last token of every sequence is this
    step's write."""
    ss = np.random.SeedSequence(seed).spawn(6)
    lens = [int(P) + int(t) for P, tails in groups for t in tails]
    S = len(lens)
    need = sum(int(P) // bs + sum(cdiv(int(P) + int(t), bs) - int(P) // bs for t in tails)
               for P, tails in groups) + 1
    if num_blocks is None:
        num_blocks = max(need + 8, 2 * need)
    free = _FreeList(num_blocks, np.random.default_rng(ss[1]))
    max_blocks = max(1, max(cdiv(n, bs) for n in lens))
    tables = np.zeros((S, max_blocks), np.int64)
    slots, new_idx, pos, s = [], [], 0, 0
    own_from = np.zeros(S, np.int64)
    own_start = np.zeros(S, np.int64)
    shared_start = np.full(S, -1, np.int64)
    for P, tails in groups:
        full = int(P) // bs
        fb = free.take(full)
        slots.append(_slots_for(fb, full * bs, bs))
        g_start = pos
        pos += full * bs
        for t in tails:
            n = int(P) + int(t)
            tables[s, :full] = fb
            tables[s, full:cdiv(n, bs)] = free.take(cdiv(n, bs) - full)
            own_from[s], shared_start[s], own_start[s] = full * bs, g_start, pos
            slots.append(_slots_for(tables[s], n - full * bs, bs, start=full * bs))
            pos += n - full * bs
            if n > full * bs:               # a member whose context is all shared writes nothing
                new_idx.append(pos - 1)
            s += 1
    pad_block = int(free.take(1)[0])
    for i in range(S):
        tables[i, cdiv(lens[i], bs):] = pad_block
    tok_slot = np.concatenate(slots) if slots else np.zeros(0, np.int64)
    return _finish(name, seed, S, Hq, Hkv, D, bs, num_blocks, kv_dtype, np.asarray(lens), tables,
                   pad_block, tok_slot, np.asarray(new_idx, np.int64), ss,
                   scale_grain=scale_grain, own_from=own_from, own_start=own_start,
                   shared_start=shared_start)


# --------------------------------------------------------------------------
# prefill workloads (new tokens are written by reshape_and_cache, then attend
# causally over the paged context)


def prefill_tiny(seed: int = 7211) -> Workload:
    """5 sequences, cached lengths {0,3,16,100,0} plus {1,5,17,40,33} new
    tokens; 8 query / 2 KV heads, head_dim 64, block_size 16, fp16."""
    return _prefill_independent("prefill_tiny", seed, [0, 3, 16, 100, 0], [1, 5, 17, 40, 33],
                                8, 2, 64, 16, 64)


def prefill_cold_2000(seed: int = 7212) -> Workload:
    """Cold prefill of 2,000-token prompts (the pages' prefix-cache example
    before any hit): 8 requests, nothing cached, 16,000 query rows; Llama-3-8B
    shape (32 query / 8 KV heads, head_dim 128, block_size 16, fp16)."""
    return _prefill_independent("prefill_cold_2000", seed, [0] * 8, [2000] * 8, 32, 8, 128,
                                16, 2048)


def prefill_chunked_8k(seed: int = 7213) -> Workload:
    """Chunked prefill under an 8,192-token budget: 16 sequences each bring a
    512-token chunk on top of 0..3,584 cached tokens (multiples of 512, seeded);
    Llama-3-8B shape, block_size 16, fp16."""
    rng = np.random.default_rng(np.random.SeedSequence(seed).spawn(7)[6])
    ctx = (rng.integers(0, 8, size=16) * 512).tolist()
    return _prefill_independent("prefill_chunked_8k", seed, ctx, [512] * 16, 32, 8, 128, 16,
                                8192)


def prefill_chunked_8k_fp8(seed: int = 7213) -> Workload:
    """The chunked 8K batch of prefill_chunked_8k (same lengths and chunks)
    with the KV cache stored as OCP fp8 e4m3fn, one scale per tensor."""
    rng = np.random.default_rng(np.random.SeedSequence(seed).spawn(7)[6])
    ctx = (rng.integers(0, 8, size=16) * 512).tolist()
    return _prefill_independent("prefill_chunked_8k_fp8", seed, ctx, [512] * 16, 32, 8, 128, 16,
                                8192, kv_dtype="fp8_e4m3fn")


def prefill_chunked_8k_d256(seed: int = 7213) -> Workload:
    """The chunked 8K batch of prefill_chunked_8k (same lengths and chunks) at
    head_dim 256 with 16 query / 4 KV heads, the hybrid example's
    full-attention shape; fp16, block_size 16."""
    rng = np.random.default_rng(np.random.SeedSequence(seed).spawn(7)[6])
    ctx = (rng.integers(0, 8, size=16) * 512).tolist()
    return _prefill_independent("prefill_chunked_8k_d256", seed, ctx, [512] * 16, 16, 4, 256,
                                16, 8192)


def prefill_chunked_8k_d256_fp8(seed: int = 7213) -> Workload:
    """prefill_chunked_8k_d256 with the KV cache stored as OCP fp8 e4m3fn,
    one scale per tensor."""
    rng = np.random.default_rng(np.random.SeedSequence(seed).spawn(7)[6])
    ctx = (rng.integers(0, 8, size=16) * 512).tolist()
    return _prefill_independent("prefill_chunked_8k_d256_fp8", seed, ctx, [512] * 16, 16, 4,
                                256, 16, 8192, kv_dtype="fp8_e4m3fn")


def prefill_prefix_hit(seed: int = 7214) -> Workload:
    """The pages' prefix-cache hit: a 2,000-token system prompt (125 full
    blocks of 16) is cached once and shared by 32 requests; each prefills its
    own 50 new tokens (4 private blocks).  Llama-3-8B shape, fp16."""
    ss = np.random.SeedSequence(seed).spawn(6)
    S, prefix, tail, bs = 32, 2000, 50, 16
    num_blocks = 1024
    free = _FreeList(num_blocks, np.random.default_rng(ss[1]))
    npb = prefix // bs
    pb = free.take(npb)
    ntail = cdiv(prefix + tail, bs) - npb
    max_blocks = npb + ntail
    tables = np.zeros((S, max_blocks), np.int64)
    slots = [_slots_for(pb, prefix, bs)]
    new_idx, own_start = [], np.zeros(S, np.int64)
    pos = prefix
    for s in range(S):
        tables[s, :npb] = pb
        tables[s, npb:] = free.take(ntail)
        slots.append(_slots_for(tables[s], tail, bs, start=prefix))
        own_start[s] = pos
        new_idx.append(np.arange(pos, pos + tail, dtype=np.int64))
        pos += tail
    pad_block = int(free.take(1)[0])
    lens = np.full(S, prefix + tail, np.int64)
    return _finish("prefill_prefix_hit", seed, S, 32, 8, 128, bs, num_blocks, "f16", lens,
                   tables, pad_block, np.concatenate(slots), np.concatenate(new_idx), ss,
                   q_rows=S * tail, q_lens=np.full(S, tail, np.int32), group_size=S,
                   prefix_tokens=prefix, own_from=np.full(S, prefix, np.int64),
                   own_start=own_start, shared_start=np.zeros(S, np.int64))


PREFILL_CONFIGS = {
    "prefill_tiny": prefill_tiny,
    "prefill_cold_2000": prefill_cold_2000,
    "prefill_chunked_8k": prefill_chunked_8k,
    "prefill_prefix_hit": prefill_prefix_hit,
    "prefill_chunked_8k_fp8": prefill_chunked_8k_fp8,
    "prefill_chunked_8k_d256": prefill_chunked_8k_d256,
    "prefill_chunked_8k_d256_fp8": prefill_chunked_8k_d256_fp8,
}


def custom_prefill(name: str, seed: int, ctx_lens, q_lens, Hq: int, Hkv: int, D: int, bs: int,
                   num_blocks: Optional[int] = None, kv_dtype: str = "f16",
                   scale_grain: str = "tensor") -> Workload:
    """Independent prefill sequences (cached lengths + new-token counts)."""
    need = sum(cdiv(int(c) + int(n), bs) for c, n in zip(ctx_lens, q_lens)) + 1
    if num_blocks is None:
        num_blocks = max(need + 7, 2 * need)
    return _prefill_independent(name, seed, list(ctx_lens), list(q_lens), Hq, Hkv, D, bs,
                                int(num_blocks), kv_dtype=kv_dtype, scale_grain=scale_grain)


CONFIGS = {
    "tiny": tiny,
    "llama3_8b_b64": llama3_8b_b64,
    "qwen25_7b_8k": qwen25_7b_8k,
    "prefix_share_bs16": lambda: prefix_share(16),
    "prefix_share_bs8": lambda: prefix_share(8),
    "long_fp8": long_fp8,
    "long_e5m2": long_e5m2,
    "long_fp8_block": long_fp8_block,
    "llama3_8b_b64_w1024": llama3_8b_b64_w1024,
    "hybrid_d256_b64": hybrid_d256_b64,
    "llama3_8b_b64_bs64": lambda: llama3_8b_b64_bs(64),
    "llama3_8b_b64_bs128": lambda: llama3_8b_b64_bs(128),
    "b64_d64": b64_d64,
}


def custom(name: str, seed: int, lens, Hq: int, Hkv: int, D: int, bs: int,
           num_blocks: Optional[int] = None, kv_dtype: str = "f16",
           scale_grain: str = "tensor") -> Workload:
    """Independent sequences of the given lengths (for edge cases and sweeps)."""
    need = sum(cdiv(int(n), bs) for n in lens) + 1
    if num_blocks is None:
        num_blocks = max(need + 7, 2 * need)
    return _independent(name, seed, list(lens), Hq, Hkv, D, bs, int(num_blocks),
                        kv_dtype=kv_dtype, scale_grain=scale_grain)


# --------------------------------------------------------------------------
# structured variants (input construction; the method is untouched)


def with_v_offset(w: Workload, c: float = 1.0) -> Workload:
    """V += c on every token: the output must then sit near c."""
    v = (w.tok_v.astype(np.float32) + np.float32(c)).astype(np.float16)
    out = dataclasses.replace(w, tok_v=v, variant=f"v_offset{c:g}")
    if w.kv_dtype in FP8_DTYPES:
        grain = "head" if w.k_head_scales is not None else "tensor"
        _, out.v_scale, _, out.v_head_scales = fp8_scales(w.kv_dtype, w.tok_k[:1], v, grain)
        if grain == "tensor":
            out.v_scale = float(_amax_f32(v) / fp8_max(w.kv_dtype))
    return out


def needle_positions(w: Workload, s: int, partition: int = 512) -> list:
    """Token positions that get a boosted key: the first and last slot of the
    first block, both sides of a block and a partition boundary, and the last
    valid slot."""
    n = int(w.seq_lens[s])
    bs = w.block_size
    cand = {0, bs - 1, bs, partition - 1, partition, n - 1, (n // 2) // bs * bs}
    return sorted(p for p in cand if 0 <= p < n)


def with_needles(w: Workload, alpha: float = 64.0, seed_offset: int = 0) -> Workload:
    """Plant keys aligned with one query head of the group (k = alpha * q_hat)
    at one seeded position per (sequence, KV head), drawn from
    needle_positions(); those heads then attend almost only to that token."""
    ss = np.random.SeedSequence(w.seed + seed_offset).spawn(6)
    rng = np.random.default_rng(ss[5])
    k = w.tok_k.copy()
    g = w.gqa
    for s in range(w.num_seqs):
        if w.seq_lens[s] == 0:
            continue
        pos = needle_positions(w, s, w.partition_size or 512)
        for kh in range(w.num_kv_heads):
            t = int(pos[rng.integers(len(pos))])
            idx = w.token_index(s, t)
            h = kh * g + int(rng.integers(g))
            qv = w.q[s, h].astype(np.float32)
            qn = qv / np.float32(np.linalg.norm(qv) + 1e-6)
            k[idx, kh] = (np.float32(alpha) * qn).astype(np.float16)
    out = dataclasses.replace(w, tok_k=k, variant="needles")
    if w.kv_dtype in FP8_DTYPES:
        if w.k_head_scales is not None:
            out.k_head_scales = (_amax_per_head_f32(k) / fp8_max(w.kv_dtype)).astype(np.float32)
        else:
            out.k_scale = float(_amax_f32(k) / fp8_max(w.kv_dtype))
    return out


def poison_pool_bits(w: Workload) -> int:
    """Bit pattern every unwritten pool element is filled with in poison runs."""
    if w.kv_dtype == "fp8_e5m2":
        return int(E5M2_NAN_BYTE)
    return int(E4M3_NAN_BYTE) if w.kv_dtype == "fp8_e4m3fn" else int(F16_NAN_BITS)
