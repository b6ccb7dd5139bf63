"""ctypes binding of libpa.so: same entry-point names as include/pa.h.

Argument marshalling only -- every step of the path runs in the library's HIP
kernels.  PyTorch provides device memory and the stream.  Loading fails
loudly if libpa.so has not been built; there is no fallback.

With PA_CHECK_INPUTS=1 in the environment (or CHECK_INPUTS set to True), the
compute calls first run the matching device-argument check of
include/pa_check.h and raise PaError instead of launching on bad tables,
lengths, slots or pairs.  Each check waits for the stream: a debugging aid.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_ALIGNMENT, PA_ERR_WORKSPACE, PA_ERR_HIP = \
    0, -1, -2, -3, -4, -5
PA_ERR_NO_BLOCKS = -6
PA_KV_F16, PA_KV_FP8_E4M3FN, PA_KV_FP8_E5M2 = 0, 1, 2
PLAN_SINGLE, PLAN_FLAT = 0, 1          # pa_decode_plan codes; >= 16 is a split partition size
PA_POOL_SHARED_BLOCKS = 1
_DTYPES = {"f16": PA_KV_F16, "fp8_e4m3fn": PA_KV_FP8_E4M3FN, "fp8_e5m2": PA_KV_FP8_E5M2}

EXPORTS = ("pa_reshape_and_cache", "pa_copy_blocks", "pa_decode_plan",
           "pa_decode_workspace_size", "pa_decode", "pa_decode_grouped", "pa_decode_grouped_plan",
           "pa_decode_grouped_workspace_size", "pa_decode_group_plan",
           "pa_decode_noalloc", "pa_prefill", "pa_prefill_plan", "pa_last_error",
           # host block pool (include/pa_blocks.h)
           "pa_bp_create", "pa_bp_destroy", "pa_bp_last_error", "pa_bp_num_free",
           "pa_bp_ref_count", "pa_bp_block_hash", "pa_bp_free_queue", "pa_bp_get_new_blocks",
           "pa_bp_free_blocks", "pa_bp_touch", "pa_bp_cache_block", "pa_bp_lookup",
           "pa_hash_block_tokens", "pa_bp_allocate_request", "pa_bp_cache_request",
           "pa_bp_append_slots", "pa_bp_free_request", "pa_bp_request_blocks",
           "pa_bp_fork_request", "pa_bp_prepare_write", "pa_bp_remove_skipped_blocks",
           "pa_bp_append_slots_batch", "pa_hash_blocks",
           # device-argument checks (include/pa_check.h)
           "pa_check_scratch_bytes", "pa_check_decode_inputs", "pa_check_prefill_inputs",
           "pa_check_slot_mapping", "pa_check_block_mapping")

CHECK_INPUTS = os.environ.get("PA_CHECK_INPUTS", "") not in ("", "0")


class PaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libpa status {status}: {msg}")
        self.status = status


class pa_kv_pool(C.Structure):
    _fields_ = [
        ("k_base", C.c_void_p), ("v_base", C.c_void_p),
        ("num_blocks", C.c_int64), ("block_stride_bytes", C.c_int64),
        ("block_size", C.c_int32), ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32),
        ("dtype", C.c_int32), ("k_scale", C.c_float), ("v_scale", C.c_float),
        ("flags", C.c_uint32), ("sliding_window", C.c_int32),
        ("k_head_scales", C.c_void_p), ("v_head_scales", C.c_void_p),
        ("k_block_scales", C.c_void_p), ("v_block_scales", C.c_void_p),
    ]


_lib = None


def load() -> C.CDLL:
    """Load libpa.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = C.CDLL(LIB_PATH)
        P, I32, I64, PP = C.c_void_p, C.c_int32, C.c_int64, C.POINTER(pa_kv_pool)
        L.pa_reshape_and_cache.restype = C.c_int
        L.pa_reshape_and_cache.argtypes = [PP, P, P, P, I64, P]
        L.pa_copy_blocks.restype = C.c_int
        L.pa_copy_blocks.argtypes = [PP, P, I64, P]
        L.pa_decode_plan.restype = I32
        L.pa_decode_plan.argtypes = [PP, I32, I32, I32, I32]
        L.pa_decode_workspace_size.restype = C.c_size_t
        L.pa_decode_workspace_size.argtypes = [PP, I32, I32, I32, I32]
        L.pa_decode.restype = C.c_int
        L.pa_decode.argtypes = [PP, P, P, I32, I32, P, I32, P, I32, C.c_float, I32, P, C.c_size_t,
                                P]
        L.pa_decode_grouped.restype = C.c_int
        L.pa_decode_grouped.argtypes = [PP, P, P, I32, I32, P, I32, P, I32, C.c_float, I32, P, P,
                                        P, I32, P, C.c_size_t, P]
        L.pa_decode_grouped_plan.restype = I32
        L.pa_decode_grouped_plan.argtypes = [PP, I32, I32, I32, I32, I32]
        L.pa_decode_grouped_workspace_size.restype = C.c_size_t
        L.pa_decode_grouped_workspace_size.argtypes = [PP, I32, I32, I32, I32, I32]
        L.pa_decode_group_plan.restype = I32
        L.pa_decode_group_plan.argtypes = [P, I32, I32, P, I32, I32, I32, P, P, P]
        L.pa_decode_noalloc.restype = C.c_int
        L.pa_decode_noalloc.argtypes = [PP, P, P, I32, I32, P, I32, P, I32, C.c_float, I32, P]
        L.pa_prefill.restype = C.c_int
        L.pa_prefill.argtypes = [PP, P, P, I32, P, I32, I32, P, I32, P, I32, C.c_float, P]
        L.pa_prefill_plan.restype = I32
        L.pa_prefill_plan.argtypes = [PP, I32, I32, I32]
        L.pa_last_error.restype = C.c_char_p
        L.pa_last_error.argtypes = []
        SZ = C.c_size_t
        L.pa_check_scratch_bytes.restype = SZ
        L.pa_check_scratch_bytes.argtypes = [PP]
        L.pa_check_decode_inputs.restype = C.c_int
        L.pa_check_decode_inputs.argtypes = [PP, I32, P, I32, P, I32, P, SZ, P]
        L.pa_check_prefill_inputs.restype = C.c_int
        L.pa_check_prefill_inputs.argtypes = [PP, I32, P, I32, P, I32, P, I32, P, SZ, P]
        L.pa_check_slot_mapping.restype = C.c_int
        L.pa_check_slot_mapping.argtypes = [PP, P, I64, P, SZ, P]
        L.pa_check_block_mapping.restype = C.c_int
        L.pa_check_block_mapping.argtypes = [PP, P, I64, P, SZ, P]
        _bind_block_pool(L)
        _lib = L
    return _lib


def pa_last_error() -> str:
    return load().pa_last_error().decode()


def _check(status: int) -> None:
    if status != PA_OK:
        raise PaError(status, pa_last_error())


def _stream(stream) -> C.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dev(t: torch.Tensor, dtype, name: str) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


class KVPool:
    """One layer's K and V pools, [num_blocks, block_size, num_kv_heads,
    head_dim] each, in device memory owned by torch."""

    def __init__(self, k: torch.Tensor, v: torch.Tensor, block_size: int, num_kv_heads: int,
                 head_dim: int, kv_dtype: str = "f16", k_scale: float = 1.0,
                 v_scale: float = 1.0, num_blocks: Optional[int] = None,
                 block_stride_bytes: int = 0, shared_blocks: bool = False,
                 k_head_scales: Optional[torch.Tensor] = None,
                 v_head_scales: Optional[torch.Tensor] = None, sliding_window: int = 0,
                 k_block_scales: Optional[torch.Tensor] = None,
                 v_block_scales: Optional[torch.Tensor] = None):
        """k_head_scales / v_head_scales: optional device float32 [num_kv_heads]
        fp8 scales, one per KV head (replacing k_scale / v_scale).
        k_block_scales / v_block_scales: optional device float32 [num_blocks,
        num_kv_heads] fp8 scales per (block, KV head), which the library
        writes as it writes the blocks."""
        self.k, self.v = k, v
        self.k_head_scales, self.v_head_scales = k_head_scales, v_head_scales
        self.k_block_scales, self.v_block_scales = k_block_scales, v_block_scales
        khp = _dev(k_head_scales, torch.float32, "k_head_scales") if k_head_scales is not None \
            else None
        vhp = _dev(v_head_scales, torch.float32, "v_head_scales") if v_head_scales is not None \
            else None
        kbp = _dev(k_block_scales, torch.float32, "k_block_scales") \
            if k_block_scales is not None else None
        vbp = _dev(v_block_scales, torch.float32, "v_block_scales") \
            if v_block_scales is not None else None
        self.block_size, self.num_kv_heads, self.head_dim = block_size, num_kv_heads, head_dim
        self.kv_dtype = kv_dtype
        self.k_scale, self.v_scale = float(k_scale), float(v_scale)
        self.num_blocks = int(num_blocks if num_blocks is not None else k.shape[0])
        self.block_stride_bytes = int(block_stride_bytes)
        self.desc = pa_kv_pool(k.data_ptr(), v.data_ptr(), self.num_blocks,
                               self.block_stride_bytes, block_size, num_kv_heads, head_dim,
                               _DTYPES[kv_dtype], self.k_scale, self.v_scale,
                               PA_POOL_SHARED_BLOCKS if shared_blocks else 0,
                               int(sliding_window), khp, vhp, kbp, vbp)

    @property
    def shared_blocks(self) -> bool:
        """Blocks may be read by several sequences of a batch (cacheable K/V reads)."""
        return bool(self.desc.flags & PA_POOL_SHARED_BLOCKS)

    @shared_blocks.setter
    def shared_blocks(self, on: bool) -> None:
        self.desc.flags = PA_POOL_SHARED_BLOCKS if on else 0

    @classmethod
    def allocate(cls, num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int,
                 kv_dtype: str = "f16", k_scale: float = 1.0, v_scale: float = 1.0,
                 device="cuda", fill_bits: Optional[int] = None,
                 shared_blocks: bool = False, k_head_scales=None,
                 v_head_scales=None, sliding_window: int = 0,
                 block_scales: bool = False) -> "KVPool":
        """block_scales: keep one fp8 scale per (block, KV head) beside the
        pools (zero-filled device arrays the library then writes)."""
        tdt = torch.int16 if kv_dtype == "f16" else torch.uint8
        shape = (num_blocks, block_size, num_kv_heads, head_dim)
        k = torch.empty(shape, dtype=tdt, device=device)
        v = torch.empty(shape, dtype=tdt, device=device)
        if fill_bits is not None:
            fb = fill_bits if kv_dtype != "f16" else (fill_bits - 65536 if fill_bits >= 32768
                                                            else fill_bits)
            k.fill_(fb)
            v.fill_(fb)
        khs = vhs = None
        if k_head_scales is not None:
            khs = torch.as_tensor(k_head_scales, dtype=torch.float32).to(device).contiguous()
            vhs = torch.as_tensor(v_head_scales, dtype=torch.float32).to(device).contiguous()
        kbs = vbs = None
        if block_scales:
            kbs = torch.zeros((num_blocks, num_kv_heads), dtype=torch.float32, device=device)
            vbs = torch.zeros((num_blocks, num_kv_heads), dtype=torch.float32, device=device)
        return cls(k, v, block_size, num_kv_heads, head_dim, kv_dtype, k_scale, v_scale,
                   shared_blocks=shared_blocks, k_head_scales=khs, v_head_scales=vhs,
                   sliding_window=sliding_window, k_block_scales=kbs, v_block_scales=vbs)

    @property
    def elem_bytes(self) -> int:
        return 2 if self.kv_dtype == "f16" else 1


def pa_reshape_and_cache(pool: KVPool, k_new: torch.Tensor, v_new: torch.Tensor,
                         slot_mapping: torch.Tensor, stream=None) -> None:
    T = int(slot_mapping.numel())
    if k_new.shape != (T, pool.num_kv_heads, pool.head_dim) or v_new.shape != k_new.shape:
        raise ValueError("k_new/v_new must be [num_tokens, num_kv_heads, head_dim]")
    if CHECK_INPUTS:
        pa_check_slot_mapping(pool, slot_mapping, stream)
    _check(load().pa_reshape_and_cache(
        C.byref(pool.desc), _dev(k_new, torch.float16, "k_new"),
        _dev(v_new, torch.float16, "v_new"), _dev(slot_mapping, torch.int64, "slot_mapping"),
        T, _stream(stream)))


def pa_copy_blocks(pool: KVPool, block_mapping: torch.Tensor, stream=None) -> None:
    if block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be [num_pairs, 2]")
    if CHECK_INPUTS:
        pa_check_block_mapping(pool, block_mapping, stream)
    _check(load().pa_copy_blocks(C.byref(pool.desc),
                                 _dev(block_mapping, torch.int64, "block_mapping"),
                                 int(block_mapping.shape[0]), _stream(stream)))


def pa_decode_plan(pool: KVPool, num_seqs: int, num_q_heads: int, max_seq_len: int,
                   partition_size: int = 0) -> int:
    r = load().pa_decode_plan(C.byref(pool.desc), num_seqs, num_q_heads, max_seq_len,
                              partition_size)
    if r < 0:
        raise PaError(r, pa_last_error())
    return int(r)


def pa_decode_workspace_size(pool: KVPool, num_seqs: int, num_q_heads: int, max_seq_len: int,
                             partition_size: int = 0) -> int:
    return int(load().pa_decode_workspace_size(C.byref(pool.desc), num_seqs, num_q_heads,
                                               max_seq_len, partition_size))


def alloc_workspace(pool: KVPool, num_seqs: int, num_q_heads: int, max_seq_len: int,
                    partition_size: int = 0, device="cuda") -> Optional[torch.Tensor]:
    """Workspace for pa_decode.  Within one call the kernels read only words
    that the same call wrote (the flat schedule's merge skips ranges that own
    no unit; the split reduce reads only partitions inside the context and the
    window), so its contents between calls do not matter and one workspace may
    be reused by consecutive calls on a stream.  It is zero-filled only so
    that dumps of unused parts are tidy."""
    n = pa_decode_workspace_size(pool, num_seqs, num_q_heads, max_seq_len, partition_size)
    return torch.zeros(n, dtype=torch.uint8, device=device) if n else None


def pa_decode(pool: KVPool, out: torch.Tensor, q: torch.Tensor, block_tables: torch.Tensor,
              seq_lens: torch.Tensor, max_seq_len: int, scale: float, partition_size: int = 0,
              workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    S, Hq, D = q.shape
    if out.shape != q.shape:
        raise ValueError("out must have q's shape [num_seqs, num_q_heads, head_dim]")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or seq_lens.shape != (S,):
        raise ValueError("block_tables must be [num_seqs, max_blocks], seq_lens [num_seqs]")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = _dev(workspace, workspace.dtype, "workspace"), workspace.numel() * \
            workspace.element_size()
    if CHECK_INPUTS:
        pa_check_decode_inputs(pool, block_tables, seq_lens, max_seq_len, stream)
    _check(load().pa_decode(
        C.byref(pool.desc), _dev(out, torch.float16, "out"), _dev(q, torch.float16, "q"), S, Hq,
        _dev(block_tables, torch.int32, "block_tables"), int(block_tables.shape[1]),
        _dev(seq_lens, torch.int32, "seq_lens"), int(max_seq_len), C.c_float(scale),
        int(partition_size), ws_ptr, ws_bytes, _stream(stream)))


class DecodeGroups:
    """A grouping of a decode batch for pa_decode_grouped: host arrays from
    pa_decode_group_plan and their device copies."""

    def __init__(self, members: np.ndarray, member_start: np.ndarray,
                 member_shared: np.ndarray, device="cuda"):
        self.members, self.member_start, self.member_shared = members, member_start, member_shared
        self.num_groups = int(member_start.size) - 1
        self.d_members = torch.from_numpy(members).to(device)
        self.d_member_start = torch.from_numpy(member_start).to(device)
        self.d_member_shared = torch.from_numpy(member_shared).to(device)


def pa_decode_group_plan(block_tables: np.ndarray, seq_lens: np.ndarray, block_size: int,
                         num_q_heads: int, num_kv_heads: int, device="cuda") -> DecodeGroups:
    """Group sequences that list the same leading physical blocks (host
    arrays in, a DecodeGroups with device copies out)."""
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    S = int(lens.size)
    members = np.zeros(max(1, S), np.int32)
    start = np.zeros(S + 1, np.int32)
    shared = np.zeros(max(1, S), np.int32)
    p = lambda a: a.ctypes.data_as(C.c_void_p)
    n = load().pa_decode_group_plan(p(bt), S, int(bt.shape[1]), p(lens), int(block_size),
                                    int(num_q_heads), int(num_kv_heads), p(members), p(start),
                                    p(shared))
    if n < 0:
        raise PaError(n, pa_last_error())
    return DecodeGroups(members[:S].copy(), start[:n + 1].copy(), shared[:S].copy(), device)


GROUPED_FLAT, GROUPED_PER_GROUP = 1, 2      # pa_decode_grouped schedules


def pa_decode_grouped_plan(pool: KVPool, num_seqs: int, num_q_heads: int, max_seq_len: int,
                           num_groups: int, schedule: int = 0) -> int:
    r = load().pa_decode_grouped_plan(C.byref(pool.desc), num_seqs, num_q_heads, max_seq_len,
                                      num_groups, schedule)
    if r < 0:
        raise PaError(r, pa_last_error())
    return int(r)


def alloc_grouped_workspace(pool: KVPool, num_seqs: int, num_q_heads: int, max_seq_len: int,
                            num_groups: int, schedule: int = 0,
                            device="cuda") -> Optional[torch.Tensor]:
    n = int(load().pa_decode_grouped_workspace_size(C.byref(pool.desc), num_seqs, num_q_heads,
                                                    max_seq_len, num_groups, schedule))
    return torch.zeros(n, dtype=torch.uint8, device=device) if n else None


def pa_decode_grouped(pool: KVPool, out: torch.Tensor, q: torch.Tensor,
                      block_tables: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                      scale: float, groups: DecodeGroups, schedule: int = 0,
                      workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """pa_decode with the batch's shared prefixes read once per group; the
    workspace (flat grouped schedule) is allocated here when not given."""
    S, Hq, D = q.shape
    if out.shape != q.shape:
        raise ValueError("out must have q's shape [num_seqs, num_q_heads, head_dim]")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or seq_lens.shape != (S,):
        raise ValueError("block_tables must be [num_seqs, max_blocks], seq_lens [num_seqs]")
    if groups.members.size != S:
        raise ValueError("the grouping must list every sequence once")
    if CHECK_INPUTS:
        pa_check_decode_inputs(pool, block_tables, seq_lens, max_seq_len, stream)
    if workspace is None:
        workspace = alloc_grouped_workspace(pool, S, Hq, max_seq_len, groups.num_groups,
                                            schedule, device=q.device)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = _dev(workspace, workspace.dtype, "workspace"), workspace.numel() * \
            workspace.element_size()
    _check(load().pa_decode_grouped(
        C.byref(pool.desc), _dev(out, torch.float16, "out"), _dev(q, torch.float16, "q"), S, Hq,
        _dev(block_tables, torch.int32, "block_tables"), int(block_tables.shape[1]),
        _dev(seq_lens, torch.int32, "seq_lens"), int(max_seq_len), C.c_float(scale),
        groups.num_groups, _dev(groups.d_members, torch.int32, "members"),
        _dev(groups.d_member_start, torch.int32, "member_start"),
        _dev(groups.d_member_shared, torch.int32, "member_shared"), int(schedule), ws_ptr,
        ws_bytes, _stream(stream)))


PA_DECODE_NOALLOC_SCRATCH_BYTES = 64 << 20


def pa_decode_noalloc(pool: KVPool, out: torch.Tensor, q: torch.Tensor,
                      block_tables: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                      scale: float, partition_size: int = 0, stream=None) -> None:
    """pa_decode without a workspace argument: the library's per-device
    scratch (PA_DECODE_NOALLOC_SCRATCH_BYTES) serves the flat and split
    schedules.  For callers that cannot allocate; overlapping calls on one
    GPU race on the scratch."""
    S, Hq, D = q.shape
    if out.shape != q.shape:
        raise ValueError("out must have q's shape [num_seqs, num_q_heads, head_dim]")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or seq_lens.shape != (S,):
        raise ValueError("block_tables must be [num_seqs, max_blocks], seq_lens [num_seqs]")
    if CHECK_INPUTS:
        pa_check_decode_inputs(pool, block_tables, seq_lens, max_seq_len, stream)
    _check(load().pa_decode_noalloc(
        C.byref(pool.desc), _dev(out, torch.float16, "out"), _dev(q, torch.float16, "q"), S, Hq,
        _dev(block_tables, torch.int32, "block_tables"), int(block_tables.shape[1]),
        _dev(seq_lens, torch.int32, "seq_lens"), int(max_seq_len), C.c_float(scale),
        int(partition_size), _stream(stream)))


def pa_prefill_plan(pool: KVPool, num_seqs: int, num_q_heads: int, max_q_len: int) -> int:
    """Query rows per workgroup pa_prefill will use (128 or 192)."""
    r = load().pa_prefill_plan(C.byref(pool.desc), num_seqs, num_q_heads, max_q_len)
    if r < 0:
        raise PaError(r, pa_last_error())
    return int(r)


def pa_prefill(pool: KVPool, out: torch.Tensor, q: torch.Tensor, q_start: torch.Tensor,
               block_tables: torch.Tensor, seq_lens: torch.Tensor, max_q_len: int, scale: float,
               stream=None) -> None:
    """Causal attention of each sequence's new tokens (q rows q_start[s] ..
    q_start[s+1] - 1, the last positions of its seq_lens[s]) over its paged
    context; their K/V must already be in the pool."""
    T, Hq, D = q.shape
    S = int(seq_lens.shape[0])
    if out.shape != q.shape:
        raise ValueError("out must have q's shape [total_q, num_q_heads, head_dim]")
    if q_start.shape != (S + 1,) or block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("q_start must be [num_seqs + 1], block_tables [num_seqs, max_blocks]")
    if CHECK_INPUTS:
        pa_check_prefill_inputs(pool, q_start, block_tables, seq_lens, T, max_q_len, stream)
    _check(load().pa_prefill(
        C.byref(pool.desc), _dev(out, torch.float16, "out"), _dev(q, torch.float16, "q"), T,
        _dev(q_start, torch.int32, "q_start"), S, Hq,
        _dev(block_tables, torch.int32, "block_tables"), int(block_tables.shape[1]),
        _dev(seq_lens, torch.int32, "seq_lens"), int(max_q_len), C.c_float(scale),
        _stream(stream)))


# ---------------------------------------------------------------------------
# device-argument checks (include/pa_check.h)

def pa_check_scratch_bytes(pool: KVPool) -> int:
    return int(load().pa_check_scratch_bytes(C.byref(pool.desc)))


def _scratch(pool: KVPool):
    """The pool's check scratch (allocated on first use, kept with the pool)."""
    n = pa_check_scratch_bytes(pool)
    t = getattr(pool, "_check_scratch", None)
    if t is None or t.numel() < n:
        t = torch.empty(max(n, 256), dtype=torch.uint8, device=pool.k.device)
        pool._check_scratch = t
    return t.data_ptr(), t.numel()


def pa_check_decode_inputs(pool: KVPool, block_tables: torch.Tensor, seq_lens: torch.Tensor,
                           max_seq_len: int, stream=None) -> None:
    S = int(seq_lens.shape[0])
    sp, sn = _scratch(pool)
    _check(load().pa_check_decode_inputs(
        C.byref(pool.desc), S, _dev(block_tables, torch.int32, "block_tables"),
        int(block_tables.shape[1]), _dev(seq_lens, torch.int32, "seq_lens"), int(max_seq_len),
        sp, sn, _stream(stream)))


def pa_check_prefill_inputs(pool: KVPool, q_start: torch.Tensor, block_tables: torch.Tensor,
                            seq_lens: torch.Tensor, total_q: int, max_q_len: int,
                            stream=None) -> None:
    S = int(seq_lens.shape[0])
    sp, sn = _scratch(pool)
    _check(load().pa_check_prefill_inputs(
        C.byref(pool.desc), int(total_q), _dev(q_start, torch.int32, "q_start"), S,
        _dev(block_tables, torch.int32, "block_tables"), int(block_tables.shape[1]),
        _dev(seq_lens, torch.int32, "seq_lens"), int(max_q_len), sp, sn, _stream(stream)))


def pa_check_slot_mapping(pool: KVPool, slot_mapping: torch.Tensor, stream=None) -> None:
    sp, sn = _scratch(pool)
    _check(load().pa_check_slot_mapping(
        C.byref(pool.desc), _dev(slot_mapping, torch.int64, "slot_mapping"),
        int(slot_mapping.numel()), sp, sn, _stream(stream)))


def pa_check_block_mapping(pool: KVPool, block_mapping: torch.Tensor, stream=None) -> None:
    sp, sn = _scratch(pool)
    _check(load().pa_check_block_mapping(
        C.byref(pool.desc), _dev(block_mapping, torch.int64, "block_mapping"),
        int(block_mapping.shape[0]), sp, sn, _stream(stream)))


# ---------------------------------------------------------------------------
# host block pool with prefix caching (include/pa_blocks.h)


class pa_block_hash(C.Structure):
    _fields_ = [("bytes", C.c_uint8 * 32)]


def _bind_block_pool(L) -> None:
    P, I32, I64 = C.c_void_p, C.c_int32, C.c_int64
    H = C.POINTER(pa_block_hash)
    IP, LP = C.POINTER(C.c_int32), C.POINTER(C.c_int64)
    sig = {
        "pa_bp_create": (P, [I32, I32]),
        "pa_bp_destroy": (None, [P]),
        "pa_bp_last_error": (C.c_char_p, []),
        "pa_bp_num_free": (I32, [P]),
        "pa_bp_ref_count": (I32, [P, I32]),
        "pa_bp_block_hash": (C.c_int, [P, I32, H]),
        "pa_bp_free_queue": (I32, [P, IP, I32]),
        "pa_bp_get_new_blocks": (C.c_int, [P, I32, IP]),
        "pa_bp_free_blocks": (C.c_int, [P, IP, I32]),
        "pa_bp_touch": (C.c_int, [P, IP, I32]),
        "pa_bp_cache_block": (C.c_int, [P, I32, H]),
        "pa_bp_lookup": (I32, [P, H, I32, IP]),
        "pa_hash_block_tokens": (None, [H, IP, I32, P, I32, H]),
        "pa_bp_allocate_request": (C.c_int, [P, I64, IP, I32, P, I32, IP]),
        "pa_bp_cache_request": (C.c_int, [P, I64, IP, I32, P, I32]),
        "pa_bp_append_slots": (C.c_int, [P, I64, I32]),
        "pa_bp_free_request": (C.c_int, [P, I64]),
        "pa_bp_request_blocks": (I32, [P, I64, IP, I32]),
        "pa_bp_fork_request": (C.c_int, [P, I64, I64]),
        "pa_bp_prepare_write": (C.c_int, [P, I64, I32, LP]),
        "pa_bp_remove_skipped_blocks": (I32, [P, I64, I32, I32]),
        "pa_bp_append_slots_batch": (C.c_int, [P, LP, IP, I32]),
        "pa_hash_blocks": (I32, [IP, I32, I32, P, I32, H, I32]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args


def _ints(xs):
    """int32 array argument: a contiguous int32 numpy array is passed in place,
    anything else is copied into a new ctypes array."""
    if isinstance(xs, np.ndarray) and xs.dtype == np.int32 and xs.flags.c_contiguous and xs.size:
        return xs.ctypes.data_as(C.POINTER(C.c_int32))
    xs = [int(x) for x in xs]
    return (C.c_int32 * max(1, len(xs)))(*xs)


def _hash_arr(hs) -> C.Array:
    arr = (pa_block_hash * max(1, len(hs)))()
    for i, h in enumerate(hs):
        C.memmove(arr[i].bytes, bytes(h), 32)
    return arr


def hash_block_tokens(parent: Optional[bytes], tokens, extra: bytes = b"") -> bytes:
    """SHA-256(parent or 32 zero bytes | token ids as int32 LE | extra)."""
    L = load()
    out = pa_block_hash()
    par = None
    if parent is not None:
        par = pa_block_hash()
        C.memmove(par.bytes, bytes(parent), 32)
    toks = _ints(tokens)
    ex = C.create_string_buffer(bytes(extra), max(1, len(extra)))
    L.pa_hash_block_tokens(C.byref(par) if par is not None else None, toks, len(tokens),
                           ex if extra else None, len(extra), C.byref(out))
    return bytes(out.bytes)


def hash_blocks(tokens, block_size: int, extra: bytes = b"") -> list:
    """Chained hashes of the full blocks of a token sequence (one native call)."""
    L = load()
    n = len(tokens) // int(block_size)
    out = (pa_block_hash * max(1, n))()
    ex = C.create_string_buffer(bytes(extra), max(1, len(extra)))
    r = L.pa_hash_blocks(_ints(tokens), len(tokens), int(block_size), ex if extra else None,
                         len(extra), out, n)
    if r < 0:
        raise PaError(r, L.pa_bp_last_error().decode())
    return [bytes(out[i].bytes) for i in range(n)]


class BlockPool:
    """The native host block pool (reference counts, LRU free queue shared
    with the prefix cache, chained block hashes, fork and copy-on-write)."""

    def __init__(self, num_blocks: int, block_size: int):
        self._L = load()
        self._p = self._L.pa_bp_create(int(num_blocks), int(block_size))
        if not self._p:
            raise PaError(PA_ERR_INVALID_ARG, self._L.pa_bp_last_error().decode())
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)

    def __del__(self):
        if getattr(self, "_p", None):
            self._L.pa_bp_destroy(self._p)
            self._p = None

    def _ok(self, st: int) -> int:
        if st < 0:
            raise PaError(st, self._L.pa_bp_last_error().decode())
        return st

    def num_free(self) -> int:
        return self._L.pa_bp_num_free(self._p)

    def ref_count(self, b: int) -> int:
        return self._ok(self._L.pa_bp_ref_count(self._p, int(b)))

    def block_hash(self, b: int) -> Optional[bytes]:
        h = pa_block_hash()
        return bytes(h.bytes) if self._ok(self._L.pa_bp_block_hash(self._p, int(b), C.byref(h))) else None

    def free_queue(self) -> list:
        n = self._ok(self._L.pa_bp_free_queue(self._p, None, 0))
        out = (C.c_int32 * max(1, n))()
        self._ok(self._L.pa_bp_free_queue(self._p, out, n))
        return list(out[:n])

    def get_new_blocks(self, n: int) -> list:
        out = (C.c_int32 * max(1, n))()
        self._ok(self._L.pa_bp_get_new_blocks(self._p, int(n), out))
        return list(out[:n])

    def free_blocks(self, ids) -> None:
        self._ok(self._L.pa_bp_free_blocks(self._p, _ints(ids), len(ids)))

    def touch(self, ids) -> None:
        self._ok(self._L.pa_bp_touch(self._p, _ints(ids), len(ids)))

    def cache_block(self, b: int, h: bytes) -> None:
        hh = pa_block_hash()
        C.memmove(hh.bytes, bytes(h), 32)
        self._ok(self._L.pa_bp_cache_block(self._p, int(b), C.byref(hh)))

    def lookup(self, hashes) -> list:
        out = (C.c_int32 * max(1, len(hashes)))()
        n = self._ok(self._L.pa_bp_lookup(self._p, _hash_arr(hashes), len(hashes), out))
        return list(out[:n])

    def allocate_request(self, rid: int, tokens, extra: bytes = b"") -> int:
        cached = C.c_int32(0)
        ex = C.create_string_buffer(bytes(extra), max(1, len(extra)))
        self._ok(self._L.pa_bp_allocate_request(self._p, int(rid), _ints(tokens), len(tokens),
                                                ex if extra else None, len(extra),
                                                C.byref(cached)))
        return cached.value

    def cache_request(self, rid: int, tokens, extra: bytes = b"") -> None:
        ex = C.create_string_buffer(bytes(extra), max(1, len(extra)))
        self._ok(self._L.pa_bp_cache_request(self._p, int(rid), _ints(tokens), len(tokens),
                                             ex if extra else None, len(extra)))

    def append_slots(self, rid: int, num_tokens_after: int) -> None:
        self._ok(self._L.pa_bp_append_slots(self._p, int(rid), int(num_tokens_after)))

    def append_slots_batch(self, rids, num_tokens_after) -> None:
        """One scheduler step: each listed request grows to its token count
        (all or nothing)."""
        n = len(rids)
        ids = (C.c_int64 * max(1, n))(*[int(r) for r in rids])
        self._ok(self._L.pa_bp_append_slots_batch(self._p, ids, _ints(num_tokens_after), n))

    def free_request(self, rid: int) -> None:
        self._ok(self._L.pa_bp_free_request(self._p, int(rid)))

    def request_blocks(self, rid: int) -> list:
        n = self._ok(self._L.pa_bp_request_blocks(self._p, int(rid), None, 0))
        out = (C.c_int32 * max(1, n))()
        self._L.pa_bp_request_blocks(self._p, int(rid), out, n)
        return list(out[:n])

    def fork_request(self, parent: int, child: int) -> None:
        self._ok(self._L.pa_bp_fork_request(self._p, int(parent), int(child)))

    def remove_skipped_blocks(self, rid: int, num_tokens: int, window: int) -> int:
        """Release the request's blocks that lie wholly before the sliding
        window of its next query; returns how many were released."""
        return self._ok(self._L.pa_bp_remove_skipped_blocks(self._p, int(rid), int(num_tokens),
                                                            int(window)))

    def prepare_write(self, rid: int, position: int) -> Optional[tuple]:
        """(src, dst) for pa_copy_blocks when the block is shared, else None."""
        pair = (C.c_int64 * 2)()
        r = self._ok(self._L.pa_bp_prepare_write(self._p, int(rid), int(position), pair))
        return (pair[0], pair[1]) if r == 1 else None
