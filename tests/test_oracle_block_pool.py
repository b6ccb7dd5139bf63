"""Pins for the oracle's block-pool model (CPU only).

The model is checked against what the pages print: the six-block free-queue
walkthrough T0-T4 ("KV Cache memory core", section 2.3, stored in
tests/golden/block_pool_walkthrough.json), the chained-hash examples (two
prompts diverging in block 2 share blocks 0 and 1; a different first token
shares nothing: "vLLM intro part 2", section 6.1; "KV Cache memory core",
section 4.1), the 2,000-token system prompt that is 125 full blocks and the
second request that prefills only its own 50 tokens, and the self-test's 2,005
tokens whose last 5 are recomputed ("KV Cache memory core", sections 4.1 and
6, question 3).  The hash itself is SHA-256 from hashlib over the documented
byte layout, checked against a hand-assembled input.
"""
import hashlib
import json
import os
import struct

import numpy as np
import pytest

from oracle.block_pool import (NONE_HASH, BlockPoolModel, PoolError, prompt_digests,
                               block_digest)

GOLD = os.path.join(os.path.dirname(__file__), "golden", "block_pool_walkthrough.json")


def _tokens(n, seed):
    return [int(x) for x in np.random.default_rng(seed).integers(0, 128000, size=n)]


def run_walkthrough(pool_factory):
    """Replay the pages' walkthrough on a pool object with the model's API and
    return the observed states, one per step."""
    g = json.load(open(GOLD))
    bs = g["block_size"]
    pool = pool_factory(g["num_blocks"], bs)
    a_tokens = _tokens(2 * bs + 8, 1)           # blocks 0 and 1 full, block 2 partial
    seen = []
    held = {}
    for st in g["steps"]:
        op = st["op"]
        if op == "get_new_blocks":
            held[st["who"]] = pool.get_new_blocks(st["n"])
            seen.append({"got": held[st["who"]]})
        elif op == "finish":
            hs = prompt_digests(a_tokens, bs)
            for b, h in zip(held["A"], hs):
                pool.cache_full_block(b, h)
            pool.free_blocks(list(reversed(held.pop("A"))))
            seen.append({})
        elif op == "prefix_lookup":
            hits = pool.lookup(prompt_digests(a_tokens, bs))
            pool.touch(hits)
            seen.append({"hits": hits})
        else:
            seen.append({})
        seen[-1]["free"] = pool.free_queue_list()
        seen[-1]["hashed"] = pool.hashed_list()
    return g, pool, seen


class _Model(BlockPoolModel):
    def free_queue_list(self):
        return list(self.queue)

    def hashed_list(self):
        return sorted(b for b, h in enumerate(self.kept) if h is not None)


def test_walkthrough_t0_to_t4():
    g, pool, seen = run_walkthrough(_Model)
    for st, obs in zip(g["steps"], seen):
        assert obs["free"] == st["free"], st["t"]
        assert obs["hashed"] == st["hashed"], st["t"]
        if "got" in st:
            assert obs["got"] == st["got"], st["t"]
        if "hits" in st:
            assert obs["hits"] == st["hits"], st["t"]
    assert pool.count[0] == 1
    with pytest.raises(PoolError):
        pool.get_new_blocks(1)               # B's second block: the queue is empty


def test_hash_byte_layout():
    toks = [1, -2, 70000, 5]
    expect = hashlib.sha256(bytes(32) + b"\x01\x00\x00\x00" + b"\xfe\xff\xff\xff" +
                            b"\x70\x11\x01\x00" + b"\x05\x00\x00\x00" + b"lora7").digest()
    assert block_digest(None, toks, b"lora7") == expect
    assert NONE_HASH == bytes(32)
    h0 = block_digest(None, toks)
    assert block_digest(h0, toks) == hashlib.sha256(h0 + b"".join(
        struct.pack("<i", t) for t in toks)).digest()


def test_chain_divergence_and_first_token():
    bs = 16
    sys_prompt = _tokens(2 * bs + 5, 2)
    r1 = sys_prompt + _tokens(20, 3)
    r2 = sys_prompt + _tokens(20, 4)
    h1, h2 = prompt_digests(r1, bs), prompt_digests(r2, bs)
    assert h1[:2] == h2[:2] and h1[2] != h2[2]
    r3 = [r1[0] + 1] + r1[1:]
    h3 = prompt_digests(r3, bs)
    assert all(a != b for a, b in zip(h1, h3))          # nothing shared after a changed head
    assert prompt_digests(r1, bs, b"tenant-1")[0] != h1[0]  # extra keys separate tenants


def test_prefix_hit_2000_token_prompt():
    bs = 16
    sys_prompt = _tokens(2000, 5)
    pool = BlockPoolModel(400, bs)
    a = sys_prompt + _tokens(2, 6)                       # "Hi"
    assert pool.allocate_request(1, a) == 0
    pool.cache_request(1, a)
    assert len([h for h in pool.kept if h is not None]) == 125      # 125 full blocks
    b = sys_prompt + _tokens(50, 7)
    assert pool.allocate_request(2, b) == 2000           # 125 blocks hit
    shared = pool.requests[1][:125]
    assert pool.requests[2][:125] == shared
    assert all(pool.count[x] == 2 for x in shared)
    assert len(pool.requests[2]) == -(-2050 // bs)       # 129 blocks, 4 of them new
    # self-test: 2,005 tokens -> 125 blocks hit, the last 5 tokens recomputed
    c = sys_prompt + _tokens(5, 8)
    assert pool.allocate_request(3, c) == 2000
    # a prompt that is exactly the cached 125 blocks still computes its last token
    d = list(sys_prompt)
    assert pool.allocate_request(4, d) == 124 * bs


def test_free_keeps_hashes_and_prefix_blocks_leave_last():
    bs = 4
    pool = BlockPoolModel(8, bs)
    t = _tokens(3 * bs, 9)
    pool.allocate_request(1, t)
    pool.cache_request(1, t)
    blocks = list(pool.requests[1])
    pool.free_request(1)
    # freed last to first: the prefix block ends nearest the tail (evicted last)
    assert pool.queue[-3:] == list(reversed(blocks))
    assert all(pool.kept[b] is not None for b in blocks)
    # shared block is released only when its last holder frees it
    pool.allocate_request(2, t)
    pool.allocate_request(3, t[:2 * bs] + [1, 2, 3, 4])
    first = pool.requests[2][0]
    assert pool.count[first] == 2
    pool.free_request(2)
    assert pool.count[first] == 1 and first not in pool.queue


def test_failed_allocation_changes_nothing():
    pool = BlockPoolModel(4, 4)
    pool.allocate_request(1, _tokens(9, 10))             # 3 blocks
    before = pool.state()
    with pytest.raises(PoolError):
        pool.allocate_request(2, _tokens(9, 11))
    assert pool.state() == before
