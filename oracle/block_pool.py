"""Plain model of the host block pool with prefix caching.

TEST INFRASTRUCTURE ONLY: the tests compare the native pool in libpa.so with
this model; nothing in the library imports it.  Lists and dicts, O(n)
operations, written from the pages' rules so that a reader can check each step
against them:

  * every block whose reference count is 0 sits in ONE free queue, whether it
    was never used or still carries the hash of a cached block; the head is
    handed out first ("KV Cache memory core", section 2.3, BlockPool sketch
    and the six-block walkthrough T0-T4);
  * handing a block out that still carries a hash removes that hash from the
    cache index -- that is the eviction (same passage; "vLLM intro part 2",
    section 6.3 step 3);
  * freeing drops the count; a block reaching 0 goes to the TAIL if it carries
    a hash (kept for future hits as long as possible) and to the HEAD if not
    (handed out first) ("KV Cache memory core", section 2.3 free_blocks notes
    and walkthrough T2); a request frees its blocks from last to first
    ("vLLM intro part 2", section 6.3 free steps);
  * a prefix hit on a block with count 0 takes it out of the middle of the
    queue and raises its count ("touch"; same passages, walkthrough T4);
  * block hashes are chained: h_i = H(h_{i-1}, the block's tokens, extra keys),
    with a fixed NONE_HASH before the first block; only full blocks get a
    hash; lookup walks the chain from the first block and stops at the first
    miss ("vLLM intro part 2", section 6.1; "KV Cache memory core", section
    4.1 chained-hash diagram);
  * H is SHA-256 ("vLLM intro part 2", section 6.1: the default since 0.11).

Readings where the pages leave a step open (each also listed in the design
notes): NONE_HASH is 32 zero bytes; H hashes the parent's 32 bytes, then the
block's token ids as little-endian int32, then the extra-key bytes; several
unhashed blocks freed in one call are prepended one after another (so the
last one freed ends at the head); a request's lookup never covers its last
token (at least one token is computed), so at most (n - 1) // block_size
blocks hit; when several blocks carry the same hash a lookup takes the one
cached first.
"""
from __future__ import annotations

import hashlib
import struct
from typing import Dict, List, Optional, Sequence

NONE_HASH = bytes(32)


def hash_block_tokens(parent: Optional[bytes], tokens: Sequence[int],
                      extra: bytes = b"") -> bytes:
    """h = SHA-256(parent hash | token ids as int32 LE | extra keys)."""
    p = NONE_HASH if parent is None else parent
    body = b"".join(struct.pack("<i", int(t)) for t in tokens)
    return hashlib.sha256(p + body + extra).digest()


def chain_hashes(tokens: Sequence[int], block_size: int, extra: bytes = b"") -> List[bytes]:
    """Hashes of the full blocks of a token sequence, chained from NONE_HASH."""
    out, parent = [], None
    for i in range(len(tokens) // block_size):
        parent = hash_block_tokens(parent, tokens[i * block_size:(i + 1) * block_size], extra)
        out.append(parent)
    return out


class PoolError(Exception):
    pass


class BlockPoolModel:
    def __init__(self, num_blocks: int, block_size: int):
        self.block_size = block_size
        self.ref = [0] * num_blocks
        self.hash: List[Optional[bytes]] = [None] * num_blocks
        self.free: List[int] = list(range(num_blocks))          # head = index 0
        self.index: Dict[bytes, List[int]] = {}                   # hash -> ids, first cached first
        self.requests: Dict[int, List[int]] = {}

    # ---------------------------------------------------------------- pool
    def num_free(self) -> int:
        return len(self.free)

    def get_new_blocks(self, n: int) -> List[int]:
        if n > len(self.free):
            raise PoolError("not enough free blocks")
        out = self.free[:n]
        del self.free[:n]
        for b in out:
            h = self.hash[b]
            if h is not None:                       # eviction
                self.index[h].remove(b)
                if not self.index[h]:
                    del self.index[h]
                self.hash[b] = None
            self.ref[b] += 1
        return out

    def free_blocks(self, ordered: Sequence[int]) -> None:
        for b in ordered:
            if self.ref[b] <= 0:
                raise PoolError(f"block {b} is not held")
        for b in ordered:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                if self.hash[b] is not None:
                    self.free.append(b)
                else:
                    self.free.insert(0, b)

    def touch(self, blocks: Sequence[int]) -> None:
        for b in blocks:
            if self.ref[b] == 0:
                self.free.remove(b)
            self.ref[b] += 1

    def cache_full_block(self, b: int, h: bytes) -> None:
        if self.hash[b] is not None:
            return                                  # already cached under its hash
        self.hash[b] = h
        self.index.setdefault(h, []).append(b)

    def lookup(self, hashes: Sequence[bytes]) -> List[int]:
        """Cached blocks for the leading run of hashes (no side effects)."""
        out = []
        for h in hashes:
            ids = self.index.get(h)
            if not ids:
                break
            out.append(ids[0])
        return out

    # ---------------------------------------------------------------- requests
    def allocate_request(self, rid: int, tokens: Sequence[int], extra: bytes = b"") -> int:
        """Give request rid blocks for its tokens, reusing the cached prefix.
        Returns the number of tokens whose K/V are already cached."""
        bs = self.block_size
        n = len(tokens)
        hashes = chain_hashes(tokens, bs, extra)
        usable = (n - 1) // bs if n > 0 else 0
        hits = self.lookup(hashes[:usable])
        need = -(-n // bs) - len(hits)
        if need > len(self.free) - sum(1 for b in hits if self.ref[b] == 0):
            raise PoolError("not enough free blocks")
        self.touch(hits)
        fresh = self.get_new_blocks(need)
        self.requests[rid] = hits + fresh
        return len(hits) * bs

    def cache_request(self, rid: int, tokens: Sequence[int], extra: bytes = b"") -> None:
        """After the request's K/V are written: register its full blocks."""
        hashes = chain_hashes(tokens, self.block_size, extra)
        for b, h in zip(self.requests[rid], hashes):
            self.cache_full_block(b, h)

    def append_slot(self, rid: int, num_tokens_after: int) -> None:
        """Grow request rid to hold num_tokens_after tokens."""
        need = -(-num_tokens_after // self.block_size) - len(self.requests[rid])
        if need > 0:
            self.requests[rid] += self.get_new_blocks(need)

    def free_request(self, rid: int) -> None:
        self.free_blocks([b for b in reversed(self.requests.pop(rid)) if b >= 0])

    def remove_skipped_blocks(self, rid: int, num_tokens: int, window: int) -> int:
        """Sliding window: the next query (position num_tokens) sees positions
        from num_tokens - window + 1; blocks wholly before that are released,
        last to first, and their table entries become -1 ("Paging saves no KV
        bytes", section 5)."""
        first = num_tokens - window + 1
        if first <= 0:
            return 0
        blocks = self.requests[rid]
        n = min(first // self.block_size, len(blocks))
        out = [b for b in reversed(blocks[:n]) if b >= 0]
        self.free_blocks(out)
        for j in range(n):
            blocks[j] = -1
        return len(out)

    # ---------------------------------------------------------------- state
    def state(self) -> dict:
        return {"free": list(self.free), "ref": list(self.ref),
                "hashed": sorted(b for b, h in enumerate(self.hash) if h is not None),
                "index": {h.hex(): list(v) for h, v in self.index.items()}}
