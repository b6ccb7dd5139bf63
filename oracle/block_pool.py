"""Plain model of the host block pool with prefix caching.

TEST INFRASTRUCTURE ONLY: the tests compare the native pool in libpa.so with
this model; nothing in the library imports it.  Python lists and dicts, O(n)
operations, built from the rules the pages state (not from any code they
print), so that a reader can check each rule in isolation:

  R1  one queue holds every block nobody holds (count 0), whether it was never
      used or still keeps the digest of a cached block; blocks are handed out
      from its front ("KV Cache memory core", section 2.3, and its six-block
      walkthrough T0-T4);
  R2  a block handed out loses the digest it kept, and the cache forgets it:
      eviction happens only as a side effect of handing out (same section;
      "vLLM intro part 2", section 6.3, step 3);
  R3  a block whose count falls to 0 joins the back of the queue if it keeps
      a digest (so it stays available for hits as long as possible) and the
      front otherwise; a request gives its blocks back last to first (same
      sections, walkthrough T2);
  R4  a prefix hit on a block nobody holds takes it out of the queue wherever
      it sits and counts it as held (walkthrough T4);
  R5  digests are chained over full blocks: the digest of block i covers the
      digest of block i - 1 (a fixed all-zero value before block 0), block i's
      token ids and the extra keys; a lookup follows the chain from block 0
      and stops at the first digest the cache does not know ("vLLM intro
      part 2", section 6.1; "KV Cache memory core", section 4.1);
  R6  the digest function is SHA-256 ("vLLM intro part 2", section 6.1).

Readings where the pages leave a step open (also listed in the design notes):
the all-zero value is 32 bytes; the digest input is the parent's 32 bytes,
then the token ids as little-endian int32, then the extra-key bytes; blocks
without a digest given back in one call go to the front one after another (the
last one given back ends up first); a request's lookup never covers its last
token, so at most (n - 1) // block_size blocks hit; when several blocks keep
the same digest a lookup takes the one cached first.  A sliding-window
release marks the request's released entries -1; such entries are skipped by
every later request-level operation.
"""
from __future__ import annotations

import hashlib
from typing import Dict, List, Optional, Sequence

import numpy as np

NONE_HASH = bytes(32)        # the digest "before" block 0 (R5)


def block_digest(parent: Optional[bytes], token_ids: Sequence[int],
                 extra: bytes = b"") -> bytes:
    """R5/R6: SHA-256 over parent digest (all-zero before block 0), the token
    ids as little-endian int32, then the extra-key bytes."""
    head = NONE_HASH if parent is None else bytes(parent)
    ids = np.asarray(list(token_ids), dtype="<i4").tobytes()
    return hashlib.sha256(head + ids + bytes(extra)).digest()


def prompt_digests(token_ids: Sequence[int], block_size: int, extra: bytes = b"") -> List[bytes]:
    """R5: digests of the full blocks of a token sequence, each chained on the
    one before."""
    toks = list(token_ids)
    digests: List[bytes] = []
    for start in range(0, len(toks) - block_size + 1, block_size):
        prev = digests[-1] if digests else None
        digests.append(block_digest(prev, toks[start:start + block_size], extra))
    return digests


class PoolError(Exception):
    pass


class BlockPoolModel:
    """count[b]: holders of block b; kept[b]: the digest block b keeps (or
    None); queue: ids nobody holds, front first; cached: digest -> ids that
    keep it, in the order they were cached; requests: id -> block table row."""

    def __init__(self, num_blocks: int, block_size: int):
        self.block_size = block_size
        self.count = [0] * num_blocks
        self.kept: List[Optional[bytes]] = [None] * num_blocks
        self.queue: List[int] = list(range(num_blocks))
        self.cached: Dict[bytes, List[int]] = {}
        self.requests: Dict[int, List[int]] = {}

    # ------------------------------------------------------------ R1-R4
    def num_free(self) -> int:
        return len(self.queue)

    def _forget_digest(self, b: int) -> None:
        """R2: drop block b's digest from the block and from the cache."""
        d = self.kept[b]
        if d is None:
            return
        self.kept[b] = None
        owners = self.cached[d]
        owners.remove(b)
        if not owners:
            del self.cached[d]

    def get_new_blocks(self, n: int) -> List[int]:
        """R1 + R2: the first n queued blocks, each now held once."""
        if n > len(self.queue):
            raise PoolError("not enough free blocks")
        given = [self.queue.pop(0) for _ in range(n)]
        for b in given:
            self._forget_digest(b)
            self.count[b] = 1
        return given

    def free_blocks(self, ordered: Sequence[int]) -> None:
        """R3: one count less per listed id, in the order given."""
        if any(self.count[b] < 1 for b in ordered):
            raise PoolError("a listed block is not held")
        for b in ordered:
            self.count[b] -= 1
            if self.count[b]:
                continue
            if self.kept[b] is None:
                self.queue.insert(0, b)
            else:
                self.queue.append(b)

    def touch(self, blocks: Sequence[int]) -> None:
        """R4: count a hit block as held, leaving the queue if nobody held it."""
        for b in blocks:
            if self.count[b] == 0:
                self.queue.remove(b)
            self.count[b] += 1

    def cache_full_block(self, b: int, digest: bytes) -> None:
        """Let block b keep this digest (a block keeps its first digest)."""
        if self.kept[b] is None:
            self.kept[b] = digest
            self.cached.setdefault(digest, []).append(b)

    def lookup(self, digests: Sequence[bytes]) -> List[int]:
        """R5: blocks for the leading run of known digests (changes nothing)."""
        hits: List[int] = []
        for d in digests:
            if d not in self.cached:
                break
            hits.append(self.cached[d][0])
        return hits

    # ------------------------------------------------------------ requests
    def allocate_request(self, rid: int, tokens: Sequence[int], extra: bytes = b"") -> int:
        """Blocks for a new request: the cached prefix (never its last token),
        then fresh blocks.  Returns how many tokens are already cached."""
        bs, n = self.block_size, len(tokens)
        lookable = (n - 1) // bs if n else 0
        hits = self.lookup(prompt_digests(tokens, bs, extra)[:lookable])
        fresh = -(-n // bs) - len(hits)
        queued_hits = sum(1 for b in hits if self.count[b] == 0)
        if fresh > len(self.queue) - queued_hits:
            raise PoolError("not enough free blocks")
        self.touch(hits)
        self.requests[rid] = hits + self.get_new_blocks(fresh)
        return len(hits) * bs

    def cache_request(self, rid: int, tokens: Sequence[int], extra: bytes = b"") -> None:
        """Once the request's K/V are written, its full blocks keep their
        digests; entries released by a sliding window (-1) are skipped."""
        row = self.requests[rid]
        for j, d in enumerate(prompt_digests(tokens, self.block_size, extra)[:len(row)]):
            if row[j] >= 0:
                self.cache_full_block(row[j], d)

    def append_slot(self, rid: int, num_tokens_after: int) -> None:
        """Grow request rid to hold num_tokens_after tokens."""
        row = self.requests[rid]
        more = -(-num_tokens_after // self.block_size) - len(row)
        if more > 0:
            row.extend(self.get_new_blocks(more))

    def free_request(self, rid: int) -> None:
        row = self.requests.pop(rid)
        self.free_blocks([b for b in row[::-1] if b >= 0])

    def remove_skipped_blocks(self, rid: int, num_tokens: int, window: int) -> int:
        """Sliding window ("Paging saves no KV bytes", section 5): the request's
        next query sits at position num_tokens and sees its last `window`
        positions, num_tokens - window + 1 onward.  Give back, last to first,
        every block all of whose positions lie before that, and mark its
        entry -1.  Returns how many blocks were given back."""
        first_seen = num_tokens - window + 1
        row = self.requests[rid]
        before = min(max(first_seen, 0) // self.block_size, len(row))
        gone = [row[j] for j in range(before - 1, -1, -1) if row[j] >= 0]
        self.free_blocks(gone)
        row[:before] = [-1] * before
        return len(gone)

    # ------------------------------------------------------------ state
    def state(self) -> dict:
        return {"free": list(self.queue), "ref": list(self.count),
                "hashed": sorted(b for b, d in enumerate(self.kept) if d is not None),
                "index": {d.hex(): list(v) for d, v in self.cached.items()}}
