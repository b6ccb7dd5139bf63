"""Host-side block bookkeeping: reference counts, fork and copy-on-write.

The GPU never sees this; it produces the block tables, slot numbers and
(src, dst) copy pairs that the device calls consume.

Rules, as the pages state them:
  * a request holds ``cdiv(num_tokens, block_size)`` blocks, allocated on
    demand ("Paging saves no KV bytes", section 3; "vLLM intro part 2",
    section 3.2);
  * a block's ``ref_cnt`` counts the requests holding it and the block returns
    to the free list only when it reaches 0 ("GPU memory & KV cache", block
    table and reference counting);
  * forking n sequences from one prompt shares the prompt's blocks, so every
    shared block's count becomes n ("vLLM intro part 2", section 5 diagram);
  * before writing a token into a block whose OWN count is above 1, allocate a
    new block, copy the old one into it, point this request's table at the
    copy, drop the old block's count by one and give the copy a count of 1;
    only then write ("GPU memory & KV cache", copy-on-write five steps and the
    incident fix that checks the block's own count, not table uniqueness);
  * freeing walks a request's blocks from tail to head ("vLLM intro part 2",
    section 6.3 free steps);
  * asking for more blocks than are free raises and changes nothing ("KV Cache
    memory core", section 2.3 BlockPool.get_new_blocks sketch).
"""
from __future__ import annotations

import collections
from typing import Dict, Iterable, List, Optional, Tuple


def cdiv(a: int, b: int) -> int:
    return -(-int(a) // int(b))


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int,
                 free_order: Optional[Iterable[int]] = None):
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            # a partial order lists the first ids handed out; the rest follow in id order
            seen = set(order)
            if len(seen) != len(order) or any(b < 0 or b >= num_blocks for b in order):
                raise ValueError("free_order must hold distinct ids in [0, num_blocks)")
            order += [b for b in range(num_blocks) if b not in seen]
        self.free: collections.deque = collections.deque(order)
        self.ref_cnt: List[int] = [0] * num_blocks
        self.tables: Dict[object, List[int]] = {}
        self.num_tokens: Dict[object, int] = {}

    # ------------------------------------------------------------ queries
    @property
    def num_free(self) -> int:
        return len(self.free)

    def table(self, seq) -> List[int]:
        return list(self.tables[seq])

    # --------------------------------------------------------- allocation
    def _take(self, n: int) -> List[int]:
        if n > len(self.free):
            raise ValueError(f"need {n} free blocks, {len(self.free)} available")
        out = [self.free.popleft() for _ in range(n)]
        for b in out:
            self.ref_cnt[b] += 1
        return out

    def _release(self, b: int) -> None:
        if self.ref_cnt[b] <= 0:
            raise RuntimeError(f"block {b} released with ref_cnt {self.ref_cnt[b]}")
        self.ref_cnt[b] -= 1
        if self.ref_cnt[b] == 0:
            self.free.append(b)

    def allocate(self, seq, num_tokens: int) -> List[int]:
        """A new request holding num_tokens tokens (e.g. its prompt)."""
        if seq in self.tables:
            raise ValueError(f"sequence {seq!r} already exists")
        blocks = self._take(cdiv(num_tokens, self.block_size))
        self.tables[seq] = blocks
        self.num_tokens[seq] = int(num_tokens)
        return list(blocks)

    def slots(self, seq, start: int = 0, stop: Optional[int] = None) -> List[int]:
        """Absolute pool slots block*block_size + offset of tokens [start, stop)."""
        stop = self.num_tokens[seq] if stop is None else stop
        t = self.tables[seq]
        return [t[i // self.block_size] * self.block_size + i % self.block_size
                for i in range(start, stop)]

    def fork(self, parent, children: List) -> None:
        """The parent's blocks are shared by the children; the parent's own
        reference passes to the first child, the others add one each."""
        blocks = self.tables.pop(parent)
        ntok = self.num_tokens.pop(parent)
        for i, c in enumerate(children):
            if c in self.tables:
                raise ValueError(f"sequence {c!r} already exists")
            self.tables[c] = list(blocks)
            self.num_tokens[c] = ntok
            if i > 0:
                for b in blocks:
                    self.ref_cnt[b] += 1

    def append_slot(self, seq) -> Tuple[int, List[Tuple[int, int]]]:
        """Reserve the slot of the sequence's next token.

        Returns (slot, copies) where copies lists the (src, dst) block pairs that
        must be copied on the device before the token is written."""
        t = self.tables[seq]
        pos = self.num_tokens[seq]
        j, off = divmod(pos, self.block_size)
        copies: List[Tuple[int, int]] = []
        if j == len(t):
            t.extend(self._take(1))
        else:
            blk = t[j]
            if self.ref_cnt[blk] > 1:          # the block's own count decides
                new = self._take(1)[0]
                copies.append((blk, new))
                t[j] = new
                self.ref_cnt[blk] -= 1
        self.num_tokens[seq] = pos + 1
        return t[j] * self.block_size + off, copies

    def cow_last_block(self, seq) -> List[Tuple[int, int]]:
        """Take a private copy of the sequence's last block if it is shared."""
        t = self.tables[seq]
        blk = t[-1]
        if self.ref_cnt[blk] <= 1:
            return []
        new = self._take(1)[0]
        t[-1] = new
        self.ref_cnt[blk] -= 1
        return [(blk, new)]

    def free_seq(self, seq) -> None:
        """Release a request's blocks, tail first."""
        for b in reversed(self.tables.pop(seq)):
            self._release(b)
        self.num_tokens.pop(seq)

    def block_table_array(self, seqs: List, pad: int = 0):
        import numpy as np
        width = max(1, max(len(self.tables[s]) for s in seqs))
        out = np.full((len(seqs), width), pad, dtype=np.int32)
        for i, s in enumerate(seqs):
            out[i, :len(self.tables[s])] = self.tables[s]
        return out
