"""Reference model of the host block manager and of one continuous-batching step.

TEST INFRASTRUCTURE: part of the CPU oracle (see the package header).

Written from the pages' description, in plain Python lists and dicts:

* "系统级优化：批处理、PagedAttention 与 FlashAttention", section 2.3 (the
  PagedAttention diagram): pages of 16 tokens handed out by one manager; a
  request of 200 tokens holds 13 pages, one of 150 holds 10; a request's
  pages need not be contiguous; the pages a finished request frees can be
  used by the next request at once.
* "17 · 连续批处理与 PagedAttention", section 三: a global pool of physical
  blocks, reference counts for shared blocks, and copy-on-write: a shared
  block is copied only when a sharer writes into it.
* same page, section 二: continuous batching re-forms the batch after every
  token; section 五: when the KV cache runs out a running request is
  preempted (and recomputed later).

Readings where the pages are silent: free blocks are handed out from the
front of a list that starts in a given order; a freed block is put back at
the front (so it is the next one handed out: "reused at once"); a freed
sequence gives its blocks back last to first, so they return in table order;
an append that finds its last block shared makes a private copy of it; a
step that cannot fit changes nothing.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

BLOCK = 16


class OutOfBlocks(Exception):
    pass


def pages_for_tokens(n: int) -> int:
    return -(-int(n) // BLOCK)


class BlockManagerRef:
    def __init__(self, num_blocks: int, free_order: Optional[Sequence[int]] = None):
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation")
        self.num_blocks = num_blocks
        self.free: List[int] = order             # index 0 is handed out next
        self.ref: List[int] = [0] * num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.tokens: Dict[int, int] = {}

    # -- block pool
    def _take(self) -> int:
        if not self.free:
            raise OutOfBlocks()
        b = self.free.pop(0)
        self.ref[b] = 1
        return b

    def _drop(self, b: int) -> None:
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.free.insert(0, b)

    def _needs_block(self, seq: int) -> bool:
        n = self.tokens[seq]
        return n % BLOCK == 0 or self.ref[self.tables[seq][-1]] > 1

    # -- sequences
    def add(self, seq: int, num_tokens: int) -> None:
        if seq in self.tables or num_tokens < 0:
            raise ValueError("bad add")
        need = pages_for_tokens(num_tokens)
        if need > len(self.free):
            raise OutOfBlocks()
        self.tables[seq] = [self._take() for _ in range(need)]
        self.tokens[seq] = num_tokens

    def fork(self, parent: int, child: int) -> None:
        if parent not in self.tables or child in self.tables:
            raise ValueError("bad fork")
        self.tables[child] = list(self.tables[parent])
        self.tokens[child] = self.tokens[parent]
        for b in self.tables[child]:
            self.ref[b] += 1

    def free_seq(self, seq: int) -> None:
        for b in reversed(self.tables.pop(seq)):
            self._drop(b)
        del self.tokens[seq]

    def append(self, seq: int) -> Tuple[int, Optional[Tuple[int, int]]]:
        """One more token: (its slot, the (src, dst) copy or None)."""
        if self._needs_block(seq) and not self.free:
            raise OutOfBlocks()
        table, n = self.tables[seq], self.tokens[seq]
        pair = None
        if n % BLOCK == 0:
            table.append(self._take())
        elif self.ref[table[-1]] > 1:
            old = table[-1]
            new = self._take()
            self._drop(old)
            table[-1] = new
            pair = (old, new)
        self.tokens[seq] = n + 1
        return table[n // BLOCK] * BLOCK + n % BLOCK, pair

    def step(self, seqs: Sequence[int]):
        """Append one token to each sequence, all or nothing.  Returns
        (tables, context_lens, slots, copy pairs) for the batch."""
        if len(set(seqs)) != len(seqs):
            raise ValueError("a sequence twice in one step")
        need = sum(1 for s in seqs if self._needs_block(s))
        if need > len(self.free):
            raise OutOfBlocks(need - len(self.free))
        slots, pairs = [], []
        for s in seqs:
            slot, pair = self.append(s)
            slots.append(slot)
            if pair:
                pairs.append(pair)
        return [list(self.tables[s]) for s in seqs], [self.tokens[s] for s in seqs], slots, pairs

    # -- accounting
    def stored_tokens(self) -> int:
        """Tokens held in distinct blocks (a shared block counts once)."""
        used: Dict[int, int] = {}
        for s, table in self.tables.items():
            for i, b in enumerate(table):
                used[b] = max(used.get(b, 0), min(BLOCK, self.tokens[s] - i * BLOCK))
        return sum(used.values())
