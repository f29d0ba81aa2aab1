"""Host-side block manager used to lay out synthetic paged-KV inputs.

This is bookkeeping, not attention arithmetic: it hands out fixed-size
physical blocks from a global pool, keeps per-block reference counts and
performs copy-on-write re-pointing of block-table entries.  The model it
follows is the one described on the pages:

* "系统级优化：批处理、PagedAttention 与 FlashAttention", section 2.3
  (PagedAttention 解决方案): every page holds the same number of tokens
  (16), a unified block manager hands pages out, a per-request block table
  maps logical pages to physical ones, freed pages are reused at once, and
  read-only pages may be shared without copying.
* "17 · 连续批处理与 PagedAttention", section 三 (PagedAttention：把虚拟内存搬过来):
  physical blocks come from a global pool on demand and need not be
  contiguous; blocks are reference counted so requests can share them;
  a shared block is copied only when a sharer diverges (copy-on-write).

Block ids are handed out in the order of a seeded shuffled free list, so
a sequence's blocks are scattered over the pool.
"""
from __future__ import annotations

from collections import deque
from typing import Deque, List, Sequence, Tuple

import numpy as np

BLOCK_SIZE = 16


def blocks_needed(num_tokens: int, block_size: int = BLOCK_SIZE) -> int:
    """Number of fixed-size blocks that hold ``num_tokens`` tokens (ceil)."""
    if num_tokens < 0:
        raise ValueError("num_tokens must be >= 0")
    return -(-num_tokens // block_size)


class OutOfBlocks(RuntimeError):
    pass


class BlockManager:
    """A global pool of ``num_blocks`` physical blocks with refcounts.

    ``free_order`` fixes the order in which free blocks are handed out
    (a seeded permutation of ``range(num_blocks)``).  Freed blocks go to
    the front of the free list so they are reused at once.
    """

    def __init__(self, num_blocks: int, free_order: Sequence[int]):
        free_order = [int(b) for b in free_order]
        if sorted(free_order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of range(num_blocks)")
        self.num_blocks = num_blocks
        self._free: Deque[int] = deque(free_order)
        self.refcount = np.zeros(num_blocks, dtype=np.int64)

    @property
    def num_free(self) -> int:
        return len(self._free)

    def allocate(self) -> int:
        if not self._free:
            raise OutOfBlocks("block pool exhausted")
        blk = self._free.popleft()
        assert self.refcount[blk] == 0
        self.refcount[blk] = 1
        return blk

    def allocate_tokens(self, num_tokens: int) -> List[int]:
        """Blocks for a new sequence of ``num_tokens`` tokens."""
        return [self.allocate() for _ in range(blocks_needed(num_tokens))]

    def share(self, table: Sequence[int]) -> List[int]:
        """A new table that shares every block of ``table`` (refcount + 1)."""
        for blk in table:
            if self.refcount[blk] <= 0:
                raise ValueError(f"block {blk} is not allocated")
            self.refcount[blk] += 1
        return list(table)

    def release(self, blk: int) -> None:
        if self.refcount[blk] <= 0:
            raise ValueError(f"block {blk} is not allocated")
        self.refcount[blk] -= 1
        if self.refcount[blk] == 0:
            self._free.appendleft(blk)

    def copy_on_write(self, table: List[int], logical: int) -> Tuple[int, int]:
        """Give ``table`` a private copy of its logical block ``logical``.

        Returns the (src, dst) physical pair whose contents the device must
        copy; the table entry is re-pointed to ``dst`` and the reference on
        ``src`` is dropped.
        """
        src = table[logical]
        dst = self.allocate()
        table[logical] = dst
        self.release(src)
        return src, dst


def validate_tables(block_tables: np.ndarray, context_lens: np.ndarray,
                    num_blocks: int, block_size: int = BLOCK_SIZE) -> None:
    """Host check of the preconditions the device code does not check.

    Every entry a sequence uses (logical block < ceil(ctx/16)) must be a
    valid physical id, and the table must be wide enough for the context.
    """
    bt = np.asarray(block_tables)
    cl = np.asarray(context_lens)
    if bt.ndim != 2 or cl.ndim != 1 or bt.shape[0] != cl.shape[0]:
        raise ValueError("block_tables must be [B, MB] and context_lens [B]")
    for b in range(bt.shape[0]):
        n = blocks_needed(int(cl[b]), block_size)
        if n > bt.shape[1]:
            raise ValueError(f"sequence {b}: context {cl[b]} needs {n} blocks > table width {bt.shape[1]}")
        used = bt[b, :n]
        if np.any(used < 0) or np.any(used >= num_blocks):
            raise ValueError(f"sequence {b}: block id out of [0, {num_blocks})")


def validate_slots(slot_mapping: np.ndarray, num_blocks: int,
                   block_size: int = BLOCK_SIZE) -> None:
    """Slots must be unique and inside the pool; negative slots are skips."""
    s = np.asarray(slot_mapping)
    live = s[s >= 0]
    if np.any(live >= num_blocks * block_size):
        raise ValueError("slot outside the pool")
    if np.unique(live).size != live.size:
        raise ValueError("duplicate slot")


def validate_copy_pairs(pairs: np.ndarray, num_blocks: int) -> None:
    """Copy pairs need unique destinations that are never also a source."""
    p = np.asarray(pairs).reshape(-1, 2)
    if p.size and (p.min() < 0 or p.max() >= num_blocks):
        raise ValueError("copy pair block id out of range")
    dst = p[:, 1]
    if np.unique(dst).size != dst.size:
        raise ValueError("duplicate destination block")
    if np.intersect1d(dst, p[:, 0]).size:
        raise ValueError("a destination block is also a source")
