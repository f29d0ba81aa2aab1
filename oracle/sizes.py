"""Closed-form KV-cache sizes.

TEST INFRASTRUCTURE: part of the CPU oracle.

* KV bytes = 2 x layers x KV heads x head_dim x tokens x bytes per element
  ("推理优化", section "KV 缓存"; the same product per token and per layer
  appears in "17 · 连续批处理与 PagedAttention", section "P/D 分离的那笔账").
* A request of n tokens occupies ceil(n / 16) pages
  ("系统级优化…" section 2.3: 200 tokens in 13 pages, 150 in 10).
* Internal waste is below one block per request
  ("17 · 连续批处理与 PagedAttention", section 三).
"""
from __future__ import annotations

BLOCK = 16


def kv_bytes(layers: int, kv_heads: int, head_dim: int, tokens: int, bytes_per_elem: int) -> int:
    return 2 * layers * kv_heads * head_dim * tokens * bytes_per_elem


def pages_for(tokens: int, block_size: int = BLOCK) -> int:
    return -(-tokens // block_size)


def internal_waste_tokens(tokens: int, block_size: int = BLOCK) -> int:
    """Slots allocated but unused in the last page of a request."""
    return pages_for(tokens, block_size) * block_size - tokens


def decode_algorithmic_bytes(context_lens, num_q_heads: int, num_kv_heads: int, head_dim: int,
                             kv_elem_bytes: int, q_elem_bytes: int, out_elem_bytes: int,
                             fp8_scales: bool = False) -> int:
    """Bytes a paged decode step must move: every live K/V element once, q, out,
    the used block-table entries, context lengths and (fp8) the used scales."""
    ctx = [int(c) for c in context_lens]
    tokens = sum(ctx)
    pages = sum(pages_for(c) for c in ctx)
    b = len(ctx)
    total = tokens * num_kv_heads * head_dim * 2 * kv_elem_bytes
    total += b * num_q_heads * head_dim * (q_elem_bytes + out_elem_bytes)
    total += pages * 4 + 4 * b
    if fp8_scales:
        total += pages * num_kv_heads * 2 * 4
    return total


def physical_kv_bytes(block_tables, context_lens, num_q_heads: int, num_kv_heads: int, head_dim: int,
                      kv_elem_bytes: int, q_rows: int, q_elem_bytes: int = 2, out_elem_bytes: int = 2,
                      fp8_scales: bool = False) -> int:
    """Bytes an attention step must move when every physical block is read
    once, however many sequences reference it ("17 · 连续批处理与
    PagedAttention", section 三: a shared block is stored once): for each
    distinct physical block, its K and V rows up to the furthest token any
    of its sequences uses; plus q and out rows (q_rows of them), the used
    block-table entries, context lengths and (fp8) the used scales."""
    visible = {}
    pages = 0
    for b, ctx in enumerate(context_lens):
        ctx = int(ctx)
        n = pages_for(ctx)
        pages += n
        for i in range(n):
            blk = int(block_tables[b][i])
            visible[blk] = max(visible.get(blk, 0), min(BLOCK, ctx - i * BLOCK))
    tokens = sum(visible.values())
    total = tokens * num_kv_heads * head_dim * 2 * kv_elem_bytes
    total += q_rows * num_q_heads * head_dim * (q_elem_bytes + out_elem_bytes)
    total += pages * 4 + 4 * len(context_lens)
    if fp8_scales:
        total += len(visible) * num_kv_heads * 2 * 4
    return total
