"""Float64 reference for paged-KV decode attention.

TEST INFRASTRUCTURE: part of the CPU oracle.  Only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import it; the library's GPU path never does, and this module imports
nothing from the library.

What it computes, and where that is stated:

* Attention is ``softmax(Q K^T / sqrt(d_k)) V``
  ("系统级优化：批处理、PagedAttention 与 FlashAttention", section 3.1, the
  attention equation; the scale convention ``head_dim ** -0.5`` is the
  ``scale`` argument of the SDPA call in section 3.3).  Decode has one query
  token per sequence ("推理优化", section "Prefill vs Decode"), so each query
  head attends over every cached token of its sequence.
* The cache is paged: fixed 16-token blocks, and a per-request block table
  that maps logical block i to a physical block anywhere in a global pool
  ("系统级优化…" section 2.3; "17 · 连续批处理与 PagedAttention" section 三;
  "推理优化" section "PagedAttention").  Paging only changes where bytes
  live, so the reference first gathers a sequence's blocks back into a
  contiguous ``[kv_heads, ctx, head_dim]`` cache and then applies the plain
  definition.
* GQA: several query heads share one KV head ("推理优化" section 五,
  exercise 3: 64 query heads, 8 KV heads).  The pages do not fix which query
  heads share which KV head; this reference takes consecutive groups:
  query head h reads KV head ``h // (Hq / Hkv)``.  The pages do not fix
  the mapping; it is a convention shared with the kernels by specification,
  and the pins check the attention itself for this mapping.
* fp8 KV: codes times one float scale per (block, KV head); the scale is
  applied to the decoded code values before attention.

Several new query tokens per sequence (``multi_query_ref``): a chunk of a
chunked prefill ("17 · 连续批处理与 PagedAttention", section 二, remedy ①:
a long prefill cut into pieces spread over iterations), the K draft tokens a
target model checks in one pass ("推理优化", section 一, speculative
decoding), or the unique suffix after a prefix-cache hit (same section,
prefix caching).  The new tokens are the last ``q_len`` positions of the
sequence and their K/V are already in the cache; token i of the chunk sits
at position ``ctx - q_len + i`` and attends to every token at or before that
position (the causal mask of "系统级优化…" section 3.3, aligned so that the
last query token sees the whole context).

Partitioned decode (``decode_partitioned_ref``) splits each sequence's
context into fixed-size token ranges, computes for each range the running
maximum ``m``, the sum ``l = sum exp(s - m)`` and the unnormalised output
``acc = sum exp(s - m) v``, and merges them with
``out = sum_p e^{m_p - M} acc_p / sum_p e^{m_p - M} l_p``, ``M = max_p m_p``.
That identity is exact in real arithmetic; it is the log-sum-exp merge the
GPU path uses across partitions.
"""
from __future__ import annotations

from typing import Iterable, Optional, Tuple

import numpy as np

from .formats import bf16_to_f64, e4m3_to_f64, int4_to_f64

BLOCK = 16


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored elements of ``dtype`` ("f32", "bf16", "fp8")."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_to_f64(x)
    if dtype == "fp8":
        return e4m3_to_f64(x)
    if dtype == "int4":
        return int4_to_f64(x)                    # unpacks the last axis: D/2 bytes -> D values
    raise ValueError(f"unknown dtype {dtype}")


def num_blocks_for(ctx: int) -> int:
    return -(-int(ctx) // BLOCK)


def gather_kv(cache: np.ndarray, block_table: np.ndarray, ctx: int, kv_dtype: str,
              scales: Optional[np.ndarray] = None) -> np.ndarray:
    """Contiguous float64 ``[Hkv, ctx, D]`` view of one sequence's paged cache.

    Logical block i of the sequence lives in physical block ``block_table[i]``;
    token t sits in logical block ``t // 16`` at offset ``t % 16``.
    """
    n = num_blocks_for(ctx)
    if n > len(block_table):
        raise ValueError("context longer than the block table")
    phys = np.asarray(block_table[:n], dtype=np.int64)
    if n and (phys.min() < 0 or phys.max() >= cache.shape[0]):
        raise ValueError("block id outside the pool")
    blocks = to_f64(cache[phys], kv_dtype)                  # [n, Hkv, 16, D]
    if scales is not None:
        blocks = blocks * np.asarray(scales, dtype=np.float32)[phys].astype(np.float64)[:, :, None, None]
    hkv, d = blocks.shape[1], blocks.shape[3]
    contiguous = blocks.transpose(1, 0, 2, 3).reshape(hkv, n * BLOCK, d)
    return contiguous[:, :ctx, :]


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """softmax(q k^T * scale) v for one query row per head, GQA by consecutive groups.

    q: [Hq, D]; k, v: [Hkv, ctx, D] (float64).  Returns (out [Hq, D], lse [Hq]),
    lse = log sum_t exp(s_t) of the scaled logits.
    """
    hq, d = q.shape
    hkv, ctx, _ = k.shape
    if hq % hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    group = hq // hkv
    out = np.zeros((hq, d), dtype=np.float64)
    lse = np.full(hq, -np.inf, dtype=np.float64)
    if ctx == 0:
        return out, lse
    for h in range(hq):
        g = h // group
        s = (k[g] @ q[h]) * scale                           # [ctx]
        m = s.max()
        p = np.exp(s - m)
        denom = p.sum()
        out[h] = (p @ v[g]) / denom
        lse[h] = m + np.log(denom)
    return out, lse


def decode_ref(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, block_tables: np.ndarray,
               context_lens: np.ndarray, scale: float, q_dtype: str, kv_dtype: str,
               k_scale: Optional[np.ndarray] = None, v_scale: Optional[np.ndarray] = None,
               seqs: Optional[Iterable[int]] = None, with_lse: bool = False):
    """Paged decode: for every sequence b, gather its K/V and attend with q[b].

    q: [B, Hq, D]; caches [NB, Hkv, 16, D]; block_tables [B, MB];
    context_lens [B].  Returns float64 out [len(seqs), Hq, D] (and lse).
    """
    if kv_dtype in ("fp8", "int4") and (k_scale is None or v_scale is None):
        raise ValueError("fp8 and int4 caches need k_scale and v_scale")
    seqs = list(range(len(context_lens))) if seqs is None else list(seqs)
    hq, d = q.shape[1], q.shape[2]
    outs = np.zeros((len(seqs), hq, d), dtype=np.float64)
    lses = np.zeros((len(seqs), hq), dtype=np.float64)
    for i, b in enumerate(seqs):
        ctx = int(context_lens[b])
        k = gather_kv(k_cache, block_tables[b], ctx, kv_dtype, k_scale)
        v = gather_kv(v_cache, block_tables[b], ctx, kv_dtype, v_scale)
        outs[i], lses[i] = attend(to_f64(q[b], q_dtype), k, v, scale)
    return (outs, lses) if with_lse else outs


def partition_stats(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, start: int, stop: int):
    """(m, l, acc) of the token range [start, stop) for every query head.

    m = max_t s_t, l = sum_t exp(s_t - m), acc = sum_t exp(s_t - m) v_t.
    An empty range gives m = -inf, l = 0, acc = 0.
    """
    hq, d = q.shape
    hkv = k.shape[0]
    group = hq // hkv
    m = np.full(hq, -np.inf)
    l = np.zeros(hq)
    acc = np.zeros((hq, d))
    if stop <= start:
        return m, l, acc
    for h in range(hq):
        g = h // group
        s = (k[g, start:stop] @ q[h]) * scale
        m[h] = s.max()
        p = np.exp(s - m[h])
        l[h] = p.sum()
        acc[h] = p @ v[g, start:stop]
    return m, l, acc


def lse_merge_ref(m: np.ndarray, l: np.ndarray, acc: np.ndarray) -> np.ndarray:
    """Merge per-partition (m [P], l [P], acc [P, D]) into the normalised output [D].

    Partitions with m = -inf hold no token and are skipped (this avoids
    exp(-inf - (-inf))).  With no token at all the output is zero.
    """
    live = np.isfinite(m)
    if not np.any(live):
        return np.zeros(acc.shape[-1])
    m, l, acc = m[live], l[live], acc[live]
    big = m.max()
    w = np.exp(m - big)
    return (w @ acc) / (w @ l)


def decode_partitioned_ref(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                           block_tables: np.ndarray, context_lens: np.ndarray, scale: float,
                           q_dtype: str, kv_dtype: str, partition_tokens: int,
                           k_scale: Optional[np.ndarray] = None, v_scale: Optional[np.ndarray] = None,
                           seqs: Optional[Iterable[int]] = None) -> np.ndarray:
    """Decode by fixed token partitions and a log-sum-exp merge (same result as decode_ref)."""
    if partition_tokens <= 0:
        raise ValueError("partition_tokens must be positive")
    seqs = list(range(len(context_lens))) if seqs is None else list(seqs)
    hq, d = q.shape[1], q.shape[2]
    outs = np.zeros((len(seqs), hq, d))
    for i, b in enumerate(seqs):
        ctx = int(context_lens[b])
        k = gather_kv(k_cache, block_tables[b], ctx, kv_dtype, k_scale)
        v = gather_kv(v_cache, block_tables[b], ctx, kv_dtype, v_scale)
        qb = to_f64(q[b], q_dtype)
        starts = list(range(0, ctx, partition_tokens))
        stats = [partition_stats(qb, k, v, scale, s, min(ctx, s + partition_tokens)) for s in starts]
        if not stats:
            continue
        ms = np.stack([s[0] for s in stats], axis=1)        # [Hq, P]
        ls = np.stack([s[1] for s in stats], axis=1)
        accs = np.stack([s[2] for s in stats], axis=1)      # [Hq, P, D]
        for h in range(hq):
            outs[i, h] = lse_merge_ref(ms[h], ls[h], accs[h])
    return outs


def multi_query_ref(q: np.ndarray, q_start: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                    block_tables: np.ndarray, context_lens: np.ndarray, scale: float, q_dtype: str,
                    kv_dtype: str, k_scale: Optional[np.ndarray] = None, v_scale: Optional[np.ndarray] = None,
                    seqs: Optional[Iterable[int]] = None) -> np.ndarray:
    """Causal attention of several new tokens per sequence over its paged cache.

    q: [T, Hq, D], the new tokens of all sequences packed in order; sequence b
    owns rows [q_start[b], q_start[b+1]), q_len = their count (<= ctx).
    Token i of sequence b sees positions [0, ctx - q_len + i].  Returns
    float64 [T, Hq, D] (rows of sequences outside ``seqs`` stay zero).
    """
    if kv_dtype in ("fp8", "int4") and (k_scale is None or v_scale is None):
        raise ValueError("fp8 and int4 caches need k_scale and v_scale")
    q_start = np.asarray(q_start, dtype=np.int64)
    n_seq = len(context_lens)
    if len(q_start) != n_seq + 1 or np.any(np.diff(q_start) < 0) or q_start[0] != 0:
        raise ValueError("q_start must be a non-decreasing offset list starting at 0")
    seqs = list(range(n_seq)) if seqs is None else list(seqs)
    out = np.zeros((q.shape[0], q.shape[1], q.shape[2]), dtype=np.float64)
    for b in seqs:
        ctx = int(context_lens[b])
        q_len = int(q_start[b + 1] - q_start[b])
        if q_len > ctx:
            raise ValueError("a sequence has more new tokens than context")
        k = gather_kv(k_cache, block_tables[b], ctx, kv_dtype, k_scale)
        v = gather_kv(v_cache, block_tables[b], ctx, kv_dtype, v_scale)
        for i, pos in enumerate(query_positions(ctx, q_len)):
            row = int(q_start[b]) + i
            out[row], _ = attend(to_f64(q[row], q_dtype), k[:, :pos + 1], v[:, :pos + 1], scale)
    return out


def query_positions(ctx: int, q_len: int) -> np.ndarray:
    """Positions of a sequence's q_len newest tokens: ctx - q_len .. ctx - 1."""
    return np.arange(ctx - q_len, ctx, dtype=np.int64)
