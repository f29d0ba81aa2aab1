"""Seeded synthetic paged-KV decode workloads.

These generators produce the inputs that both the CPU oracle and the GPU
library consume: a query per sequence, a paged K/V pool laid out as
``[num_blocks, kv_heads, 16, head_dim]``, per-sequence block tables and
context lengths, the slot mapping of one new token per sequence, and (for
the shared-prefix layout) copy-on-write block pairs.  They hold none of
the attention arithmetic and no format conversion beyond drawing bits:

* bf16 values are drawn i.i.d. from a 65536-entry table of N(0,1)*sigma
  float32 samples cut to their upper 16 bits (random data needs no rounding
  rule);
* fp8-e4m3 and int4 pools are either drawn directly as random codes with
  random per-(block, kv head) scales (``fp8_mode="codes"``), or returned as
  float32 values plus per-(block, kv head) scales (``fp8_mode="values"``;
  amax/448 for e4m3, amax/7 for int4)
  for a quantiser to turn into codes;
* every byte the decode must not read is NaN: unused pool blocks, slots of a
  last block past the context, block-table padding (which points at an
  unused block) and, until the new token is written, the new token's slot.

Generation order (fixed, so a seed fixes everything): context lengths ->
pool permutation -> q -> K/V pool -> new tokens -> poison.

The page model (16-token blocks, per-request block table, global pool,
reference-counted sharing with copy-on-write) follows
"系统级优化：批处理、PagedAttention 与 FlashAttention" section 2.3 and
"17 · 连续批处理与 PagedAttention" section 三; the GQA head grouping follows
"推理优化" section 五 (exercise 3: 64 query heads over 8 KV heads).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

from .block_manager import BLOCK_SIZE, BlockManager, blocks_needed

F32_NAN_BITS = np.uint32(0x7FC00000)
BF16_NAN_BITS = np.uint16(0x7FC0)
FP8_NAN_CODE = np.uint8(0x7F)

STORAGE = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8, "int4": np.uint8}
ELEM_BYTES = {"f32": 4, "bf16": 2, "fp8": 1, "int4": 0.5}
# int4 has no NaN: bytes the decode must not read hold code 15 (value 7) in both nibbles
INT4_POISON = np.uint8(0xFF)


@dataclass
class PagedWorkload:
    name: str
    seed: int
    q_dtype: str                     # "f32" | "bf16"
    kv_dtype: str                    # "f32" | "bf16" | "fp8"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    scale: float
    q: np.ndarray                    # [B, Hq, D] float32 or bf16 bits (uint16)
    k_cache: Optional[np.ndarray]    # [NB, Hkv, 16, D]; None until fp8 values are quantised
    v_cache: Optional[np.ndarray]
    block_tables: np.ndarray         # [B, MB] int32, the tables the decode uses
    context_lens: np.ndarray         # [B] int32
    new_k: np.ndarray                # [T, Hkv, D] in q_dtype storage
    new_v: np.ndarray
    slot_mapping: np.ndarray         # [T] int64
    k_scale: Optional[np.ndarray] = None   # [NB, Hkv] float32 (fp8 only)
    v_scale: Optional[np.ndarray] = None
    k_values: Optional[np.ndarray] = None  # fp8_mode="values": float32 pool values
    v_values: Optional[np.ndarray] = None
    copy_pairs: Optional[np.ndarray] = None          # [n, 2] int32 (src, dst)
    block_tables_shared: Optional[np.ndarray] = None  # tables before copy-on-write
    refcount: Optional[np.ndarray] = None            # per-block refcount before copy-on-write
    partition_tokens: int = 0
    block_size: int = BLOCK_SIZE
    meta: Dict[str, object] = field(default_factory=dict)
    # several new tokens per sequence: q is [sum(q_lens), Hq, D] and sequence b
    # owns rows q_start[b] .. q_start[b+1]-1 (None: one query per sequence)
    q_start: Optional[np.ndarray] = None

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.meta["num_blocks"])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0


# ---------------------------------------------------------------------------
# value drawing (bits only)

def _bf16_table(rng: np.random.Generator, sigma: float) -> np.ndarray:
    x = (rng.standard_normal(65536, dtype=np.float32) * np.float32(sigma))
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _draw_bf16(rng: np.random.Generator, table: np.ndarray, shape) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    chunk = 1 << 24
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        idx = rng.integers(0, 65536, size=e - s, dtype=np.uint32)
        np.take(table, idx, out=out[s:e])
    return out.reshape(shape)


def _draw_f32(rng: np.random.Generator, sigma: float, shape) -> np.ndarray:
    out = rng.standard_normal(int(np.prod(shape)), dtype=np.float32)
    if sigma != 1.0:
        out *= np.float32(sigma)
    return out.reshape(shape)


def _draw_fp8_codes(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniformly random finite e4m3 codes (the two NaN codes are moved down by one)."""
    n = int(np.prod(shape))
    out = np.frombuffer(rng.bytes(n), dtype=np.uint8).copy()
    nan = (out & np.uint8(0x7F)) == np.uint8(0x7F)
    out[nan] -= np.uint8(1)
    return out.reshape(shape)


def _nan_like(dtype: str):
    if dtype == "f32":
        return F32_NAN_BITS.view(np.float32)
    if dtype == "bf16":
        return BF16_NAN_BITS
    if dtype == "int4":
        return INT4_POISON
    return FP8_NAN_CODE


# ---------------------------------------------------------------------------
# generic builder

def _layout_sequences(rng, context_lens: Sequence[int], pool_blocks: Optional[int],
                      pool_slack: float, max_blocks_per_seq: Optional[int]):
    need = sum(blocks_needed(int(c)) for c in context_lens)
    if pool_blocks is None:
        pool_blocks = int(math.ceil(pool_slack * need))
    pool_blocks = max(pool_blocks, need + 1)          # always keep one spare block for padding
    free_order = rng.permutation(pool_blocks)
    bm = BlockManager(pool_blocks, free_order)
    tables = [bm.allocate_tokens(int(c)) for c in context_lens]
    mb = max_blocks_per_seq or max(1, max(len(t) for t in tables))
    return bm, tables, mb


def _tables_array(tables: List[List[int]], mb: int, pad_block: int) -> np.ndarray:
    bt = np.full((len(tables), mb), pad_block, dtype=np.int32)
    for b, t in enumerate(tables):
        if len(t) > mb:
            raise ValueError("table wider than max_blocks_per_seq")
        bt[b, :len(t)] = t
    return bt


def _new_token_slots(tables: List[List[int]], context_lens: Sequence[int]) -> np.ndarray:
    slots = np.empty(len(context_lens), dtype=np.int64)
    for b, c in enumerate(context_lens):
        pos = int(c) - 1
        slots[b] = tables[b][pos // BLOCK_SIZE] * BLOCK_SIZE + pos % BLOCK_SIZE
    return slots


def _poison(cache: np.ndarray, nan, used_blocks: np.ndarray, tables, context_lens, new_slots):
    unused = np.ones(cache.shape[0], dtype=bool)
    unused[used_blocks] = False
    cache[unused] = nan
    for b, c in enumerate(context_lens):
        c = int(c)
        if c % BLOCK_SIZE:
            last = tables[b][(c - 1) // BLOCK_SIZE]
            cache[last, :, c % BLOCK_SIZE:, :] = nan
    for s in new_slots:
        cache[s // BLOCK_SIZE, :, s % BLOCK_SIZE, :] = nan


def _fp8_scales_from_values(values: np.ndarray, tables, context_lens, top: float = 448.0) -> np.ndarray:
    """Per-(block, kv head) scale = amax/top over the block's live tokens (recipe;
    top = 448 for e4m3, 7 for int4)."""
    nb, hkv = values.shape[:2]
    scale = np.ones((nb, hkv), dtype=np.float32)
    for b, c in enumerate(context_lens):
        c = int(c)
        for i, blk in enumerate(tables[b]):
            n = min(BLOCK_SIZE, c - i * BLOCK_SIZE)
            amax = np.abs(values[blk, :, :n, :]).reshape(hkv, -1).max(axis=1)
            scale[blk] = np.where(amax > 0, amax / np.float32(top), np.float32(1.0))
    return scale


def make_workload(*, name: str, seed: int, context_lens: Sequence[int], num_q_heads: int,
                  num_kv_heads: int, head_dim: int, q_dtype: str, kv_dtype: str,
                  sigma: float = 0.5, pool_slack: float = 1.1, pool_blocks: Optional[int] = None,
                  max_blocks_per_seq: Optional[int] = None, partition_tokens: int = 0,
                  fp8_mode: str = "values", rng: Optional[np.random.Generator] = None,
                  scale: Optional[float] = None, with_values: bool = True) -> PagedWorkload:
    """One decode step over independent sequences laid out in a shuffled pool.

    ``with_values=False`` stops after the layout (block tables, lengths, slot
    mapping): q, caches and new tokens are then None.
    """
    if num_q_heads % num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    rng = rng or np.random.default_rng(seed)
    context_lens = [int(c) for c in context_lens]
    if any(c < 1 for c in context_lens):
        raise ValueError("every sequence needs at least its new token")
    B, D, Hkv = len(context_lens), head_dim, num_kv_heads
    # 1-2: lengths (given) and pool permutation
    bm, tables, mb = _layout_sequences(rng, context_lens, pool_blocks, pool_slack, max_blocks_per_seq)
    nb = bm.num_blocks
    pad = bm._free[0]
    if not with_values:
        return PagedWorkload(
            name=name, seed=seed, q_dtype=q_dtype, kv_dtype=kv_dtype, num_q_heads=num_q_heads,
            num_kv_heads=Hkv, head_dim=D,
            scale=float(scale if scale is not None else 1.0 / math.sqrt(D)), q=None, k_cache=None,
            v_cache=None, block_tables=_tables_array(tables, mb, pad),
            context_lens=np.asarray(context_lens, dtype=np.int32), new_k=None, new_v=None,
            slot_mapping=_new_token_slots(tables, context_lens), refcount=bm.refcount.copy(),
            partition_tokens=partition_tokens,
            meta={"num_blocks": nb, "pad_block": pad, "sigma": sigma})
    # 3: q
    table16 = _bf16_table(rng, sigma) if "bf16" in (q_dtype, kv_dtype) else None
    q = (_draw_f32(rng, sigma, (B, num_q_heads, D)) if q_dtype == "f32"
         else _draw_bf16(rng, table16, (B, num_q_heads, D)))
    # 4: K/V pool
    new_slots = _new_token_slots(tables, context_lens)
    k_values = v_values = k_scale = v_scale = None
    if kv_dtype == "f32":
        k_cache = _draw_f32(rng, sigma, (nb, Hkv, BLOCK_SIZE, D))
        v_cache = _draw_f32(rng, sigma, (nb, Hkv, BLOCK_SIZE, D))
    elif kv_dtype == "bf16":
        k_cache = _draw_bf16(rng, table16, (nb, Hkv, BLOCK_SIZE, D))
        v_cache = _draw_bf16(rng, table16, (nb, Hkv, BLOCK_SIZE, D))
    elif kv_dtype == "int4" and fp8_mode == "codes":
        # every byte is a valid pair of int4 codes; scales 2^U(-4,-2): values up to 8/4 = 2
        k_cache = np.frombuffer(rng.bytes(nb * Hkv * BLOCK_SIZE * D // 2), dtype=np.uint8).copy().reshape(
            nb, Hkv, BLOCK_SIZE, D // 2)
        v_cache = np.frombuffer(rng.bytes(nb * Hkv * BLOCK_SIZE * D // 2), dtype=np.uint8).copy().reshape(
            nb, Hkv, BLOCK_SIZE, D // 2)
        k_scale = np.exp2(rng.uniform(-4.0, -2.0, size=(nb, Hkv))).astype(np.float32)
        v_scale = np.exp2(rng.uniform(-4.0, -2.0, size=(nb, Hkv))).astype(np.float32)
    elif kv_dtype == "fp8" and fp8_mode == "codes":
        k_cache = _draw_fp8_codes(rng, (nb, Hkv, BLOCK_SIZE, D))
        v_cache = _draw_fp8_codes(rng, (nb, Hkv, BLOCK_SIZE, D))
        # scales 2^u, u ~ U(-8, -6): dequantised magnitudes up to 448/64 = 7
        k_scale = np.exp2(rng.uniform(-8.0, -6.0, size=(nb, Hkv))).astype(np.float32)
        v_scale = np.exp2(rng.uniform(-8.0, -6.0, size=(nb, Hkv))).astype(np.float32)
    elif kv_dtype in ("fp8", "int4") and fp8_mode == "values":
        k_values = _draw_f32(rng, sigma, (nb, Hkv, BLOCK_SIZE, D))
        v_values = _draw_f32(rng, sigma, (nb, Hkv, BLOCK_SIZE, D))
        k_cache = v_cache = None
    else:
        raise ValueError(f"unsupported kv_dtype/fp8_mode {kv_dtype}/{fp8_mode}")
    # 5: new tokens (in the query's storage type)
    new_k, new_v = _extract_new_tokens(rng, q_dtype, kv_dtype, fp8_mode, sigma, table16,
                                       k_cache, v_cache, k_values, v_values, new_slots, Hkv, D)
    if kv_dtype in ("fp8", "int4") and fp8_mode == "values":
        top = 448.0 if kv_dtype == "fp8" else 7.0
        k_scale = _fp8_scales_from_values(k_values, tables, context_lens, top)
        v_scale = _fp8_scales_from_values(v_values, tables, context_lens, top)
    # 6: poison
    used = np.array(sorted({blk for t in tables for blk in t}), dtype=np.int64)
    if k_cache is not None:
        _poison(k_cache, _nan_like(kv_dtype), used, tables, context_lens, new_slots)
        _poison(v_cache, _nan_like(kv_dtype), used, tables, context_lens, new_slots)
    if k_values is not None:
        nanf = F32_NAN_BITS.view(np.float32)
        _poison(k_values, nanf, used, tables, context_lens, new_slots)
        _poison(v_values, nanf, used, tables, context_lens, new_slots)
    wl = PagedWorkload(
        name=name, seed=seed, q_dtype=q_dtype, kv_dtype=kv_dtype, num_q_heads=num_q_heads,
        num_kv_heads=Hkv, head_dim=D, scale=float(scale if scale is not None else 1.0 / math.sqrt(D)),
        q=q, k_cache=k_cache, v_cache=v_cache, block_tables=_tables_array(tables, mb, pad),
        context_lens=np.asarray(context_lens, dtype=np.int32), new_k=new_k, new_v=new_v,
        slot_mapping=new_slots, k_scale=k_scale, v_scale=v_scale, k_values=k_values,
        v_values=v_values, refcount=bm.refcount.copy(), partition_tokens=partition_tokens,
        meta={"num_blocks": nb, "pad_block": pad, "fp8_mode": fp8_mode if kv_dtype in ("fp8", "int4") else None,
              "sigma": sigma})
    return wl


def _extract_new_tokens(rng, q_dtype, kv_dtype, fp8_mode, sigma, table16, k_cache, v_cache,
                        k_values, v_values, new_slots, Hkv, D):
    T = len(new_slots)
    blk = new_slots // BLOCK_SIZE
    off = new_slots % BLOCK_SIZE
    if kv_dtype in ("f32", "bf16"):
        # the new token's K/V are the pool's values at its slot (then poisoned in the pool)
        return k_cache[blk, :, off, :].copy(), v_cache[blk, :, off, :].copy()
    if fp8_mode == "values":
        nk = k_values[blk, :, off, :].copy()
        nv = v_values[blk, :, off, :].copy()
        if q_dtype == "bf16":
            nk = (nk.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
            nv = (nv.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
        return nk, nv
    # fp8 codes mode: fresh draws in the source type
    if q_dtype == "bf16":
        return _draw_bf16(rng, table16, (T, Hkv, D)), _draw_bf16(rng, table16, (T, Hkv, D))
    return _draw_f32(rng, sigma, (T, Hkv, D)), _draw_f32(rng, sigma, (T, Hkv, D))


# ---------------------------------------------------------------------------
# several new tokens per sequence (chunked prefill, draft verification)

def make_multi_query_workload(*, name: str, seed: int, context_lens: Sequence[int], q_lens: Sequence[int],
                              num_q_heads: int, num_kv_heads: int, head_dim: int, kv_dtype: str = "bf16",
                              fp8_mode: str = "values", sigma: float = 0.5,
                              pool_slack: float = 1.1) -> PagedWorkload:
    """The layout and pool of ``make_workload`` (one new token per sequence
    still to be written by a slot scatter), then bf16 queries for the last
    q_lens[b] positions of every sequence, packed in sequence order.

    Draw order: everything ``make_workload`` draws, then the packed queries.
    """
    q_lens = [int(n) for n in q_lens]
    if len(q_lens) != len(context_lens) or any(n < 0 or n > c for n, c in zip(q_lens, context_lens)):
        raise ValueError("need 0 <= q_lens[b] <= context_lens[b] for every sequence")
    rng = np.random.default_rng(seed)
    wl = make_workload(name=name, seed=seed, context_lens=context_lens, num_q_heads=num_q_heads,
                       num_kv_heads=num_kv_heads, head_dim=head_dim, q_dtype="bf16", kv_dtype=kv_dtype,
                       sigma=sigma, pool_slack=pool_slack, fp8_mode=fp8_mode, rng=rng)
    table16 = _bf16_table(rng, sigma)
    wl.q = _draw_bf16(rng, table16, (int(sum(q_lens)), num_q_heads, head_dim))
    wl.q_start = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    return wl


# ---------------------------------------------------------------------------
# shared-prefix / parallel-sampling layout

def make_shared_prefix_workload(*, name: str, seed: int, num_prompts: int, samples_per_prompt: int,
                                prefix_tokens: int, suffix_max: int, num_q_heads: int,
                                num_kv_heads: int, head_dim: int, sigma: float = 0.5,
                                pool_slack: float = 1.1, dtype: str = "bf16",
                                suffix_lens: Optional[Sequence[int]] = None,
                                with_values: bool = True) -> PagedWorkload:
    """Parallel sampling: every sample of a prompt shares the prompt's prefix blocks.

    The prefix blocks carry refcount = samples_per_prompt.  Each sample then
    takes a private copy of the last prefix block (copy-on-write), which
    yields one (src, dst) pair per sample, applied in one copy call.
    """
    rng = np.random.default_rng(seed)
    P, S, D, Hkv = num_prompts, samples_per_prompt, head_dim, num_kv_heads
    n_prefix = blocks_needed(prefix_tokens)
    # 1: lengths
    if suffix_lens is None:
        suffix_lens = rng.integers(1, suffix_max + 1, size=P * S)
    suffix_lens = np.asarray(suffix_lens, dtype=np.int64)
    context_lens = prefix_tokens + suffix_lens
    # suffix blocks start at the first block boundary at or after the prefix end
    prefix_cap = n_prefix * BLOCK_SIZE
    # 2: pool permutation and layout
    need = P * n_prefix + sum(blocks_needed(int(c)) - n_prefix for c in context_lens) + P * S
    nb = max(int(math.ceil(pool_slack * need)), need + 1)
    bm = BlockManager(nb, rng.permutation(nb))
    tables: List[List[int]] = []
    for p in range(P):
        prefix = bm.allocate_tokens(prefix_tokens)
        for s in range(S):
            tables.append(bm.share(prefix))
        for blk in prefix:
            bm.release(blk)                     # the prompt itself keeps no reference
    for i, c in enumerate(context_lens):
        if prefix_tokens % BLOCK_SIZE:
            raise ValueError("prefix must end on a block boundary in this layout")
        tables[i] += bm.allocate_tokens(int(c) - prefix_cap)
    refcount_shared = bm.refcount.copy()
    shared_tables = [list(t) for t in tables]
    # copy-on-write of the last prefix block, all destinations taken before any source is freed
    pairs = []
    for t in tables:
        src = t[n_prefix - 1]
        dst = bm.allocate()
        t[n_prefix - 1] = dst
        pairs.append((src, dst))
    for src, _ in pairs:
        bm.release(src)
    mb = blocks_needed(prefix_tokens + suffix_max)
    pad = bm._free[0]
    meta = {"num_blocks": nb, "pad_block": pad, "prefix_blocks": n_prefix,
            "num_prompts": P, "samples_per_prompt": S, "sigma": sigma}
    if not with_values:
        return PagedWorkload(
            name=name, seed=seed, q_dtype="bf16", kv_dtype="bf16", num_q_heads=num_q_heads,
            num_kv_heads=Hkv, head_dim=D, scale=1.0 / math.sqrt(D), q=None, k_cache=None,
            v_cache=None, block_tables=_tables_array(tables, mb, pad),
            context_lens=np.asarray(context_lens, dtype=np.int32), new_k=None, new_v=None,
            slot_mapping=_new_token_slots(tables, context_lens),
            copy_pairs=np.asarray(pairs, dtype=np.int32).reshape(-1, 2),
            block_tables_shared=_tables_array(shared_tables, mb, pad), refcount=refcount_shared,
            meta=meta)
    # 3: q
    table16 = _bf16_table(rng, sigma)
    B = P * S
    if dtype != "bf16":
        raise ValueError("shared-prefix layout is defined for bf16")
    q = _draw_bf16(rng, table16, (B, num_q_heads, D))
    # 4: K/V pool
    k_cache = _draw_bf16(rng, table16, (nb, Hkv, BLOCK_SIZE, D))
    v_cache = _draw_bf16(rng, table16, (nb, Hkv, BLOCK_SIZE, D))
    # 5: new tokens at position ctx-1 (always in a private suffix block)
    new_slots = _new_token_slots(tables, context_lens)
    blk, off = new_slots // BLOCK_SIZE, new_slots % BLOCK_SIZE
    new_k = k_cache[blk, :, off, :].copy()
    new_v = v_cache[blk, :, off, :].copy()
    # 6: poison everything not referenced before the copy (copy destinations included)
    used = np.array(sorted({b for t in shared_tables for b in t}), dtype=np.int64)
    for cache in (k_cache, v_cache):
        _poison(cache, BF16_NAN_BITS, used, shared_tables, context_lens, new_slots)
    return PagedWorkload(
        name=name, seed=seed, q_dtype="bf16", kv_dtype="bf16", num_q_heads=num_q_heads,
        num_kv_heads=Hkv, head_dim=D, scale=1.0 / math.sqrt(D), q=q, k_cache=k_cache,
        v_cache=v_cache, block_tables=_tables_array(tables, mb, pad),
        context_lens=np.asarray(context_lens, dtype=np.int32), new_k=new_k, new_v=new_v,
        slot_mapping=new_slots, copy_pairs=np.asarray(pairs, dtype=np.int32).reshape(-1, 2),
        block_tables_shared=_tables_array(shared_tables, mb, pad), refcount=refcount_shared,
        meta=meta)


# ---------------------------------------------------------------------------
# the five workloads

def config1(with_values: bool = True) -> PagedWorkload:
    """Tiny fp32 layer: 4 sequences {17,33,48,5}, 4 q = 4 kv heads, D=64, 16-block pool."""
    return make_workload(name="tiny_fp32", seed=1, context_lens=[17, 33, 48, 5], num_q_heads=4,
                         num_kv_heads=4, head_dim=64, q_dtype="f32", kv_dtype="f32", sigma=1.0,
                         pool_blocks=16, max_blocks_per_seq=4, with_values=with_values)


def config2_lengths(rng: np.random.Generator, batch: int = 64) -> np.ndarray:
    return rng.integers(128, 4096 + 1, size=batch)


def config2(batch: int = 64, with_values: bool = True, seed: int = 2) -> PagedWorkload:
    """Llama-3-8B-shaped layer: 32 q / 8 kv heads, D=128, bf16, ctx ~ U{128..4096}."""
    rng = np.random.default_rng(seed)
    lens = config2_lengths(rng, batch)
    return make_workload(name="llama3_8b_bs64", seed=seed, context_lens=lens, num_q_heads=32,
                         num_kv_heads=8, head_dim=128, q_dtype="bf16", kv_dtype="bf16",
                         max_blocks_per_seq=4096 // BLOCK_SIZE, rng=rng, with_values=with_values)


LOGNORMAL_SIGMA = 1.0


def config3(batch: int = 256, with_values: bool = True) -> PagedWorkload:
    """Llama-3-70B-shaped layer: 64 q / 8 kv heads, ctx = clip(lognormal(ln 2048, 1.0), 16, 8192)."""
    rng = np.random.default_rng(3)
    lens = np.clip(np.rint(rng.lognormal(math.log(2048.0), LOGNORMAL_SIGMA, size=batch)), 16, 8192)
    return make_workload(name="llama3_70b_bs256", seed=3, context_lens=lens.astype(np.int64),
                         num_q_heads=64, num_kv_heads=8, head_dim=128, q_dtype="bf16",
                         kv_dtype="bf16", max_blocks_per_seq=8192 // BLOCK_SIZE, rng=rng,
                         with_values=with_values)


def config4(with_values: bool = True) -> PagedWorkload:
    """32 prompts x 8 samples sharing a 2000-token prefix (125 blocks, refcount 8)."""
    return make_shared_prefix_workload(name="shared_prefix_32x8", seed=4, num_prompts=32,
                                       samples_per_prompt=8, prefix_tokens=2000, suffix_max=512,
                                       num_q_heads=32, num_kv_heads=8, head_dim=128,
                                       with_values=with_values)


def config5(batch: int = 8, context: int = 131072, fp8_mode: str = "codes",
            with_values: bool = True) -> PagedWorkload:
    """Long-context fp8 KV: 64 q / 8 kv heads, 8 x 131072 tokens, 512-token partitions."""
    return make_workload(name="long_ctx_fp8", seed=5, context_lens=[context] * batch,
                         num_q_heads=64, num_kv_heads=8, head_dim=128, q_dtype="bf16",
                         kv_dtype="fp8", partition_tokens=512, fp8_mode=fp8_mode,
                         with_values=with_values)


CONFIGS = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}
