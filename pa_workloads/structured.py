"""Sequence-major decode inputs, and the "needle" structure.

Sequence-major: the K/V values of sequence b are drawn by their own
generator, seeded by (seed, b), as a logical ``[ctx, kv_heads, head_dim]``
float32 array.  Any subset of sequences can therefore be regenerated on its
own: a test can stream the long-context batch (8 x 131072 tokens) to the
device one sequence at a time and rebuild on the host only what a
comparison needs, without ever holding the whole pool in host memory.

Two recipes:

* ``"normal"``: q, K and V i.i.d. N(0,1)*sigma (the stated distribution of
  the bf16 workloads; for e4m3/int4 caches these are the values before
  quantisation with one amax/top scale per (block, KV head));
* ``"needle"``: every 16-token block of every KV head holds one dominant
  key ("needle") per query head of its group, with a distinctive value row,
  so that each block carries a share of the output far above the parity
  tolerance.  Under the random recipe, long contexts average thousands of
  similar value rows and a missing, repeated or mis-weighted block moves the
  output by less than the tolerance; under this one it moves it by at
  least 1/16 in every element of its group's rows.

Needle construction (G = query heads per KV head, A = 2^ceil(log2 n) / 16
for a sequence whose n blocks have at least G tokens):

* query head j of a group is ``NEEDLE_Q * e_j`` plus N(0,1)*``Q_NOISE`` on
  dimensions G .. D-9, and zero on the last 8 dimensions;
* in every block with at least G tokens, for each KV head, G distinct
  random token slots get the key ``NEEDLE_K * e_j`` (zero elsewhere), one per
  query head j, so that head's logit there is exactly NEEDLE_Q*NEEDLE_K*scale
  (22.6 nats at head_dim 128), about 19 nats above any background key; the
  other heads of the group see 0 there;
* the needle's value row is ``a * A * s`` with an amplitude a in {1, 2}
  drawn per (block, KV head) and a sign vector s in {-1, +1}^D chosen so
  that, per (query head, dimension), the running sum of a*s over the
  sequence's needles (in a random order) is steered to +-NEEDLE_TARGET: the
  output is then (sum of a*s)*A/n, between 1/8 and 3/4 in magnitude, while
  any single needle holds a*A/n >= 1/16 of it;
* e4m3 and int4 pools also get "amax carriers": in a random (block, KV
  head) a background token's last key dimension (where every query is zero)
  is set to +-NEEDLE_K*2^u, u in {1, 2} (e4m3), or +-NEEDLE_K*7/4 (int4),
  so that key scales differ from block to block while the needle's value
  stays exact (e4m3 code 448, 224 or 112; int4 code 7 or 4), and a block
  read with another block's key scale moves its needle logit by a factor
  of 2 or more.

All other tokens are N(0,1)*sigma background.  This module only draws and
places values: no attention arithmetic, no quantisation.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from .block_manager import BLOCK_SIZE
from .configs import (BF16_NAN_BITS, F32_NAN_BITS, PagedWorkload, _bf16_table, _draw_bf16, _poison,
                      make_workload)

NEEDLE_Q = 16.0
NEEDLE_K = 16.0
NEEDLE_TARGET = 4
Q_NOISE = 0.25
ZERO_Q_DIMS = 8          # trailing dimensions where every needle query is zero


@dataclass
class SequenceMajorWorkload:
    """Layout (tables, lengths, slots, pool size) and queries of a decode
    step whose K/V values are drawn per sequence by ``values(b)``."""
    name: str
    seed: int
    recipe: str                      # "normal" | "needle"
    kv_dtype: str                    # "bf16" | "fp8" | "int4"
    layout: PagedWorkload            # values None: block_tables, context_lens, slot_mapping, num_blocks
    q: np.ndarray                    # [B, Hq, D] bf16 bits
    sigma: float = 0.5
    meta: Dict[str, object] = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return self.layout.num_seqs

    @property
    def num_q_heads(self) -> int:
        return self.layout.num_q_heads

    @property
    def num_kv_heads(self) -> int:
        return self.layout.num_kv_heads

    @property
    def head_dim(self) -> int:
        return self.layout.head_dim

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return self.layout.scale

    @property
    def context_lens(self) -> np.ndarray:
        return self.layout.context_lens

    @property
    def block_tables(self) -> np.ndarray:
        return self.layout.block_tables

    @property
    def slot_mapping(self) -> np.ndarray:
        return self.layout.slot_mapping

    @property
    def num_blocks(self) -> int:
        return self.layout.num_blocks

    @property
    def max_context_len(self) -> int:
        return self.layout.max_context_len

    def values(self, b: int) -> Tuple[np.ndarray, np.ndarray]:
        """float32 K, V of sequence b, ``[ctx, kv_heads, head_dim]``, token order."""
        ctx = int(self.context_lens[b])
        rng = np.random.default_rng([self.seed, 7919, b])
        shape = (ctx, self.num_kv_heads, self.head_dim)
        k = rng.standard_normal(shape, dtype=np.float32)
        k *= np.float32(self.sigma)
        v = rng.standard_normal(shape, dtype=np.float32)
        v *= np.float32(self.sigma)
        if self.recipe == "needle":
            plant_needles(rng, k, v, self.group, carriers=self.kv_dtype if self.kv_dtype != "bf16" else None)
        return k, v

    def iter_values(self, seqs: Optional[Sequence[int]] = None, workers: Optional[int] = None):
        """Yield (b, K, V) for ``seqs`` in order, drawing up to ``workers``
        sequences ahead in threads (numpy's generators release the GIL)."""
        seqs = list(range(self.num_seqs)) if seqs is None else [int(b) for b in seqs]
        workers = max(1, min(workers or default_workers(), len(seqs) or 1))
        with ThreadPoolExecutor(workers) as ex:
            futs = [ex.submit(self.values, b) for b in seqs[:workers]]
            for i, b in enumerate(seqs):
                k, v = futs[i].result()
                futs[i] = None
                if i + workers < len(seqs):
                    futs.append(ex.submit(self.values, seqs[i + workers]))
                yield b, k, v


def default_workers() -> int:
    """Threads for drawing sequences: the CPUs this process may use, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def needle_blocks(ctx: int, group: int) -> np.ndarray:
    """Logical blocks of a ctx-token sequence that hold needles (at least `group` tokens)."""
    nblk = -(-int(ctx) // BLOCK_SIZE)
    valid = np.minimum(BLOCK_SIZE, int(ctx) - BLOCK_SIZE * np.arange(nblk))
    return np.flatnonzero(valid >= group)


def needle_amplitude(n: int) -> float:
    """A for a sequence with n needle blocks: the power of two in [n/16, n/8)."""
    return 2.0 ** math.ceil(math.log2(n)) / 16 if n > 0 else 0.0


def plant_needles(rng: np.random.Generator, k: np.ndarray, v: np.ndarray, group: int,
                  carriers: Optional[str] = None) -> None:
    """Overwrite token rows of one sequence's logical K/V with needles (in
    place); ``carriers`` = "fp8" or "int4" adds that format's amax carriers."""
    ctx, hkv, d = k.shape
    blocks = needle_blocks(ctx, group)
    n = len(blocks)
    if n == 0:
        return
    amp_a = needle_amplitude(n)
    valid = np.minimum(BLOCK_SIZE, ctx - BLOCK_SIZE * blocks)               # [n]
    # a random order of each (block, KV head)'s valid slots; needles take the first G
    keys = rng.random((n, hkv, BLOCK_SIZE))
    keys[np.broadcast_to(np.arange(BLOCK_SIZE)[None, None, :] >= valid[:, None, None], keys.shape)] = 2.0
    order = np.argsort(keys, axis=2)
    pos = BLOCK_SIZE * blocks[:, None, None] + order                           # token positions
    npos = pos[:, :, :group]                                                   # [n, Hkv, G]
    amp = rng.integers(1, 3, size=(n, hkv)).astype(np.float32)                 # a in {1, 2}
    target = np.where(rng.random((hkv, group, d)) < 0.5, -NEEDLE_TARGET, NEEDLE_TARGET).astype(np.float32)
    tie = rng.random((n, hkv, group, d)) < 0.5
    visit = rng.permutation(n)
    partial = np.zeros((hkv, group, d), np.float32)
    signs = np.empty((n, hkv, group, d), np.float32)
    for step in range(n):
        i = visit[step]
        want = target - partial
        s = np.where(want > 0, 1.0, np.where(want < 0, -1.0, np.where(tie[step], 1.0, -1.0))).astype(np.float32)
        signs[i] = s
        partial += s * amp[i][:, None, None]
    gi = np.arange(hkv)[None, :, None]
    ji = np.arange(group)[None, None, :]
    k[npos, gi, :] = 0.0
    k[npos, gi, ji] = np.float32(NEEDLE_K)
    v[npos, gi, :] = (amp[:, :, None, None] * np.float32(amp_a)) * signs
    if carriers and group < BLOCK_SIZE:
        # amax carriers: a background token's last key dimension (every query
        # is zero there) sets the block's key scale without moving any logit
        sign = np.where(rng.random((n, hkv)) < 0.5, -1.0, 1.0)
        if carriers == "fp8":
            u = rng.integers(0, 3, size=(n, hkv))        # scale x1, x2, x4: needle code 448, 224, 112
            mag = NEEDLE_K * np.exp2(u)
        else:
            u = rng.integers(0, 2, size=(n, hkv))        # scale NEEDLE_K/7 or NEEDLE_K/4: needle code 7 or 4
            mag = np.where(u > 0, NEEDLE_K * 7.0 / 4.0, NEEDLE_K)
        use = (u > 0) & (valid[:, None] > group)
        bi, hi = np.nonzero(use)
        k[pos[bi, hi, group], hi, d - 1] = (sign[bi, hi] * mag[bi, hi]).astype(np.float32)


def needle_queries(rng: np.random.Generator, num_seqs: int, num_q_heads: int, num_kv_heads: int,
                   head_dim: int) -> np.ndarray:
    """bf16 bits [B, Hq, D]: head j of each group is NEEDLE_Q * e_j plus noise on dims G .. D-9."""
    group = num_q_heads // num_kv_heads
    q = np.zeros((num_seqs, num_q_heads, head_dim), np.float32)
    noise = rng.standard_normal((num_seqs, num_q_heads, head_dim - group - ZERO_Q_DIMS), dtype=np.float32)
    q[:, :, group:head_dim - ZERO_Q_DIMS] = noise * np.float32(Q_NOISE)
    j = np.arange(num_q_heads) % group
    q[:, np.arange(num_q_heads), j] = np.float32(NEEDLE_Q)
    return (q.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def make_sequence_major(*, name: str, seed: int, context_lens: Sequence[int], num_q_heads: int,
                        num_kv_heads: int, head_dim: int, kv_dtype: str, recipe: str, sigma: float = 0.5,
                        pool_slack: float = 1.1, max_blocks_per_seq: Optional[int] = None,
                        partition_tokens: int = 0) -> SequenceMajorWorkload:
    """Layout from a seeded shuffled free list (as make_workload), then the queries."""
    if recipe not in ("normal", "needle"):
        raise ValueError(f"unknown recipe {recipe}")
    if kv_dtype not in ("bf16", "fp8", "int4"):
        raise ValueError(f"unsupported kv_dtype {kv_dtype}")
    rng = np.random.default_rng(seed)
    layout = make_workload(name=name, seed=seed, context_lens=context_lens, num_q_heads=num_q_heads,
                           num_kv_heads=num_kv_heads, head_dim=head_dim, q_dtype="bf16", kv_dtype=kv_dtype,
                           sigma=sigma, pool_slack=pool_slack, max_blocks_per_seq=max_blocks_per_seq,
                           partition_tokens=partition_tokens, rng=rng, with_values=False)
    b = len(layout.context_lens)
    if recipe == "needle":
        q = needle_queries(rng, b, num_q_heads, num_kv_heads, head_dim)
    else:
        q = _draw_bf16(rng, _bf16_table(rng, sigma), (b, num_q_heads, head_dim))
    return SequenceMajorWorkload(name=name, seed=seed, recipe=recipe, kv_dtype=kv_dtype, layout=layout, q=q,
                                 sigma=sigma, meta={"num_blocks": layout.num_blocks})


def block_scales(values: np.ndarray, top: float) -> np.ndarray:
    """Recipe scales of one sequence's logical values: amax/top per (block, KV head)
    over the block's tokens (1 where the block is all zero).  [nblk, Hkv] float32."""
    ctx, hkv, d = values.shape
    nblk = -(-ctx // BLOCK_SIZE)
    pad = np.zeros((nblk * BLOCK_SIZE, hkv, d), np.float32)
    pad[:ctx] = np.abs(values)
    amax = pad.reshape(nblk, BLOCK_SIZE, hkv, d).max(axis=(1, 3))
    return np.where(amax > 0, amax / np.float32(top), np.float32(1.0)).astype(np.float32)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values (the draws need no rounding rule; needle values are exact)."""
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def materialize(swl: SequenceMajorWorkload, seqs: Optional[Sequence[int]] = None,
                compact: bool = False, values: Optional[Dict[int, Tuple[np.ndarray, np.ndarray]]] = None
                ) -> PagedWorkload:
    """A PagedWorkload holding the values of ``seqs`` (default: all).

    compact=False: the workload's own pool and tables (blocks of other
    sequences stay poisoned).  compact=True: a pool holding only these
    sequences' blocks, numbered in sequence order, one spare block for table
    padding; tables, lengths and slots are those of the chosen sequences, in
    that order.  bf16 pools hold bits; e4m3/int4 pools are returned as
    float32 values with amax/top scales (``k_values``, ``k_scale``) for a
    quantiser.  The new token of every sequence (position ctx-1) is taken out
    into new_k/new_v (bf16 bits) and its slot poisoned, as in make_workload.
    ``values`` may hold sequences' (K, V) already drawn by ``values(b)``.
    """
    lay = swl.layout
    seqs = list(range(swl.num_seqs)) if seqs is None else [int(s) for s in seqs]
    hkv, d = swl.num_kv_heads, swl.head_dim
    lens = np.array([int(lay.context_lens[b]) for b in seqs], dtype=np.int32)
    nblks = [-(-int(c) // BLOCK_SIZE) for c in lens]
    if compact:
        nb = sum(nblks) + 1
        starts = np.concatenate([[0], np.cumsum(nblks)]).astype(np.int64)
        mb = max(1, max(nblks))
        tables = np.full((len(seqs), mb), nb - 1, dtype=np.int32)
        for i, n in enumerate(nblks):
            tables[i, :n] = np.arange(starts[i], starts[i] + n)
        pad = nb - 1
    else:
        nb = lay.num_blocks
        tables = lay.block_tables[seqs].astype(np.int32)
        pad = int(lay.meta["pad_block"])
    scaled = swl.kv_dtype in ("fp8", "int4")
    top = 448.0 if swl.kv_dtype == "fp8" else 7.0
    store = np.float32 if scaled else np.uint16
    kpool = np.zeros((nb, hkv, BLOCK_SIZE, d), store)
    vpool = np.zeros((nb, hkv, BLOCK_SIZE, d), store)
    ks = np.ones((nb, hkv), np.float32) if scaled else None
    vs = np.ones((nb, hkv), np.float32) if scaled else None
    new_k = np.empty((len(seqs), hkv, d), np.uint16)
    new_v = np.empty((len(seqs), hkv, d), np.uint16)
    drawn = ((b, *values[b]) for b in seqs) if values is not None else swl.iter_values(seqs)
    for i, (b, k, v) in enumerate(drawn):
        ctx, n = int(lens[i]), nblks[i]
        ids = tables[i, :n].astype(np.int64)
        for pool, src in ((kpool, k), (vpool, v)):
            full = np.zeros((n * BLOCK_SIZE, hkv, d), np.float32)
            full[:ctx] = src
            blocks = full.reshape(n, BLOCK_SIZE, hkv, d).transpose(0, 2, 1, 3)
            pool[ids] = blocks if scaled else to_bf16_bits(blocks)
        if scaled:
            ks[ids] = block_scales(k, top)
            vs[ids] = block_scales(v, top)
        new_k[i] = to_bf16_bits(k[ctx - 1])
        new_v[i] = to_bf16_bits(v[ctx - 1])
    slots = np.array([int(tables[i, (c - 1) // BLOCK_SIZE]) * BLOCK_SIZE + (c - 1) % BLOCK_SIZE
                      for i, c in enumerate(lens)], dtype=np.int64)
    live_tables = [list(tables[i, :n]) for i, n in enumerate(nblks)]
    used = np.array(sorted({blk for t in live_tables for blk in t}), dtype=np.int64)
    nan = F32_NAN_BITS.view(np.float32) if scaled else BF16_NAN_BITS
    for pool in (kpool, vpool):
        _poison(pool, nan, used, live_tables, lens, slots)
    wl = PagedWorkload(
        name=swl.name + ("-compact" if compact else ""), seed=swl.seed, q_dtype="bf16", kv_dtype=swl.kv_dtype,
        num_q_heads=swl.num_q_heads, num_kv_heads=hkv, head_dim=d, scale=swl.scale, q=swl.q[seqs].copy(),
        k_cache=None if scaled else kpool, v_cache=None if scaled else vpool, block_tables=tables,
        context_lens=lens, new_k=new_k, new_v=new_v, slot_mapping=slots, k_scale=ks, v_scale=vs,
        k_values=kpool if scaled else None, v_values=vpool if scaled else None,
        partition_tokens=lay.partition_tokens,
        meta={"num_blocks": nb, "pad_block": pad, "recipe": swl.recipe, "seqs": seqs,
              "fp8_mode": "values" if scaled else None, "sigma": swl.sigma})
    return wl


def config5_sequence_major(recipe: str = "normal", batch: int = 8, context: int = 131072) -> SequenceMajorWorkload:
    """The long-context e4m3 workload (64 q / 8 KV heads, D=128, 8 x 131072
    tokens, 512-token partitions) drawn sequence by sequence: K/V N(0,1)*0.5
    (or the needle recipe) quantised with one amax/448 scale per (block, KV head)."""
    return make_sequence_major(name=f"long_ctx_fp8_{recipe}", seed=5 if recipe == "normal" else 55,
                               context_lens=[context] * batch, num_q_heads=64, num_kv_heads=8, head_dim=128,
                               kv_dtype="fp8", recipe=recipe, partition_tokens=512)


def needle_config(cfg: int, kv_dtype: Optional[str] = None) -> SequenceMajorWorkload:
    """The needle recipe on the shape and lengths of workload 2 (8B, bs 64),
    3 (70B, bs 256) or 5 (long-context e4m3)."""
    from .configs import config2, config3
    if cfg == 2:
        lay = config2(with_values=False)
        return make_sequence_major(name="needle_8b", seed=202, context_lens=lay.context_lens, num_q_heads=32,
                                   num_kv_heads=8, head_dim=128, kv_dtype=kv_dtype or "bf16", recipe="needle",
                                   max_blocks_per_seq=lay.max_blocks_per_seq)
    if cfg == 3:
        lay = config3(with_values=False)
        return make_sequence_major(name="needle_70b", seed=303, context_lens=lay.context_lens, num_q_heads=64,
                                   num_kv_heads=8, head_dim=128, kv_dtype=kv_dtype or "bf16", recipe="needle",
                                   max_blocks_per_seq=lay.max_blocks_per_seq)
    if cfg == 5:
        return config5_sequence_major("needle")
    raise ValueError("needle recipe is defined on workloads 2, 3 and 5")
