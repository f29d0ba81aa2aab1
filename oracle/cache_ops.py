"""Reference for the two cache-mutating operations: slot scatter and block copy.

TEST INFRASTRUCTURE: part of the CPU oracle.  Only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import it.

* ``cache_write_ref`` is the paged form of appending new K/V to a cache:
  "推理优化" (section 二, Step 1) writes new keys/values into a contiguous
  ``[layers, heads, seq, head_dim]`` cache at the next positions; with a
  paged cache, position t of a sequence lives in slot
  ``block_table[t // 16] * 16 + t % 16`` ("系统级优化…" section 2.3), so
  the write becomes a scatter to slots.  A negative slot means "skip".
  For an fp8 cache each value is stored as the e4m3 code of
  ``float32(x) / float32(scale[block, head])``, rounded to nearest even and
  saturated at 448; for an int4 cache as the int4 code of the same
  quotient (round half to even, clamped to [-8, 7]), two per byte.
* ``copy_blocks_ref`` is the copy step of copy-on-write: a block shared by
  several sequences is duplicated when one of them diverges
  ("17 · 连续批处理与 PagedAttention" section 三, 写时复制的共享;
  "推理优化" section "PagedAttention").  Each (src, dst) pair copies all
  KV heads of the K and V blocks, and for fp8 caches the per-(block, head)
  scales.

Both return new arrays and leave their inputs untouched.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .formats import bf16_to_f32, e4m3_quantize, e4m3_to_f64, int4_quantize, int4_to_f64

BLOCK = 16


def _src_f32(x: np.ndarray, src_dtype: str) -> np.ndarray:
    if src_dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    if src_dtype == "bf16":
        return bf16_to_f32(x)
    raise ValueError(f"unsupported source dtype {src_dtype}")


def cache_write_ref(k_cache: np.ndarray, v_cache: np.ndarray, new_k: np.ndarray, new_v: np.ndarray,
                    slot_mapping: np.ndarray, src_dtype: str, cache_dtype: str,
                    k_scale: Optional[np.ndarray] = None,
                    v_scale: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Scatter token t's K/V ``[Hkv, D]`` rows into ``cache[slot // 16, :, slot % 16, :]``.

    Tokens are applied in order; slots < 0 are skipped.  For f32 and bf16
    caches the source must have the cache's type and its bits are copied.
    """
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    for t, slot in enumerate(slots):
        if slot < 0:
            continue
        blk, off = int(slot) // BLOCK, int(slot) % BLOCK
        if cache_dtype in ("f32", "bf16"):
            if src_dtype != cache_dtype:
                raise ValueError("f32/bf16 caches take sources of the same type")
            k_out[blk, :, off, :] = new_k[t]
            v_out[blk, :, off, :] = new_v[t]
        elif cache_dtype in ("fp8", "int4"):
            quantize = e4m3_quantize if cache_dtype == "fp8" else int4_quantize
            ks = np.asarray(k_scale, dtype=np.float32)[blk][:, None]
            vs = np.asarray(v_scale, dtype=np.float32)[blk][:, None]
            k_out[blk, :, off, :] = quantize(_src_f32(new_k[t], src_dtype), ks)
            v_out[blk, :, off, :] = quantize(_src_f32(new_v[t], src_dtype), vs)
        else:
            raise ValueError(f"unknown cache dtype {cache_dtype}")
    return k_out, v_out


def quantize_pool_ref(values: np.ndarray, scales: np.ndarray, cache_dtype: str = "fp8") -> np.ndarray:
    """Codes of a float32 pool ``[NB, Hkv, 16, D]`` with scales ``[NB, Hkv]``:
    e4m3 (``[NB, Hkv, 16, D]`` bytes) or packed int4 (``[NB, Hkv, 16, D/2]``)."""
    quantize = e4m3_quantize if cache_dtype == "fp8" else int4_quantize
    width = values.shape[-1] if cache_dtype == "fp8" else values.shape[-1] // 2
    out = np.empty(values.shape[:-1] + (width,), dtype=np.uint8)
    step = max(1, (1 << 22) // max(1, int(np.prod(values.shape[1:]))))
    for s in range(0, values.shape[0], step):
        e = min(values.shape[0], s + step)
        out[s:e] = quantize(values[s:e], scales[s:e][:, :, None, None])
    return out


def copy_blocks_ref(k_cache: np.ndarray, v_cache: np.ndarray, pairs: np.ndarray,
                    k_scale: Optional[np.ndarray] = None, v_scale: Optional[np.ndarray] = None):
    """Copy block src to block dst for every (src, dst) pair, in order."""
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    ks = None if k_scale is None else np.array(k_scale, copy=True)
    vs = None if v_scale is None else np.array(v_scale, copy=True)
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        k_out[dst] = k_out[src]
        v_out[dst] = v_out[src]
        if ks is not None:
            ks[dst] = ks[src]
            vs[dst] = vs[src]
    return k_out, v_out, ks, vs


def _decode_codes(codes: np.ndarray, cache_dtype: str) -> np.ndarray:
    """float32 value of stored codes (e4m3 bytes, or packed int4 unpacked along the last axis)."""
    if cache_dtype == "fp8":
        return e4m3_to_f64(codes).astype(np.float32)
    return int4_to_f64(codes).astype(np.float32)


def cache_write_autoscale_ref(k_cache: np.ndarray, v_cache: np.ndarray, k_scale: np.ndarray, v_scale: np.ndarray,
                              new_k: np.ndarray, new_v: np.ndarray, slot_mapping: np.ndarray, src_dtype: str,
                              cache_dtype: str):
    """Slot scatter into an e4m3 or int4 cache that sets the block scales itself.

    The rows one call writes into a block form a run (consecutive tokens of the
    call, consecutive offsets from o0).  Per (block, head), with top = 448
    (e4m3) or 7 (int4) and a = max |x| over the run's new values:
      * o0 == 0 (the block starts here): scale = a / top (1 if a == 0);
      * otherwise, if a > old_scale * top, the scale grows to a / top and the
        rows already in the block (offsets < o0) are re-encoded: value =
        float32(code value) * old_scale, code = encode(value / new_scale);
      * otherwise the old scale stays.
    The new rows are then encoded with the block's scale, as cache_write_ref
    does.  All arithmetic is float32 (IEEE products and quotients).
    Returns (k_cache, v_cache, k_scale, v_scale), new arrays.
    """
    top = np.float32(448.0 if cache_dtype == "fp8" else 7.0)
    quantize = e4m3_quantize if cache_dtype == "fp8" else int4_quantize
    outs = []
    for cache, scale, new in ((k_cache, k_scale, new_k), (v_cache, v_scale, new_v)):
        cache = np.array(cache, copy=True)
        scale = np.array(scale, dtype=np.float32, copy=True)
        slots = np.asarray(slot_mapping, dtype=np.int64)
        t = 0
        while t < len(slots):
            if slots[t] < 0:
                t += 1
                continue
            blk, o0 = int(slots[t]) // BLOCK, int(slots[t]) % BLOCK
            e = t + 1
            while e < len(slots) and slots[e] >= 0 and int(slots[e]) // BLOCK == blk:
                e += 1
            rows = _src_f32(new[t:e], src_dtype)                            # [n, Hkv, D]
            for h in range(cache.shape[1]):
                a = np.float32(np.abs(rows[:, h, :]).max())
                old = scale[blk, h]
                if o0 == 0:
                    s = np.float32(a / top) if a > 0 else np.float32(1.0)
                elif a > np.float32(old * top):
                    s = np.float32(a / top)
                    kept = _decode_codes(cache[blk, h, :o0], cache_dtype) * old   # float32 products
                    cache[blk, h, :o0] = quantize(kept, s)
                else:
                    s = old
                scale[blk, h] = s
                for i in range(e - t):
                    off = int(slots[t + i]) % BLOCK
                    cache[blk, h, off] = quantize(rows[i, h], s)
            t = e
        outs.append((cache, scale))
    return outs[0][0], outs[1][0], outs[0][1], outs[1][1]
