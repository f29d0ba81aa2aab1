"""Running the CPU oracle on large inputs: the same oracle functions, called on
slices of the input in a thread pool (numpy releases the GIL in the array
loops that dominate), so that full-size workloads fit a test's time.

Nothing here computes anything itself: quantisation, the slot scatter and
the decode are the oracle's, applied to independent pieces (blocks of a
pool, whole sequences) whose results do not interact.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Sequence

import numpy as np

import oracle


def workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def quantize_pool(values: np.ndarray, scales: np.ndarray, kv_dtype: str) -> np.ndarray:
    """oracle.quantize_pool_ref over block ranges in threads (identical result)."""
    nb = values.shape[0]
    width = values.shape[-1] if kv_dtype == "fp8" else values.shape[-1] // 2
    out = np.empty(values.shape[:-1] + (width,), dtype=np.uint8)
    step = max(1, -(-nb // (4 * workers())))

    def one(s):
        e = min(nb, s + step)
        out[s:e] = oracle.quantize_pool_ref(values[s:e], scales[s:e], kv_dtype)

    with ThreadPoolExecutor(workers()) as ex:
        list(ex.map(one, range(0, nb, step)))
    return out


def quantize_values(wl) -> None:
    """Turn an e4m3/int4 'values' workload into codes (in place), as the oracle does."""
    if wl.k_cache is None:
        wl.k_cache = quantize_pool(wl.k_values, wl.k_scale, wl.kv_dtype)
        wl.v_cache = quantize_pool(wl.v_values, wl.v_scale, wl.kv_dtype)


def after_write(wl):
    """Host caches after the oracle's slot scatter of the new tokens."""
    return oracle.cache_write_ref(wl.k_cache, wl.v_cache, wl.new_k, wl.new_v, wl.slot_mapping, wl.q_dtype,
                                  wl.kv_dtype, wl.k_scale, wl.v_scale)


def decode(wl, k_cache, v_cache, seqs: Optional[Sequence[int]] = None, block_tables=None, context_lens=None,
           k_scale=None, v_scale=None) -> np.ndarray:
    """oracle.decode_ref for `seqs` (default: all), one sequence per task."""
    seqs = list(range(wl.num_seqs)) if seqs is None else [int(s) for s in seqs]
    bt = wl.block_tables if block_tables is None else block_tables
    cl = wl.context_lens if context_lens is None else context_lens
    ks = wl.k_scale if k_scale is None else k_scale
    vs = wl.v_scale if v_scale is None else v_scale

    def one(b):
        return oracle.decode_ref(wl.q, k_cache, v_cache, bt, cl, wl.scale, wl.q_dtype, wl.kv_dtype, ks, vs,
                                 seqs=[b])[0]

    n = min(len(seqs), max(1, workers() // 2))
    if n <= 1:
        return np.stack([one(b) for b in seqs]) if seqs else np.zeros((0,) + wl.q.shape[1:])
    with ThreadPoolExecutor(n) as ex:
        return np.stack(list(ex.map(one, seqs)))
