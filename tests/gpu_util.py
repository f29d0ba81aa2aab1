"""Helpers for the GPU parity tests: move seeded workloads to the device, run the
library through its C-ABI binding, and compare with the CPU oracle."""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import oracle
import pa_workloads as W
from parity import TOL, parity_error


def log(msg: str) -> None:
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(arr: np.ndarray, kind: str, device: str = "cuda") -> torch.Tensor:
    arr = np.ascontiguousarray(arr)
    if kind == "bf16":
        t = torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(arr)
    return t.to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def out_to_f64(t: torch.Tensor) -> np.ndarray:
    h = to_host(t)
    return oracle.bf16_to_f64(h) if t.dtype == torch.bfloat16 else h.astype(np.float64)


def quantize_fp8_values(wl: W.PagedWorkload) -> None:
    """Turn an fp8 or int4 'values' workload into codes with the oracle's quantiser (CPU)."""
    if wl.k_cache is None:
        wl.k_cache = oracle.quantize_pool_ref(wl.k_values, wl.k_scale, wl.kv_dtype)
        wl.v_cache = oracle.quantize_pool_ref(wl.v_values, wl.v_scale, wl.kv_dtype)


class DeviceWorkload:
    def __init__(self, wl: W.PagedWorkload):
        self.wl = wl
        qk = wl.q_dtype
        self.q = to_dev(wl.q, qk)
        self.k_cache = to_dev(wl.k_cache, wl.kv_dtype)
        self.v_cache = to_dev(wl.v_cache, wl.kv_dtype)
        self.k_scale = None if wl.k_scale is None else to_dev(wl.k_scale, "f32")
        self.v_scale = None if wl.v_scale is None else to_dev(wl.v_scale, "f32")
        self.block_tables = to_dev(wl.block_tables.astype(np.int32), "i32")
        self.context_lens = to_dev(wl.context_lens.astype(np.int32), "i32")
        self.slot_mapping = to_dev(wl.slot_mapping.astype(np.int64), "i64")
        self.new_k = to_dev(wl.new_k, qk)
        self.new_v = to_dev(wl.new_v, qk)
        self.out = torch.empty_like(self.q)

    def cache_write(self, pa):
        pa.pa_cache_write(self.new_k, self.new_v, self.k_cache, self.v_cache, self.slot_mapping,
                          self.k_scale, self.v_scale)

    def decode(self, pa, partition_tokens=None, block_tables=None, out=None):
        wl = self.wl
        out = self.out if out is None else out
        pa.pa_decode(out, self.q, self.k_cache, self.v_cache,
                     self.block_tables if block_tables is None else block_tables, self.context_lens,
                     wl.max_context_len, wl.scale, self.k_scale, self.v_scale,
                     wl.partition_tokens if partition_tokens is None else partition_tokens)
        return out

    def decode_append(self, pa, partition_tokens=None, out=None):
        wl = self.wl
        out = self.out if out is None else out
        pa.pa_decode_append(out, self.q, self.new_k, self.new_v, self.k_cache, self.v_cache, self.block_tables,
                            self.context_lens, wl.max_context_len, wl.scale, self.k_scale, self.v_scale,
                            wl.partition_tokens if partition_tokens is None else partition_tokens)
        return out


def oracle_after_write(wl: W.PagedWorkload):
    """Host caches after the oracle's slot scatter of the new tokens."""
    return oracle.cache_write_ref(wl.k_cache, wl.v_cache, wl.new_k, wl.new_v, wl.slot_mapping, wl.q_dtype,
                                  wl.kv_dtype, wl.k_scale, wl.v_scale)


def assert_written_rows_equal(dw: DeviceWorkload, k_ref: np.ndarray, v_ref: np.ndarray, orig_k, orig_v):
    """Bit-exact check of a slot scatter on a large pool: the rows at the
    live slots equal the oracle's, and no other byte of the device pool changed."""
    slots = dw.wl.slot_mapping
    live = slots[slots >= 0]
    blk = torch.from_numpy(live // 16).cuda()
    off = torch.from_numpy(live % 16).cuda()
    for dev, ref, orig in ((dw.k_cache, k_ref, orig_k), (dw.v_cache, v_ref, orig_v)):
        got = to_host(dev[blk, :, off, :])
        want = ref[live // 16, :, live % 16, :]
        assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), "written rows differ from the oracle"
        changed = (dev.view(torch.uint8) != orig.view(torch.uint8))
        changed[blk, :, off, :] = False
        assert not bool(changed.any()), "the scatter touched bytes outside the written slots"


def sample_seqs(wl: W.PagedWorkload, n: int):
    cl = wl.context_lens
    if len(cl) <= n:
        return list(range(len(cl)))
    picks = {int(np.argmin(cl)), int(np.argmax(cl))}
    picks |= set(int(i) for i in np.linspace(0, len(cl) - 1, n - 2).round())
    return sorted(picks)


def decode_error(wl: W.PagedWorkload, out_dev: torch.Tensor, k_host, v_host, seqs):
    got = out_to_f64(out_dev)[seqs]
    want = oracle.decode_ref(wl.q, k_host, v_host, wl.block_tables, wl.context_lens, wl.scale, wl.q_dtype,
                             wl.kv_dtype, wl.k_scale, wl.v_scale, seqs=seqs)
    return parity_error(got, want)
