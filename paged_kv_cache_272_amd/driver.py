"""Continuous-batching decode loop over libpa.

The native host block manager (pa_bm_*) decides every iteration's slots,
copy-on-write pairs and block tables; this class moves those small host
arrays to the device in one pa_upload (a copy kernel on the compute stream)
and issues the library's kernels in order: pa_copy_blocks for the pairs
(if any), then pa_decode_append (the newest
token's K/V written into its slot and attended over).  This is the
per-iteration scheduling of "17 · 连续批处理与 PagedAttention" section 二 (the
batch is re-formed after every token; finished sequences leave and waiting
ones join) on the paged cache of section 三.  Which sequences run, finish
or are preempted is the caller's policy; when the pool cannot hold a step,
`step` raises OutOfBlocks and changes nothing, so the caller can preempt a
sequence (free it, recompute it later: section 五) and retry.

No kernel runs on the host: this module only orders calls and copies
host arrays.  Device memory comes from PyTorch.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np
import torch

from . import _lib
from ._lib import BLOCK_SIZE, HostBlockManager


class DecodeDriver:
    def __init__(self, num_blocks: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                 max_blocks_per_seq: int, max_batch: int, scale: Optional[float] = None,
                 dtype: torch.dtype = torch.bfloat16, device="cuda", free_order=None):
        self.bm = HostBlockManager(num_blocks, free_order)
        self.hq, self.hkv, self.d = num_q_heads, num_kv_heads, head_dim
        self.mb, self.max_batch = max_blocks_per_seq, max_batch
        self.scale = head_dim ** -0.5 if scale is None else scale
        self.device = torch.device(device)
        self.k_cache = torch.empty(num_blocks, num_kv_heads, BLOCK_SIZE, head_dim, dtype=dtype, device=self.device)
        self.v_cache = torch.empty_like(self.k_cache)
        # The per-iteration arrays share one buffer, [lens | pairs | tables],
        # each section starting on 16 bytes, so that one pa_upload moves the
        # used prefix to the device copy of the same layout.  Two pinned host
        # buffers are used in turn; a buffer is refilled only after the
        # upload that read it has finished.
        r16 = lambda n: (n + 3) // 4 * 4  # int32 elements to a multiple of 16 bytes
        self._off_pr = r16(max_batch)
        self._off_bt = self._off_pr + r16(2 * max_batch)
        self._words = self._off_bt + r16(max_batch * max_blocks_per_seq)
        self._host = []
        for _ in range(2):
            buf = torch.zeros(self._words, dtype=torch.int32).pin_memory()
            self._host.append({
                "buf": buf,
                "views": self._views(buf),
                "sl": torch.zeros(max_batch, dtype=torch.int64).pin_memory(),
                "done": None,
            })
        self._turn = 0
        self._dev = torch.zeros(self._words, dtype=torch.int32, device=self.device)
        self.cl, self.pr, self.bt = self._views(self._dev)
        ws = _lib.pa_decode_workspace_size(max_batch, num_q_heads, num_kv_heads, head_dim,
                                           max_blocks_per_seq * BLOCK_SIZE, 0)
        self.workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=self.device)
        self.last_pairs = 0

    def _views(self, buf: torch.Tensor):
        """(lens [max_batch], pairs [max_batch, 2], tables [max_batch, mb]) over a packed buffer."""
        n, mb = self.max_batch, self.mb
        return (buf[:n], buf[self._off_pr:self._off_pr + 2 * n].view(n, 2),
                buf[self._off_bt:self._off_bt + n * mb].view(n, mb))

    # -- sequences
    def add_sequence(self, seq: int, k: torch.Tensor, v: torch.Tensor) -> None:
        """A new sequence whose K/V for its first n tokens are k, v [n, Hkv, D]
        (device, cache dtype): blocks from the manager, rows written by
        pa_cache_write."""
        n = int(k.shape[0])
        self.bm.add(seq, n)
        if n == 0:
            return
        table, _ = self.bm.table(seq)
        pos = np.arange(n, dtype=np.int64)
        slots = torch.from_numpy(table[pos // BLOCK_SIZE].astype(np.int64) * BLOCK_SIZE + pos % BLOCK_SIZE)
        _lib.pa_cache_write(k, v, self.k_cache, self.v_cache, slots.to(self.device, non_blocking=True))

    def fork(self, parent: int, child: int) -> None:
        self.bm.fork(parent, child)

    def finish(self, seq: int) -> None:
        self.bm.free(seq)

    # -- one iteration
    def step(self, seqs: Sequence[int], q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
             out: torch.Tensor) -> None:
        """Append one token to each of ``seqs`` and attend: q, out [B, Hq, D];
        k_new, v_new [B, Hkv, D] (cache dtype).  Raises OutOfBlocks (nothing
        changed) if the pool cannot hold the step."""
        b = len(seqs)
        if b == 0:
            return
        if b > self.max_batch:
            raise ValueError("batch larger than max_batch")
        h = self._host[self._turn]
        self._turn ^= 1
        if h["done"] is not None:
            h["done"].synchronize()
        hcl, hpr, hbt = h["views"]
        bt, cl, _, pr = self.bm.step(seqs, self.mb, out=(hbt.numpy(), hcl.numpy(), h["sl"].numpy(), hpr.numpy()))
        npairs = len(pr)
        _lib.pa_upload(self._dev, h["buf"], (self._off_bt + (b * self.mb + 3) // 4 * 4) * 4)
        ev = torch.cuda.Event()
        ev.record()
        h["done"] = ev
        if npairs:
            _lib.pa_copy_blocks(self.k_cache, self.v_cache, self.pr[:npairs])
        self.last_pairs = npairs
        _lib.pa_decode_append(out, q, k_new, v_new, self.k_cache, self.v_cache, self.bt[:b], self.cl[:b],
                              int(cl.max()), self.scale, workspace=self.workspace)
