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
    kHostSets = 8
    kEventEvery = 4
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
        # used prefix to the device copy of the same layout.  kHostSets pinned
        # host buffers are used in turn; a buffer is refilled only after the
        # upload that read it has finished.  That is known from an event
        # recorded after every kEventEvery-th upload (an event between two
        # kernels costs the stream a few microseconds, so not every step
        # records one): the one recorded at or after the buffer's last use.
        r16 = lambda n: (n + 3) // 4 * 4  # int32 elements to a multiple of 16 bytes
        self._off_pr = r16(max_batch)
        self._off_bt = self._off_pr + r16(2 * max_batch)
        self._words = self._off_bt + r16(max_batch * max_blocks_per_seq)
        self._host = []
        for _ in range(self.kHostSets):
            buf = torch.zeros(self._words, dtype=torch.int32).pin_memory()
            self._host.append({
                "buf": buf,
                "views": self._views(buf),
                "sl": torch.zeros(max_batch, dtype=torch.int64).pin_memory(),
            })
        # slot mappings of admitted prompts: two pinned staging buffers in turn
        # (each reused once the upload that read it has finished), one device copy
        max_tokens = max_blocks_per_seq * BLOCK_SIZE
        self._slot_stage = [torch.zeros(max_tokens + 1, dtype=torch.int64).pin_memory() for _ in range(2)]
        self._slot_event = [torch.cuda.Event() for _ in range(2)]
        self._slot_used = [False, False]
        self._slot_turn = 0
        self._slots_dev = torch.zeros(max_tokens + 1, dtype=torch.int64, device=self.device)
        self._pos = np.arange(max_tokens, dtype=np.int64)
        self._events = [torch.cuda.Event() for _ in range(3)]
        self._event_step = [-1] * 3      # the step whose upload each event follows
        self._step_no = 0
        self._dev = torch.zeros(self._words, dtype=torch.int32, device=self.device)
        self.cl, self.pr, self.bt = self._views(self._dev)
        ws = _lib.pa_decode_workspace_size(max_batch, num_q_heads, num_kv_heads, head_dim,
                                           max_blocks_per_seq * BLOCK_SIZE, 0)
        self.workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=self.device)
        self.last_pairs = 0
        # marshalled pa_decode_append arguments per (batch, caller tensors, stream):
        # validated on first use; only max_context_len changes between steps
        self._calls = {}

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
        if n > self._pos.size:
            raise ValueError("prompt longer than max_blocks_per_seq * 16 tokens")
        table, _ = self.bm.table(seq)
        turn = self._slot_turn
        self._slot_turn ^= 1
        if self._slot_used[turn]:
            self._slot_event[turn].synchronize()
        pos = self._pos[:n]
        stage = self._slot_stage[turn].numpy()
        np.add(table[pos // BLOCK_SIZE].astype(np.int64) * BLOCK_SIZE, pos % BLOCK_SIZE, out=stage[:n])
        stream = torch.cuda.current_stream(self.device)
        _lib.pa_upload(self._slots_dev, self._slot_stage[turn], (n * 8 + 15) // 16 * 16, stream=stream.cuda_stream)
        self._slot_event[turn].record(stream)
        self._slot_used[turn] = True
        _lib.pa_cache_write(k, v, self.k_cache, self.v_cache, self._slots_dev[:n], stream=stream.cuda_stream)

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
        t = self._step_no
        h = self._host[t % self.kHostSets]
        if t >= self.kHostSets:
            # the upload of step t - kHostSets read this buffer: wait for the
            # first event recorded after it (one of the last three)
            need = t - self.kHostSets
            k = min((k for k in range(3) if self._event_step[k] >= need), key=lambda k: self._event_step[k])
            self._events[k].synchronize()
        hcl, hpr, hbt = h["views"]
        bt, cl, _, pr = self.bm.step(seqs, self.mb, out=(hbt.numpy(), hcl.numpy(), h["sl"].numpy(), hpr.numpy()))
        npairs = len(pr)
        stream = torch.cuda.current_stream(self.device)
        sh = stream.cuda_stream
        _lib.pa_upload(self._dev, h["buf"], (self._off_bt + (b * self.mb + 3) // 4 * 4) * 4, stream=sh)
        if t % self.kEventEvery == self.kEventEvery - 1:
            k = (t // self.kEventEvery) % 3
            self._events[k].record(stream)
            self._event_step[k] = t
        self._step_no = t + 1
        if npairs:
            _lib.pa_copy_blocks(self.k_cache, self.v_cache, self.pr[:npairs], stream=sh)
        self.last_pairs = npairs
        key = (b, sh, q.dtype, tuple(q.shape), tuple(k_new.shape), tuple(out.shape), q.data_ptr(), k_new.data_ptr(),
               v_new.data_ptr(), out.data_ptr())
        args = self._calls.get(key)
        if args is None:
            args, _ = _lib._decode_append_args(out, q, k_new, v_new, self.k_cache, self.v_cache, self.bt[:b],
                                               self.cl[:b], self.mb * BLOCK_SIZE, self.scale, None, None, 0,
                                               self.workspace, sh)
            args = list(args)
            self._calls[key] = args
        args[13] = int(cl.max())          # max_context_len
        _lib.check_status(_lib.raw_call("pa_decode_append", *args), "pa_decode_append")
