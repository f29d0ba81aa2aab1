"""ctypes binding of libpa (include/pa.h): argument marshalling only.

Every step of the decode runs in the library's HIP kernels; this module
turns torch tensors into device pointers, sizes and dtype codes, passes the
current HIP stream, and raises ``PaError`` on a non-zero status.  There is
no fallback: if ``libpa.so`` is missing, importing this module fails.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")

PA_DTYPE_F32, PA_DTYPE_BF16, PA_DTYPE_FP8_E4M3, PA_DTYPE_INT4 = 0, 1, 2, 3
BLOCK_SIZE = 16


class PaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {pa_status_string(status)} (status {status})")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m paged_kv_cache_272_amd.build` "
                          "(or __graft_entry__.build()) first")
    return ctypes.CDLL(LIB_PATH)


_lib = _load()

_vp, _i32, _i64, _sz, _f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float

PA_PLAN_SHARE_PREFIX = 1
PA_ERR_OUT_OF_BLOCKS = -8


class BmStats(ctypes.Structure):
    """pa_bm_stats (include/pa.h)."""
    _fields_ = [("num_blocks", _i32), ("free_blocks", _i32), ("num_seqs", _i32), ("reserved", _i32),
                ("logical_tokens", _i64), ("block_refs", _i64), ("stored_tokens", _i64)]


class PlanInfo(ctypes.Structure):
    """pa_plan_info (include/pa.h)."""
    _fields_ = [("num_seqs", _i32), ("num_q_tokens", _i32), ("num_q_heads", _i32), ("num_kv_heads", _i32),
                ("head_dim", _i32), ("num_items", _i32), ("num_columns", _i32), ("num_records", _i32),
                ("num_merge_rows", _i32), ("num_merge_entries", _i32), ("num_shared_groups", _i32),
                ("num_wgs", _i32), ("max_item_columns", _i32), ("num_wide_groups", _i32), ("plan_bytes", _i64),
                ("workspace_bytes", _i64), ("block_reads", _i64)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_ if name != "reserved"}

_SIGNATURES = {
    "pa_cache_write": (ctypes.c_int, [_vp, _vp, ctypes.c_int, _vp, _vp, ctypes.c_int, _vp, _vp, _vp,
                                      _i32, _i32, _i32, _i32, _vp]),
    "pa_cache_write_autoscale": (ctypes.c_int, [_vp, _vp, ctypes.c_int, _vp, _vp, ctypes.c_int, _vp, _vp, _vp,
                                                _i32, _i32, _i32, _i32, _vp]),
    "pa_decode_partition_tokens": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_decode_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_decode": (ctypes.c_int, [_vp, _vp, ctypes.c_int, _vp, _vp, ctypes.c_int, _vp, _vp, _vp, _i32,
                                 _vp, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _sz, _vp]),
    "pa_decode_append": (ctypes.c_int, [_vp, _vp, ctypes.c_int, _vp, _vp, _vp, _vp, ctypes.c_int, _vp, _vp, _vp,
                                        _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _sz, _vp]),
    "pa_decode_noalloc": (ctypes.c_int, [_vp, _vp, ctypes.c_int, _vp, _vp, ctypes.c_int, _vp, _vp, _vp, _i32,
                                         _vp, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp]),
    "pa_copy_blocks": (ctypes.c_int, [_vp, _vp, ctypes.c_int, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp]),
    "pa_upload": (ctypes.c_int, [_vp, _vp, _sz, _vp]),
    "pa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pa_timing_enable": (ctypes.c_int, [ctypes.c_int]),
    "pa_timing_read": (ctypes.c_int, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double),
                                      ctypes.POINTER(_i64)]),
    "pa_plan_attention": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _sz,
                                         ctypes.POINTER(PlanInfo)]),
    "pa_attend_planned": (ctypes.c_int, [_vp, _vp, ctypes.c_int, _vp, _vp, ctypes.c_int, _vp, _vp, _vp, _i32, _i32,
                                         _f32, _vp, ctypes.POINTER(PlanInfo), _vp, _sz, _vp]),
    "pa_bm_create": (_vp, [_i32, _vp]),
    "pa_bm_destroy": (None, [_vp]),
    "pa_bm_add": (ctypes.c_int, [_vp, _i32, _i32]),
    "pa_bm_fork": (ctypes.c_int, [_vp, _i32, _i32]),
    "pa_bm_free": (ctypes.c_int, [_vp, _i32]),
    "pa_bm_append": (ctypes.c_int, [_vp, _i32, ctypes.POINTER(_i64), ctypes.POINTER(_i32), ctypes.POINTER(_i32)]),
    "pa_bm_table": (ctypes.c_int, [_vp, _i32, _vp, _i32, ctypes.POINTER(_i32), ctypes.POINTER(_i64)]),
    "pa_bm_get_stats": (ctypes.c_int, [_vp, ctypes.POINTER(BmStats)]),
    "pa_bm_step": (ctypes.c_int, [_vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp, ctypes.POINTER(_i32),
                                  ctypes.POINTER(_i32)]),
    "pa_probe_sink_bytes": (_sz, []),
    "pa_probe_stream_read": (ctypes.c_int, [_vp, _sz, _vp, _vp]),
    "pa_probe_copy": (ctypes.c_int, [_vp, _vp, _sz, _vp]),
}
for _name, (_res, _args) in _SIGNATURES.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = tuple(_SIGNATURES)


def pa_status_string(status: int) -> str:
    return _lib.pa_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise PaError(status, where)


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return PA_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return PA_DTYPE_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return PA_DTYPE_FP8_E4M3
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def cache_code(cache: torch.Tensor, head_dim: int) -> int:
    """dtype code of a K/V pool: a byte pool whose rows hold head_dim / 2 bytes is int4."""
    if cache.dtype == torch.uint8 and cache.shape[-1] * 2 == head_dim:
        return PA_DTYPE_INT4
    return dtype_code(cache)


def _row(cache: torch.Tensor, head_dim: int) -> int:
    """Logical head_dim of a pool (int4 pools hold two values per byte)."""
    return cache.shape[-1] * 2 if cache_code(cache, head_dim) == PA_DTYPE_INT4 else cache.shape[-1]


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libpa takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libpa takes contiguous tensors")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _scratch(nbytes: int, device, stream) -> torch.Tensor:
    """Scratch that a wrapper allocates for one call.  torch's caching
    allocator may hand the memory out again once the tensor is released,
    to work ordered after it on the *current* stream only; when the call
    runs on another stream, the tensor is marked as used there so that the
    memory is not reused before that stream's kernels are done with it."""
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if stream is not None:
        s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(
            _stream(stream), device=ws.device)
        if s.cuda_stream != torch.cuda.current_stream(ws.device).cuda_stream:
            ws.record_stream(s)
    return ws


def pa_cache_write(k: torch.Tensor, v: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   slot_mapping: torch.Tensor, k_scale: Optional[torch.Tensor] = None,
                   v_scale: Optional[torch.Tensor] = None, stream=None) -> None:
    """k, v [T, Hkv, D]; caches [NB, Hkv, 16, D]; slot_mapping [T] int64."""
    if slot_mapping.dtype != torch.int64:
        raise TypeError("slot_mapping must be int64")
    num_blocks, hkv, bs, _ = k_cache.shape
    d = k.shape[-1]
    if bs != BLOCK_SIZE or tuple(k.shape) != (k.shape[0], hkv, _row(k_cache, d)) or k.shape != v.shape:
        raise ValueError("shape mismatch between new K/V and the cache")
    _check(_lib.pa_cache_write(_ptr(k), _ptr(v), dtype_code(k), _ptr(k_cache), _ptr(v_cache),
                               cache_code(k_cache, d), _ptr(k_scale), _ptr(v_scale), _ptr(slot_mapping),
                               k.shape[0], hkv, d, num_blocks, _stream(stream)), "pa_cache_write")


def pa_cache_write_autoscale(k: torch.Tensor, v: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                             k_scale: torch.Tensor, v_scale: torch.Tensor, slot_mapping: torch.Tensor,
                             stream=None) -> None:
    """Slot scatter into an e4m3 or int4 cache (uint8 pools; int4 rows hold D/2
    bytes) that sets the (block, head) scales itself: k_scale/v_scale
    [NB, Hkv] float32 are read and written."""
    if slot_mapping.dtype != torch.int64:
        raise TypeError("slot_mapping must be int64")
    num_blocks, hkv, bs, _ = k_cache.shape
    d = k.shape[-1]
    if bs != BLOCK_SIZE or tuple(k.shape) != (k.shape[0], hkv, _row(k_cache, d)) or k.shape != v.shape:
        raise ValueError("shape mismatch between new K/V and the cache")
    _check(_lib.pa_cache_write_autoscale(_ptr(k), _ptr(v), dtype_code(k), _ptr(k_cache), _ptr(v_cache),
                                         cache_code(k_cache, d), _ptr(k_scale), _ptr(v_scale), _ptr(slot_mapping),
                                         k.shape[0], hkv, d, num_blocks, _stream(stream)), "pa_cache_write_autoscale")


def pa_decode_partition_tokens(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                               max_context_len: int, partition_tokens: int = 0) -> int:
    p = _lib.pa_decode_partition_tokens(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                                        partition_tokens)
    if p < 0:
        raise PaError(p, "pa_decode_partition_tokens")
    return p


def pa_decode_workspace_size(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                             max_context_len: int, partition_tokens: int = 0) -> int:
    return int(_lib.pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                             max_context_len, partition_tokens))


def pa_decode(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
              block_tables: torch.Tensor, context_lens: torch.Tensor, max_context_len: int, scale: float,
              k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None,
              partition_tokens: int = 0, workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """out, q [B, Hq, D]; caches [NB, Hkv, 16, D]; block_tables [B, MB] int32; context_lens [B] int32.

    If the call needs scratch and ``workspace`` is None, a byte tensor of
    pa_decode_workspace_size() bytes is allocated on q's device.  The
    workspace needs no initialisation: every byte the merge reads was
    written by the same call.
    """
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    b, hq, d = q.shape
    num_blocks, hkv, bs, _ = k_cache.shape
    if bs != BLOCK_SIZE or _row(k_cache, d) != d or tuple(out.shape) != (b, hq, d) or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch among q, out and the caches")
    mb = block_tables.shape[1]
    need = pa_decode_workspace_size(b, hq, hkv, d, max_context_len, partition_tokens)
    if workspace is None and need:
        workspace = _scratch(need, q.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.pa_decode(_ptr(out), _ptr(q), dtype_code(q), _ptr(k_cache), _ptr(v_cache),
                          cache_code(k_cache, d), _ptr(k_scale), _ptr(v_scale), _ptr(block_tables), mb,
                          _ptr(context_lens), int(max_context_len), b, hq, hkv, d, num_blocks, float(scale),
                          int(partition_tokens), _ptr(workspace), ws_bytes, _stream(stream)), "pa_decode")


def pa_decode_noalloc(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      block_tables: torch.Tensor, context_lens: torch.Tensor, max_context_len: int, scale: float,
                      k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None,
                      partition_tokens: int = 0, stream=None) -> None:
    """pa_decode with the library's static scratch (allocates nothing; see include/pa.h)."""
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    b, hq, d = q.shape
    num_blocks, hkv, bs, _ = k_cache.shape
    if bs != BLOCK_SIZE or _row(k_cache, d) != d or tuple(out.shape) != (b, hq, d) or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch among q, out and the caches")
    _check(_lib.pa_decode_noalloc(_ptr(out), _ptr(q), dtype_code(q), _ptr(k_cache), _ptr(v_cache),
                                  cache_code(k_cache, d), _ptr(k_scale), _ptr(v_scale), _ptr(block_tables),
                                  block_tables.shape[1], _ptr(context_lens), int(max_context_len), b, hq, hkv, d,
                                  num_blocks, float(scale), int(partition_tokens), _stream(stream)),
           "pa_decode_noalloc")


# PA_DECODE_NOALLOC_MAX_WORKSPACE (include/pa.h): bytes of pa_decode_noalloc's static scratch
PA_DECODE_NOALLOC_MAX_WORKSPACE = 64 << 20


def _decode_append_args(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, max_context_len, scale,
                        k_scale, v_scale, partition_tokens, workspace, stream):
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    b, hq, d = q.shape
    num_blocks, hkv, bs, _ = k_cache.shape
    if bs != BLOCK_SIZE or _row(k_cache, d) != d or tuple(out.shape) != (b, hq, d) or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch among q, out and the caches")
    if tuple(k_new.shape) != (b, hkv, d) or k_new.shape != v_new.shape or k_new.dtype != q.dtype:
        raise ValueError("k_new/v_new must be [num_seqs, num_kv_heads, head_dim] in q's dtype")
    need = pa_decode_workspace_size(b, hq, hkv, d, max_context_len, partition_tokens)
    if workspace is None and need:
        workspace = _scratch(need, q.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(out), _ptr(q), dtype_code(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
            cache_code(k_cache, d), _ptr(k_scale), _ptr(v_scale), _ptr(block_tables), block_tables.shape[1],
            _ptr(context_lens), int(max_context_len), b, hq, hkv, d, num_blocks, float(scale), int(partition_tokens),
            _ptr(workspace), ws_bytes, _stream(stream))
    return args, workspace


def pa_decode_append(out: torch.Tensor, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                     k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: torch.Tensor,
                     context_lens: torch.Tensor, max_context_len: int, scale: float,
                     k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None,
                     partition_tokens: int = 0, workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Write each sequence's newest token (k_new/v_new [B, Hkv, D], q's dtype) at position
    context_lens[b] - 1, then decode over the cache including it."""
    args, _ = _decode_append_args(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens,
                                  max_context_len, scale, k_scale, v_scale, partition_tokens, workspace, stream)
    _check(_lib.pa_decode_append(*args), "pa_decode_append")


def pa_copy_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor, block_pairs: torch.Tensor,
                   k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None,
                   stream=None, head_dim: Optional[int] = None) -> None:
    """block_pairs [n, 2] int32 (src, dst).  head_dim: needed to recognise an
    int4 pool (rows of head_dim / 2 bytes)."""
    if block_pairs.dtype != torch.int32:
        raise TypeError("block_pairs must be int32")
    num_blocks, hkv, bs, d = k_cache.shape
    code = dtype_code(k_cache)
    if head_dim is not None:
        code, d = cache_code(k_cache, head_dim), head_dim
    _check(_lib.pa_copy_blocks(_ptr(k_cache), _ptr(v_cache), code, _ptr(k_scale),
                               _ptr(v_scale), _ptr(block_pairs), block_pairs.shape[0], hkv, d, num_blocks,
                               _stream(stream)), "pa_copy_blocks")


def pa_upload(dst: torch.Tensor, src: torch.Tensor, nbytes: Optional[int] = None, stream=None) -> None:
    """Copy the first ``nbytes`` (default: all of ``src``) of a pinned host
    tensor into a device tensor with a kernel on ``stream``.  Both contiguous,
    16-byte aligned, ``nbytes`` a multiple of 16."""
    if src.is_cuda or not src.is_contiguous():
        raise ValueError("pa_upload: src must be a contiguous host tensor")
    n = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    if n > src.numel() * src.element_size() or n > dst.numel() * dst.element_size():
        raise ValueError("pa_upload: nbytes exceeds a buffer")
    _check(_lib.pa_upload(_ptr(dst), src.data_ptr(), n, _stream(stream)), "pa_upload")


def _host_i32(a, name: str) -> Optional[np.ndarray]:
    if a is None:
        return None
    if isinstance(a, torch.Tensor):
        if a.is_cuda:
            raise ValueError(f"{name}: the planner takes host arrays")
        a = a.numpy()
    return np.ascontiguousarray(a, dtype=np.int32)


def pa_plan_attention(context_lens, num_q_heads: int, num_kv_heads: int, head_dim: int, q_start=None,
                      block_tables=None, share_prefix: bool = False,
                      target_slices: int = 0) -> Tuple[np.ndarray, PlanInfo]:
    """Build a plan on the host (host int32 arrays).  Returns (plan bytes, info).

    q_start [B+1] (None: one new token per sequence); block_tables [B, MB]
    host copy (needed for share_prefix; its width is max_blocks_per_seq).
    """
    cl = _host_i32(context_lens, "context_lens")
    qs = _host_i32(q_start, "q_start")
    bt = _host_i32(block_tables, "block_tables")
    b = cl.shape[0]
    if qs is not None and qs.shape != (b + 1,):
        raise ValueError("q_start must have num_seqs + 1 entries")
    mb = bt.shape[1] if bt is not None else max(1, -(-int(cl.max(initial=0)) // BLOCK_SIZE))
    flags = PA_PLAN_SHARE_PREFIX if share_prefix else 0
    if share_prefix and bt is None:
        raise ValueError("share_prefix needs the host block tables")
    info = PlanInfo()
    args = [None if qs is None else qs.ctypes.data, cl.ctypes.data, None if bt is None else bt.ctypes.data, mb, b,
            num_q_heads, num_kv_heads, head_dim, flags, int(target_slices)]
    _check(_lib.pa_plan_attention(*args, None, 0, ctypes.byref(info)), "pa_plan_attention")
    plan = np.zeros(max(16, info.plan_bytes), dtype=np.uint8)
    _check(_lib.pa_plan_attention(*args, plan.ctypes.data, plan.nbytes, ctypes.byref(info)), "pa_plan_attention")
    return plan, info


def plan_to_device(plan: np.ndarray, device="cuda") -> torch.Tensor:
    """Copy a host plan to device memory (16-byte aligned, as the library requires)."""
    return torch.from_numpy(plan).to(device)


def pa_attend_planned(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      block_tables: torch.Tensor, scale: float, plan: torch.Tensor, info: PlanInfo,
                      k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """out, q [T, Hq, D] bf16; block_tables [B, MB] int32 (device); plan: device copy of the plan bytes."""
    if block_tables.dtype != torch.int32:
        raise TypeError("block_tables must be int32")
    num_blocks, hkv, bs, _ = k_cache.shape
    d = _row(k_cache, info.head_dim)
    if bs != BLOCK_SIZE or tuple(q.shape) != (info.num_q_tokens, info.num_q_heads, info.head_dim) \
            or out.shape != q.shape or hkv != info.num_kv_heads or d != info.head_dim:
        raise ValueError("tensor shapes do not match the plan")
    if workspace is None and info.workspace_bytes:
        workspace = _scratch(info.workspace_bytes, q.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.pa_attend_planned(_ptr(out), _ptr(q), dtype_code(q), _ptr(k_cache), _ptr(v_cache),
                                  cache_code(k_cache, info.head_dim), _ptr(k_scale), _ptr(v_scale), _ptr(block_tables),
                                  block_tables.shape[1], num_blocks, float(scale), _ptr(plan), ctypes.byref(info),
                                  _ptr(workspace), ws_bytes, _stream(stream)), "pa_attend_planned")


def prepare_attend_planned(out, q, k_cache, v_cache, block_tables, scale, plan, info, k_scale=None, v_scale=None,
                           workspace=None, stream=None) -> PreparedCall:
    num_blocks = k_cache.shape[0]
    if workspace is None and info.workspace_bytes:
        workspace = torch.empty(info.workspace_bytes, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(out), _ptr(q), dtype_code(q), _ptr(k_cache), _ptr(v_cache), cache_code(k_cache, info.head_dim),
            _ptr(k_scale), _ptr(v_scale), _ptr(block_tables), block_tables.shape[1], num_blocks, float(scale),
            _ptr(plan),
            ctypes.byref(info), _ptr(workspace), ws_bytes, _stream(stream))
    return PreparedCall("pa_attend_planned", args, (out, q, k_cache, v_cache, block_tables, k_scale, v_scale,
                                                    plan, info, workspace))


class OutOfBlocks(PaError):
    """The block pool cannot hold the request; ``blocks_short`` says by how much (steps only)."""

    def __init__(self, where: str, blocks_short: int = 0):
        super().__init__(PA_ERR_OUT_OF_BLOCKS, where)
        self.blocks_short = blocks_short


class HostBlockManager:
    """The library's host block manager (pa_bm_*): a pool of 16-token blocks,
    per-sequence tables, reference counts, copy-on-write and the
    continuous-batching step.  Host memory only."""

    def __init__(self, num_blocks: int, free_order=None):
        order = None if free_order is None else np.ascontiguousarray(free_order, dtype=np.int32)
        self._order = order
        self._h = _lib.pa_bm_create(int(num_blocks), None if order is None else order.ctypes.data)
        if not self._h:
            raise PaError(-2, "pa_bm_create")
        self.num_blocks = int(num_blocks)

    def __del__(self):
        if getattr(self, "_h", None):
            _lib.pa_bm_destroy(self._h)
            self._h = None

    def _call(self, name, *args):
        st = getattr(_lib, name)(self._h, *args)
        if st == PA_ERR_OUT_OF_BLOCKS:
            raise OutOfBlocks(name)
        _check(st, name)

    def add(self, seq: int, num_tokens: int) -> None:
        self._call("pa_bm_add", int(seq), int(num_tokens))

    def fork(self, parent: int, child: int) -> None:
        self._call("pa_bm_fork", int(parent), int(child))

    def free(self, seq: int) -> None:
        self._call("pa_bm_free", int(seq))

    def append(self, seq: int):
        """(slot of the new token, (src, dst) copy pair or None)."""
        slot, src, dst = _i64(), _i32(), _i32()
        self._call("pa_bm_append", int(seq), ctypes.byref(slot), ctypes.byref(src), ctypes.byref(dst))
        return slot.value, (None if src.value < 0 else (src.value, dst.value))

    def table(self, seq: int):
        """(block ids as an int32 array, token count)."""
        nb, nt = _i32(), _i64()
        self._call("pa_bm_table", int(seq), None, 0, ctypes.byref(nb), ctypes.byref(nt))
        out = np.zeros(max(nb.value, 1), dtype=np.int32)
        self._call("pa_bm_table", int(seq), out.ctypes.data, out.size, ctypes.byref(nb), ctypes.byref(nt))
        return out[:nb.value], nt.value

    def stats(self) -> dict:
        st = BmStats()
        _check(_lib.pa_bm_get_stats(self._h, ctypes.byref(st)), "pa_bm_get_stats")
        return {name: getattr(st, name) for name, _ in st._fields_ if name != "reserved"}

    def step(self, seqs, max_blocks_per_seq: int, out=None):
        """One decode iteration for ``seqs``: returns (block_tables [B, MB] int32,
        context_lens [B] int32, slot_mapping [B] int64, copy pairs [n, 2] int32).
        Raises OutOfBlocks (with ``blocks_short``) and changes nothing if the
        pool cannot hold the step.  ``out`` may pass preallocated host arrays
        (tables, lens, slots, pairs) to fill, e.g. pinned tensors' numpy views."""
        ids = np.ascontiguousarray(seqs, dtype=np.int32)
        b = ids.size
        if out is None:
            out = (np.zeros((b, max_blocks_per_seq), np.int32), np.zeros(b, np.int32), np.zeros(b, np.int64),
                   np.zeros((max(b, 1), 2), np.int32))
        bt, cl, sl, pr = out
        ncow, short = _i32(), _i32()
        st = _lib.pa_bm_step(self._h, ids.ctypes.data, b, int(max_blocks_per_seq), bt.ctypes.data, cl.ctypes.data,
                             sl.ctypes.data, pr.ctypes.data, ctypes.byref(ncow), ctypes.byref(short))
        if st == PA_ERR_OUT_OF_BLOCKS:
            raise OutOfBlocks("pa_bm_step", short.value)
        _check(st, "pa_bm_step")
        return bt[:b], cl[:b], sl[:b], pr[:ncow.value]


def pa_timing_enable(every: int = 1) -> None:
    """Record HIP events around the decode kernels of every `every`-th call (0 = off)."""
    _check(_lib.pa_timing_enable(int(every)), "pa_timing_enable")


def pa_timing_read() -> Tuple[float, float, int]:
    """(summed partition-kernel ms, summed merge-kernel ms, calls) since the last read."""
    p, m, n = ctypes.c_double(), ctypes.c_double(), ctypes.c_int64()
    _check(_lib.pa_timing_read(ctypes.byref(p), ctypes.byref(m), ctypes.byref(n)), "pa_timing_read")
    return p.value, m.value, n.value


def pa_probe_sink_bytes() -> int:
    return int(_lib.pa_probe_sink_bytes())


def pa_probe_stream_read(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    if sink.numel() * sink.element_size() < pa_probe_sink_bytes():
        raise ValueError("sink smaller than pa_probe_sink_bytes()")
    nbytes = buf.numel() * buf.element_size()
    _check(_lib.pa_probe_stream_read(_ptr(buf), nbytes - nbytes % 16, _ptr(sink), _stream(stream)),
           "pa_probe_stream_read")


def pa_probe_copy(dst: torch.Tensor, src: torch.Tensor, stream=None) -> None:
    nbytes = min(dst.numel() * dst.element_size(), src.numel() * src.element_size())
    _check(_lib.pa_probe_copy(_ptr(dst), _ptr(src), nbytes - nbytes % 16, _stream(stream)), "pa_probe_copy")


class PreparedCall:
    """A C-ABI call with its arguments marshalled once (fixed tensors, fixed
    stream), for tight loops where per-call Python work would dominate."""

    def __init__(self, name: str, args, keep):
        self._fn = getattr(_lib, name)
        self._name = name
        self._args = args
        self._keep = keep            # tensors whose pointers are baked into args

    def __call__(self) -> None:
        _check(self._fn(*self._args), self._name)


def prepare_cache_write(k, v, k_cache, v_cache, slot_mapping, k_scale=None, v_scale=None,
                        stream=None) -> PreparedCall:
    num_blocks, hkv, _, _ = k_cache.shape
    d = k.shape[-1]
    args = (_ptr(k), _ptr(v), dtype_code(k), _ptr(k_cache), _ptr(v_cache), cache_code(k_cache, d),
            _ptr(k_scale), _ptr(v_scale), _ptr(slot_mapping), k.shape[0], hkv, d, num_blocks, _stream(stream))
    return PreparedCall("pa_cache_write", args, (k, v, k_cache, v_cache, slot_mapping, k_scale, v_scale))


def prepare_decode(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len, scale,
                   k_scale=None, v_scale=None, partition_tokens=0, workspace=None,
                   stream=None) -> PreparedCall:
    b, hq, d = q.shape
    num_blocks, hkv, _, _ = k_cache.shape
    need = pa_decode_workspace_size(b, hq, hkv, d, max_context_len, partition_tokens)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(out), _ptr(q), dtype_code(q), _ptr(k_cache), _ptr(v_cache), cache_code(k_cache, d),
            _ptr(k_scale), _ptr(v_scale), _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
            int(max_context_len), b, hq, hkv, d, num_blocks, float(scale), int(partition_tokens),
            _ptr(workspace), ws_bytes, _stream(stream))
    return PreparedCall("pa_decode", args, (out, q, k_cache, v_cache, block_tables, context_lens, k_scale,
                                            v_scale, workspace))


def prepare_decode_append(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, max_context_len,
                          scale, k_scale=None, v_scale=None, partition_tokens=0, workspace=None,
                          stream=None) -> PreparedCall:
    args, workspace = _decode_append_args(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens,
                                          max_context_len, scale, k_scale, v_scale, partition_tokens, workspace,
                                          stream)
    return PreparedCall("pa_decode_append", args, (out, q, k_new, v_new, k_cache, v_cache, block_tables,
                                                   context_lens, k_scale, v_scale, workspace))


def check_status(status: int, where: str) -> None:
    """Raise PaError for a non-zero status of an entry point called through raw_call."""
    _check(status, where)


def raw_call(name: str, *args):
    """Call an exported entry point with raw ctypes arguments (for ABI tests)."""
    return getattr(_lib, name)(*args)
