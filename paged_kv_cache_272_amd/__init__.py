"""Paged-KV attention for AMD MI355X (gfx950): HIP kernels behind a C ABI (include/pa.h).

``import paged_kv_cache_272_amd`` loads the built ``libpa.so`` and fails if
it is missing; build it with ``python -m paged_kv_cache_272_amd.build``.
"""
from ._lib import (BLOCK_SIZE, EXPORTED, HostBlockManager, LIB_PATH, OutOfBlocks, PA_DTYPE_BF16, PA_DTYPE_F32,
                   PA_DTYPE_FP8_E4M3, PA_DTYPE_INT4, PA_PLAN_SHARE_PREFIX, PaError, PlanInfo, pa_attend_planned,
                   pa_cache_write, pa_cache_write_autoscale, pa_copy_blocks, pa_decode, pa_decode_append,
                   PA_DECODE_NOALLOC_MAX_WORKSPACE, pa_decode_noalloc, pa_decode_partition_tokens, pa_decode_workspace_size, pa_plan_attention, pa_probe_copy,
                   pa_probe_sink_bytes, pa_probe_stream_read, pa_status_string, pa_timing_enable, pa_timing_read,
                   pa_upload, plan_to_device, prepare_attend_planned, prepare_cache_write, prepare_decode,
                   prepare_decode_append)

__all__ = [
    "BLOCK_SIZE", "EXPORTED", "HostBlockManager", "LIB_PATH", "OutOfBlocks", "PA_DTYPE_BF16", "PA_DTYPE_F32",
    "PA_DTYPE_FP8_E4M3", "PA_DTYPE_INT4", "PA_PLAN_SHARE_PREFIX", "PaError", "PlanInfo", "pa_attend_planned",
    "pa_cache_write", "pa_cache_write_autoscale", "pa_copy_blocks", "pa_decode", "pa_decode_append",
    "PA_DECODE_NOALLOC_MAX_WORKSPACE", "pa_decode_noalloc", "pa_decode_partition_tokens", "pa_decode_workspace_size", "pa_plan_attention", "pa_probe_copy",
    "pa_probe_sink_bytes", "pa_probe_stream_read", "pa_status_string", "pa_timing_enable", "pa_timing_read",
    "pa_upload", "plan_to_device", "prepare_attend_planned", "prepare_cache_write", "prepare_decode", "prepare_decode_append",
]
