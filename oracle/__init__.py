"""CPU oracle for paged-KV decode: plain, slow, float64, written from the pages.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import, call or execute anything in
this package.  It shares no code with the GPU library and imports nothing
from it; the two meet only through the seeded inputs of ``pa_workloads``.
"""
from .block_manager_ref import BlockManagerRef, pages_for_tokens
from .cache_ops import cache_write_autoscale_ref, cache_write_ref, copy_blocks_ref, quantize_pool_ref
from .formats import (E4M3_MAX, bf16_to_f32, bf16_to_f64, e4m3_encode, e4m3_quantize, e4m3_table,
                      e4m3_to_f64, e4m3_value, int4_encode, int4_pack, int4_quantize, int4_to_f64, int4_unpack)
from .paged_attention import (attend, decode_partitioned_ref, decode_ref, gather_kv, lse_merge_ref,
                              multi_query_ref, partition_stats, to_f64)
from .sizes import decode_algorithmic_bytes, internal_waste_tokens, kv_bytes, pages_for, physical_kv_bytes

__all__ = [
    "BlockManagerRef", "pages_for_tokens",
    "cache_write_autoscale_ref", "cache_write_ref", "copy_blocks_ref", "quantize_pool_ref", "E4M3_MAX", "bf16_to_f32",
    "bf16_to_f64", "e4m3_encode", "e4m3_quantize", "e4m3_table", "e4m3_to_f64", "e4m3_value",
    "int4_encode", "int4_pack", "int4_quantize", "int4_to_f64", "int4_unpack",
    "attend", "decode_partitioned_ref", "decode_ref", "gather_kv", "lse_merge_ref", "multi_query_ref",
    "partition_stats", "to_f64", "decode_algorithmic_bytes", "internal_waste_tokens", "kv_bytes",
    "pages_for", "physical_kv_bytes",
]
