"""Seeded synthetic inputs for paged-KV decode (shared by the oracle tests and the GPU path).

Holds no attention arithmetic: only random draws, pool layout and block
bookkeeping.
"""
from .block_manager import (BLOCK_SIZE, BlockManager, OutOfBlocks, blocks_needed,
                            validate_copy_pairs, validate_slots, validate_tables)
from .configs import (CONFIGS, ELEM_BYTES, PagedWorkload, config1, config2, config3, config4,
                      config5, make_multi_query_workload, make_shared_prefix_workload, make_workload)

__all__ = [
    "BLOCK_SIZE", "BlockManager", "OutOfBlocks", "blocks_needed", "validate_copy_pairs",
    "validate_slots", "validate_tables", "CONFIGS", "ELEM_BYTES", "PagedWorkload", "config1",
    "config2", "config3", "config4", "config5", "make_multi_query_workload", "make_shared_prefix_workload",
    "make_workload",
]
