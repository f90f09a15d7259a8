"""CPU oracle for the paged-attention path.  TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It shares no code with the HIP library and imports nothing
from it.
"""
from .paged_attention import (BLOCK_SIZE, attend, blocks_needed, cascade_decode, decode, gather,
                              slot_mapping, swap_blocks, varlen_prefill, widen, write_kv)

__all__ = ["BLOCK_SIZE", "attend", "blocks_needed", "cascade_decode", "decode", "gather",
           "slot_mapping", "swap_blocks", "varlen_prefill", "widen", "write_kv"]
