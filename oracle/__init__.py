"""CPU oracle (test infrastructure only; never imported by the product path)."""
from .paged_attention import (alibi_bias, attend, fp8_e4m3_value, fp8_to_float64, gather_cached_kv,
                              kv_cache_write, kv_head_of,
                              merge_partitions,
                              paged_decode, paged_decode_partitioned, paged_prefill,
                              partition_stats,
                              round_to_storage, sequence_kv, to_float64)

__all__ = [
    "alibi_bias", "attend", "fp8_e4m3_value", "fp8_to_float64", "gather_cached_kv", "kv_cache_write", "kv_head_of", "merge_partitions",
    "paged_decode", "paged_decode_partitioned", "paged_prefill", "partition_stats", "round_to_storage",
    "sequence_kv", "to_float64",
]
