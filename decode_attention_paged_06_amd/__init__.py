"""Paged decode attention for AMD Instinct MI355X (gfx950).

The computation lives in the HIP kernels of ``libpagedattn.so`` behind the C
ABI of ``include/paged_attention.h``; this package only marshals arguments.
"""
from .ops import (gather_cached_kv, joint_kv_cache, kv_layout_of, make_dims, make_opts,
                  paged_attention_decode, paged_attention_decode_noalloc,
                  paged_attention_plan, paged_attention_prefill,
                  paged_attention_workspace_bytes, paged_kv_cache_write)

__all__ = ["gather_cached_kv", "joint_kv_cache", "kv_layout_of", "make_dims", "make_opts",
           "paged_attention_decode", "paged_attention_decode_noalloc", "paged_attention_plan",
           "paged_attention_prefill", "paged_attention_workspace_bytes", "paged_kv_cache_write"]
