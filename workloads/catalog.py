"""Named decode workloads (shapes, dtypes, length mixes, seeds).

Each entry describes one family of synthetic batches.  The shapes follow the
decode workloads the reference pages discuss: the LLaMA-13B-shaped MHA batch
of the shared-query-load change (vLLM PR #420), and the 64-query/8-KV-head
bf16 GQA kernel-latency tables of the FlashAttention-decode change (vLLM PR
#2744, "Kernel latency" tables for context_len 1024 and 4096).
"""
from __future__ import annotations

WORKLOADS = {
    # 4 sequences, lengths uniform on 1..64, MHA with 4 heads, D = 64, fp16,
    # tables drawn from a random permutation of a 64-block pool.
    "tiny_mha": dict(num_seqs=4, num_heads=4, num_kv_heads=4, head_size=64,
                     block_size=16, dtype="f16", context_lens=(1, 64),
                     pool_blocks=64, max_blocks_per_seq=4, alibi=False, seed_base=0,
                     batches=(4,)),
    # LLaMA-13B-shaped MHA: 40 heads, D = 128, batch 8, context 256, fp16,
    # 4096-block pool with shuffled tables.
    "llama13b_mha": dict(num_seqs=8, num_heads=40, num_kv_heads=40, head_size=128,
                         block_size=16, dtype="f16", context_lens=256,
                         pool_blocks=4096, alibi=False, seed_base=1000, batches=(8,)),
    # GQA 64 query heads / 8 KV heads, D = 128, bf16, context 1024.
    "gqa_ctx1024": dict(num_heads=64, num_kv_heads=8, head_size=128, block_size=16,
                        dtype="bf16", context_lens=1024, alibi=False, seed_base=2000,
                        batches=(1, 4, 16, 64, 256)),
    # Same at context 4096 (the long-context case that needs partitions at
    # small batch).
    "gqa_ctx4096": dict(num_heads=64, num_kv_heads=8, head_size=128, block_size=16,
                        dtype="bf16", context_lens=4096, alibi=False, seed_base=3000,
                        batches=(1, 4, 16, 64, 256)),
    # MQA, 48 query heads / 1 KV head, ragged lengths 64..8192, ALiBi slopes
    # 2^(-8 i / 48), fp16, batch 256 (and 32: fewer sequences than CUs).
    "mqa_ragged_alibi": dict(num_seqs=256, num_heads=48, num_kv_heads=1, head_size=128,
                             block_size=16, dtype="f16", context_lens=(64, 8192),
                             alibi=True, seed_base=4000, batches=(32, 256)),
}

# The headline measurement: GQA 64/8 bf16, context 4096, batch 256.
HEADLINE = ("gqa_ctx4096", 256)


def workload_args(name: str, batch: int) -> dict:
    """Keyword arguments for ``generate.decode_inputs`` for one (workload, batch)."""
    w = dict(WORKLOADS[name])
    w.pop("batches")
    seed = w.pop("seed_base") + batch
    w["num_seqs"] = batch
    w["seed"] = seed
    return w


def algorithmic_bytes(*, context_lens, num_heads, num_kv_heads, head_size, block_size,
                      elem_bytes=2, alibi=False, kv_elem_bytes=None) -> int:
    """Bytes a decode call must move at minimum.

    K and V of every valid token once per KV head (kv_elem_bytes each, 1 for an
    FP8 cache), q read and out written once,
    one table entry per used block, the context length of every sequence, and
    the ALiBi slopes when present.
    """
    lens = [int(x) for x in context_lens]
    S = len(lens)
    kv = sum(lens) * num_kv_heads * head_size * 2 * (kv_elem_bytes or elem_bytes)
    qo = 2 * S * num_heads * head_size * elem_bytes
    tables = 4 * sum((L + block_size - 1) // block_size for L in lens)
    return kv + qo + tables + 4 * S + (4 * num_heads if alibi else 0)


def algorithmic_flops(*, context_lens, num_heads, head_size) -> int:
    """QK and PV multiply-adds, two flops each."""
    return 4 * num_heads * head_size * sum(int(x) for x in context_lens)
