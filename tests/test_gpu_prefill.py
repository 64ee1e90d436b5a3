"""GPU parity of the causal multi-query (prefill) call against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_paged_06_amd import paged_attention_decode, paged_attention_prefill
from gpu_util import TOL, compare, device
from workloads import prefill_inputs, raw_bits, raw_u16

pytestmark = pytest.mark.gpu


def run_prefill(inp, q, qs, max_q, partition_size=0):
    out = torch.full_like(q, float("nan"))
    paged_attention_prefill(out, q, inp.key_cache, inp.value_cache, inp.block_tables,
                            inp.context_lens, qs, max_q, inp.scale, inp.block_size,
                            inp.alibi_slopes, partition_size=partition_size,
                            k_scale=inp.k_scale, v_scale=inp.v_scale)
    torch.cuda.synchronize()
    return out


def ref_prefill(inp, q, qs):
    slopes = None if inp.alibi_slopes is None else inp.alibi_slopes.cpu().numpy()
    return oracle.paged_prefill(raw_u16(q), raw_bits(inp.key_cache), raw_bits(inp.value_cache),
                                inp.block_tables.cpu().numpy(), inp.context_lens.cpu().numpy(),
                                qs.cpu().numpy(), inp.scale, inp.block_size, slopes,
                                dtype=inp.dtype, k_scale=inp.k_scale, v_scale=inp.v_scale)


CASES = [
    # (name, heads, kv heads, head size, dtype, block, lengths, new tokens, alibi, kv dtype)
    ("gqa-prefix", 16, 2, 128, "bf16", 16, [40, 300, 17, 129], [7, 64, 17, 1], True, None),
    ("mha-fresh", 4, 4, 64, "f16", 16, [33, 70, 5], [33, 70, 5], False, None),
    ("mqa-48", 48, 1, 128, "f16", 16, [100, 260], [20, 3], True, None),
    ("gqa-block8", 16, 2, 128, "bf16", 8, [50, 9, 200], [50, 2, 31], True, None),
    ("gqa-block64", 8, 1, 64, "f16", 64, [65, 300], [1, 128], False, None),
    ("fp8-cache", 16, 2, 128, "bf16", 16, [90, 257], [45, 100], True, "fp8"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_prefill_parity(case):
    dev = device()
    name, Hq, Hkv, D, dtype, BS, lens, news, alibi, kvd = case
    inp, q, qs, max_q = prefill_inputs(new_tokens=news, seed=len(name) + sum(news), device=dev,
                                       num_seqs=len(lens), num_heads=Hq, num_kv_heads=Hkv,
                                       head_size=D, block_size=BS, dtype=dtype,
                                       context_lens=lens, alibi=alibi, poison=True, kv_dtype=kvd)
    ref = ref_prefill(inp, q, qs)
    for ps in (-1, 0, max(BS, 64)):
        compare(run_prefill(inp, q, qs, max_q, ps), ref, dtype, what=f"{name} partition={ps}")


def test_prefill_one_token_matches_decode():
    dev = device()
    lens = [1, 50, 300, 1000]
    inp, q, qs, max_q = prefill_inputs(new_tokens=[1] * 4, seed=5, device=dev, num_seqs=4,
                                       num_heads=64, num_kv_heads=8, head_size=128,
                                       block_size=16, dtype="bf16", context_lens=lens,
                                       alibi=True, poison=True)
    a = run_prefill(inp, q, qs, max_q)
    b = torch.empty_like(q)
    paged_attention_decode(b, q, inp.key_cache, inp.value_cache, inp.block_tables,
                           inp.context_lens, inp.scale, 16, inp.alibi_slopes)
    torch.cuda.synchronize()
    assert float((a.float() - b.float()).abs().max()) <= TOL["bf16"]
    compare(a, ref_prefill(inp, q, qs), "bf16", what="prefill n=1")


def test_prefill_empty_sequences_and_chunk():
    """Sequences with no new tokens produce no rows; a long chunk spans many row tiles."""
    dev = device()
    lens = [64, 2000, 10, 700]
    news = [0, 300, 0, 77]
    inp, q, qs, max_q = prefill_inputs(new_tokens=news, seed=9, device=dev, num_seqs=4,
                                       num_heads=32, num_kv_heads=4, head_size=128,
                                       block_size=16, dtype="bf16", context_lens=lens,
                                       poison=True)
    ref = ref_prefill(inp, q, qs)
    for ps in (0, 256):
        compare(run_prefill(inp, q, qs, max_q, ps), ref, "bf16", what=f"chunk partition={ps}")


def test_prefill_table_window():
    """A partition longer than the block-table window the staged loop keeps in
    LDS (512 entries): 8-token blocks, 5000 + tokens of context, one pass."""
    dev = device()
    lens = [5000, 4203]
    news = [37, 6]
    inp, q, qs, max_q = prefill_inputs(new_tokens=news, seed=13, device=dev, num_seqs=2,
                                       num_heads=16, num_kv_heads=2, head_size=64,
                                       block_size=8, dtype="f16", context_lens=lens,
                                       alibi=True, poison=True)
    ref = ref_prefill(inp, q, qs)
    for ps in (-1, 0, 4096):
        compare(run_prefill(inp, q, qs, max_q, ps), ref, "f16", what=f"window partition={ps}")


@pytest.mark.parametrize("kv", [None, "fp8"])
def test_prefill_bench_shape_sampled(kv):
    """The multi-query shape bench.py times (GQA 64/8 bf16, 4 sequences x 512 new
    tokens on 4096 context, automatic plan), checked on sampled rows: a new token's
    rows equal decode of that token over the context cut at its position (an
    identity the oracle's own pins check), so the fp64 decode oracle serves."""
    dev = device()
    S, L, n = 4, 4096, 512
    inp, q, qs, max_q = prefill_inputs(new_tokens=[n] * S, seed=77, device=dev, num_seqs=S,
                                       num_heads=64, num_kv_heads=8, head_size=128,
                                       block_size=16, dtype="bf16", context_lens=L, kv_dtype=kv)
    out = run_prefill(inp, q, qs, max_q)
    rng = np.random.default_rng(5)
    picks = [(s, i) for s in range(S) for i in (0, n - 1, int(rng.integers(1, n - 1)))]
    starts = qs.cpu().numpy()
    rows = [int(starts[s]) + i for s, i in picks]
    tables = inp.block_tables.cpu().numpy()[[s for s, _ in picks]]
    lens = np.array([L - n + i + 1 for _, i in picks], dtype=np.int64)
    ref = oracle.paged_decode(raw_u16(q[rows]), raw_bits(inp.key_cache), raw_bits(inp.value_cache),
                              tables, lens, inp.scale, inp.block_size, None, dtype="bf16",
                              k_scale=inp.k_scale, v_scale=inp.v_scale)
    compare(out[rows], ref, "bf16", what=f"prefill bench shape ({kv or 'bf16'} cache), sampled rows")


# Calls on 32 x 32 matrix tiles: head size 128, 16-bit caches, blocks of at
# least 16 tokens (the dispatch rule of the library).  Row chunks of 128 rows
# with a group that does not divide them, ragged tails, several cache block
# sizes (a block holds 1, 2 or 16 of the kernel's 16-row tiles), ALiBi, and
# forced single-pass and split plans.
P32_CASES = [
    # (name, heads, kv heads, dtype, block, lengths, new tokens, alibi)
    ("p32-gqa-bs16-alibi", 16, 2, "bf16", 16, [300, 1000, 77], [129, 300, 77], True),
    ("p32-bs32-f16", 32, 4, "f16", 32, [513, 64], [200, 64], False),
    ("p32-bs256", 8, 1, "bf16", 256, [700, 2100], [150, 33], True),
    ("p32-mqa48", 48, 1, "bf16", 16, [400, 45], [100, 45], True),
    ("p32-g12-f16-bs128-alibi", 24, 2, "f16", 128, [1500, 257, 3000], [400, 257, 64], True),
]


@pytest.mark.parametrize("case", P32_CASES, ids=[c[0] for c in P32_CASES])
def test_prefill32_parity(case):
    dev = device()
    name, Hq, Hkv, dtype, BS, lens, news, alibi = case
    inp, q, qs, max_q = prefill_inputs(new_tokens=news, seed=len(name) + sum(lens), device=dev,
                                       num_seqs=len(lens), num_heads=Hq, num_kv_heads=Hkv,
                                       head_size=128, block_size=BS, dtype=dtype,
                                       context_lens=lens, alibi=alibi, poison=True)
    ref = ref_prefill(inp, q, qs)
    for ps in (-1, 0, max(BS, 256)):
        compare(run_prefill(inp, q, qs, max_q, ps), ref, dtype, what=f"{name} partition={ps}")


@pytest.mark.parametrize("BS", [16, 64])
def test_prefill32_window_refill(BS):
    """One pass over more than the 512 tiles (8192 tokens) whose source offsets
    the kernel keeps in LDS at a time, so the window is refilled mid-loop."""
    dev = device()
    lens = [9000, 8450]
    news = [33, 3]
    inp, q, qs, max_q = prefill_inputs(new_tokens=news, seed=21 + BS, device=dev, num_seqs=2,
                                       num_heads=8, num_kv_heads=1, head_size=128,
                                       block_size=BS, dtype="bf16", context_lens=lens,
                                       alibi=True, poison=True)
    ref = ref_prefill(inp, q, qs)
    for ps in (-1, 0):
        compare(run_prefill(inp, q, qs, max_q, ps), ref, "bf16", what=f"refill BS={BS} partition={ps}")


def test_prefill32_full_causal_sampled():
    """One sequence whose whole 4096-token context is new (a full causal
    prefill: 256 row chunks per kv head, up to 128 steps each, longest chunks
    first), on the 32 x 32 kernel under the automatic plan; sampled rows are
    checked through the fp64 decode oracle on the context cut at each row's
    position."""
    dev = device()
    L = n = 4096
    inp, q, qs, max_q = prefill_inputs(new_tokens=[n], seed=4096, device=dev, num_seqs=1,
                                       num_heads=64, num_kv_heads=8, head_size=128,
                                       block_size=16, dtype="bf16", context_lens=L, alibi=True)
    out = run_prefill(inp, q, qs, max_q)
    rows = [0, 1, 15, 16, 31, 32, 127, 128, 2047, 2048, 4094, 4095]
    tables = inp.block_tables.cpu().numpy()[[0] * len(rows)]
    lens = np.array([r + 1 for r in rows], dtype=np.int64)
    ref = oracle.paged_decode(raw_u16(q[rows]), raw_bits(inp.key_cache), raw_bits(inp.value_cache),
                              tables, lens, inp.scale, inp.block_size, inp.alibi_slopes.cpu().numpy(),
                              dtype="bf16", k_scale=inp.k_scale, v_scale=inp.v_scale)
    compare(out[rows], ref, "bf16", what="full causal prefill 4096, sampled rows")
