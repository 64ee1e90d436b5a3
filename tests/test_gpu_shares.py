"""GPU tests of the equal-share schedule of the decode call (groups of more
than 16 heads on the LDS-staged kernel): every launched workgroup walks an
equal share of the batch's tiles across sequence (and kv head) boundaries,
and the reduce merges the pieces.  Checked against the fp64 oracle with the
parity gate on the sampled rows, across the staged configurations (2, 3 and 4
head tiles; head size 64 and 128; fp16, bf16 and FP8 caches; 8- to 256-token
blocks), on batches that put the cuts in awkward places (one sequence spread
over every workgroup, empty sequences, many short ones), and with needles at
the cuts themselves.
"""
import zlib

import numpy as np
import pytest
import torch

import needles
import share_bounds
from decode_attention_paged_06_amd import kv_layout_of, make_dims, make_opts, paged_attention_plan
from decode_attention_paged_06_amd.ops import share_occupancy
from gpu_util import compare, device, make, oracle_ref, run, sample_seqs
from workloads import workload_args

pytestmark = pytest.mark.gpu

SHARES = 3


def dims_of(inp):
    return make_dims(inp.query, inp.key_cache, inp.block_tables, inp.k_scale, inp.v_scale,
                     kv_layout_of(inp.key_cache, inp.value_cache))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("head_size", [64, 128])
@pytest.mark.parametrize("group", [32, 48, 64])
@pytest.mark.parametrize("kv", [None, "fp8"])
def test_share_occupancy(dtype, head_size, group, kv):
    """The planner's workgroups per CU (from the kernel's LDS) bound what the
    device holds of the compiled kernel; the launch takes the device's figure."""
    dev = device()
    inp = make(device_=dev, num_seqs=2, num_heads=group, num_kv_heads=1, head_size=head_size,
               block_size=16, dtype=dtype, seed=1, context_lens=64, kv_dtype=kv)
    table, occ, cost = share_occupancy(dims_of(inp))
    print(f"  G={group} D={head_size} {dtype} {kv}: table {table}, device {occ}, piece cost {cost}",
          flush=True)
    assert 1 <= occ <= table and cost >= 1


# (name, inputs): sizes the oracle finishes in seconds
CASES = {
    # 48-head MQA, ragged with ALiBi
    "g48_f16_alibi_ragged": dict(num_seqs=64, num_heads=48, num_kv_heads=1, head_size=128,
                                 block_size=16, dtype="f16", context_lens=(1, 6000), alibi=True),
    # two kv heads (items of both in one stream), 32-head groups, 32-token blocks
    "g32_bf16_hkv2_bs32": dict(num_seqs=24, num_heads=64, num_kv_heads=2, head_size=128,
                               block_size=32, dtype="bf16", context_lens=(0, 5000)),
    # 24-head groups (padded second tile), 256-token blocks, awkward lengths
    "g24_bf16_bs256": dict(num_seqs=7, num_heads=24, num_kv_heads=1, head_size=128, block_size=256,
                           dtype="bf16", context_lens=[0, 1, 17, 9000, 255, 256, 4097], alibi=True),
    # 64-head groups, head size 64, 8-token blocks (8-row tiles)
    "g64_f16_d64_bs8": dict(num_seqs=16, num_heads=64, num_kv_heads=1, head_size=64, block_size=8,
                            dtype="f16", context_lens=(0, 3000)),
    # one sequence spread over every workgroup
    "g48_one_sequence": dict(num_seqs=1, num_heads=48, num_kv_heads=1, head_size=128, block_size=16,
                             dtype="f16", context_lens=[12000], alibi=True),
    # one long sequence among short and empty ones
    "g48_unbalanced": dict(num_seqs=5, num_heads=48, num_kv_heads=1, head_size=128, block_size=16,
                           dtype="bf16", context_lens=[16384, 3, 0, 40, 1]),
    # fewer tiles than workgroups (73 tiles): some workgroups take no share
    "g48_fewer_tiles": dict(num_seqs=7, num_heads=48, num_kv_heads=1, head_size=128, block_size=16,
                            dtype="f16", context_lens=[1, 5, 16, 17, 100, 257, 700], alibi=True),
    "g64_fewer_tiles_fp8": dict(num_seqs=7, num_heads=64, num_kv_heads=1, head_size=128,
                                block_size=16, dtype="bf16", context_lens=[1, 5, 16, 17, 100, 257, 700],
                                kv_dtype="fp8"),
    "g32_fewer_tiles_hkv2": dict(num_seqs=3, num_heads=64, num_kv_heads=2, head_size=64, block_size=16,
                                 dtype="bf16", context_lens=[33, 0, 400], alibi=True),
    # many short sequences: shares of many items each
    "g48_many_short": dict(num_seqs=1500, num_heads=48, num_kv_heads=1, head_size=128, block_size=16,
                           dtype="f16", context_lens=(1, 200)),
    # FP8 caches (tile pairs in the staged ring), 32- and 64-head groups
    "g32_fp8_bf16": dict(num_seqs=12, num_heads=32, num_kv_heads=1, head_size=128, block_size=16,
                         dtype="bf16", context_lens=(0, 7000), kv_dtype="fp8", alibi=True),
    "g64_fp8_f16_d64": dict(num_seqs=9, num_heads=128, num_kv_heads=2, head_size=64, block_size=32,
                            dtype="f16", context_lens=(100, 4000), kv_dtype="fp8"),
}


@pytest.mark.parametrize("case", list(CASES))
def test_equal_shares_parity(case):
    dev = device()
    args = CASES[case]
    inp = make(device_=dev, seed=zlib.crc32(case.encode()) % 10000, poison=True, kv_layout="joint",
               **args)
    p = paged_attention_plan(dims_of(inp), 1 << 40, make_opts(0, "auto", schedule="equal_shares"))
    assert p.schedule == SHARES
    S = inp.query.shape[0]
    seqs = sample_seqs(S, 24, seed=5)
    ref = oracle_ref(inp, seqs)
    out = run(inp, schedule="equal_shares")
    assert torch.isfinite(out.float()).all(), f"{case}: non-finite output"
    compare(out, ref, inp.dtype, seqs, what=f"{case} equal shares")
    lens = inp.context_lens.cpu().numpy()
    for s in range(S):  # empty sequences: zero rows
        if lens[s] == 0:
            assert (out[s] == 0).all(), f"{case}: sequence {s} is empty but its row is not zero"
    # the partitioned schedule meets the same bar on the same rows
    compare(run(inp, schedule="longest_first"), ref, inp.dtype, seqs, what=f"{case} longest first")


def test_equal_shares_maximum_sizes():
    """The largest batch equal shares take (2048 sequences) and a 65536-token
    context spread over every workgroup."""
    dev = device()
    inp = make(device_=dev, num_seqs=2048, num_heads=48, num_kv_heads=1, head_size=128, block_size=16,
               dtype="bf16", seed=61, context_lens=(1, 100), alibi=True)
    p = paged_attention_plan(dims_of(inp), 1 << 40, make_opts(0, "auto", schedule="equal_shares"))
    assert p.schedule == SHARES
    seqs = sample_seqs(2048, 16, seed=6)
    compare(run(inp, schedule="equal_shares"), oracle_ref(inp, seqs), "bf16", seqs,
            what="2048 sequences, equal shares")
    inp = make(device_=dev, num_seqs=2, num_heads=48, num_kv_heads=1, head_size=128, block_size=16,
               dtype="f16", seed=62, context_lens=[65536, 30000], alibi=True)
    compare(run(inp, schedule="equal_shares"), oracle_ref(inp), "f16", [0, 1],
            what="65536-token context, equal shares")


def test_equal_shares_empty_batch():
    dev = device()
    inp = make(device_=dev, num_seqs=6, num_heads=48, num_kv_heads=1, head_size=128, block_size=16,
               dtype="f16", seed=3, context_lens=[0] * 6, max_blocks_per_seq=4)
    out = run(inp, schedule="equal_shares")
    assert (out == 0).all()


@pytest.mark.parametrize("kv", [None, "fp8"])
@pytest.mark.parametrize("batch", [256, 48])
def test_equal_shares_needles_at_cuts(kv, batch):
    """MQA 48/1 ragged with ALiBi at batch 256 in equal shares: needles right
    at, before and after the tile where a share starts inside each sampled
    sequence, so a piece that starts or ends one tile off, or a merge that drops
    or repeats a piece, moves that row by O(1)."""
    dev = device()
    args = dict(workload_args("mqa_ragged_alibi", batch), kv_layout="joint")
    if kv:
        args["kv_dtype"] = kv
    inp = make(device_=dev, poison=True, **args)
    p = paged_attention_plan(dims_of(inp), 1 << 40, make_opts(0, "auto", schedule="equal_shares"))
    assert p.schedule == SHARES
    if batch < 256:  # fewer items than workgroup slots: the auto plan's choice too
        assert paged_attention_plan(dims_of(inp), 1 << 40, make_opts()).schedule == SHARES
    lens = inp.context_lens.cpu().numpy()
    cut = share_bounds.cuts(lens, 1, inp.block_size, *share_bounds.launched(inp))
    cut_seqs = sorted(cut)
    rng = np.random.default_rng(7)
    seqs = sorted(set(rng.choice(cut_seqs, size=min(16, len(cut_seqs)), replace=False).tolist())
                  | {int(np.argmax(lens))})
    Hq = inp.query.shape[1]
    pos = {}
    for s in seqs:
        b = cut.get(s, [])[:4]  # (4 cuts x 9 positions + 10 fit the 48 heads)
        near = [x for t in b for x in (t - 15, t, t + 15)]
        pos[s] = needles.positions_for(int(lens[s]), Hq, inp.block_size, boundaries=near, seed=s)
        for t in b:  # every chosen cut is covered, one tile either side
            for x in (t - 16, t - 1, t, t + 15):
                assert not (0 <= x < lens[s]) or x in pos[s], (s, t, x)
    planted = needles.plant(inp, pos)
    ref = oracle_ref(inp, seqs)
    for i, s in enumerate(seqs):
        assert np.abs(ref[i] - planted["v"][s]).max() <= 1e-6 * max(1.0, np.abs(ref[i]).max())
    compare(run(inp, schedule="equal_shares"), ref, inp.dtype, seqs,
            what=f"mqa batch {batch} equal shares needles {kv}")
