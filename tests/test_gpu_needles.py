"""GPU needle tests at full size: every sampled (sequence, head) gets a query
that points at one chosen token (tests/needles.py), so a tile read from the
wrong place changes that row by O(1) -- far beyond any tolerance -- while the
rest of the gate (max-abs, relative L2 per row and overall) still applies.

Positions: 0, the first block and tile edges (BS - 1, BS, BS + 1, 15, 16, 17),
every partition boundary of the plan +-1, L - 2, L - 1 and seeded random
tokens.  Cases, each in the auto plan and with each engine (and forced
partitions where the auto plan is a single pass):
  * the headline batch: GQA 64/8, bf16, D 128, block 16, context 4096, batch
    256, joint cache layout (16 sequences sampled);
  * the same with an FP8 E4M3 cache;
  * MQA 48/1 fp16 ragged 64..8192 with ALiBi, batch 256 (the LDS-staged path
    of groups above 16 heads: equal shares, and split partitions);
  * 8-token blocks with contexts past the 512-tile LDS window of tile
    source offsets that the staged path keeps (refills at 4096, 8192 ...
    tokens),
    16-bit and FP8 caches, 48- and 64-head groups.
"""
import numpy as np
import pytest
import torch

import needles
from decode_attention_paged_06_amd import make_dims, make_opts, paged_attention_plan, kv_layout_of
from gpu_util import compare, device, make, oracle_ref, run, sample_seqs
from workloads import workload_args

pytestmark = pytest.mark.gpu


def plan_of(inp, engine="auto", partition_size=0, schedule="auto"):
    dims = make_dims(inp.query, inp.key_cache, inp.block_tables, inp.k_scale, inp.v_scale,
                     kv_layout_of(inp.key_cache, inp.value_cache))
    return paged_attention_plan(dims, 1 << 40, make_opts(partition_size, engine, schedule=schedule))


def check_needles(inp, seqs, runs, boundaries, what):
    """Plant needles in `seqs`, then compare every (engine, partition size[,
    schedule]) run."""
    lens = inp.context_lens.cpu().numpy()
    Hq = inp.query.shape[1]
    pos = {s: needles.positions_for(int(lens[s]), Hq, inp.block_size, boundaries, seed=s)
           for s in seqs}
    planted = needles.plant(inp, pos)
    ref = oracle_ref(inp, seqs)
    for i, s in enumerate(seqs):   # the needles hold: the exact output is the value row
        assert np.abs(ref[i] - planted["v"][s]).max() <= 1e-6 * max(1.0, np.abs(ref[i]).max())
    for r in runs:
        engine, ps, schedule = r if len(r) == 3 else r + ("auto",)
        p = plan_of(inp, engine, ps, schedule)
        out = run(inp, engine=engine, partition_size=ps, schedule=schedule)
        compare(out, ref, inp.dtype, seqs,
                what=f"{what} engine={engine} partition={ps} schedule={schedule} (plan: "
                     f"{p.num_partitions} x {p.partition_size}, schedule {p.schedule})")


@pytest.mark.parametrize("kv", ["native", "fp8"])
def test_headline_needles(kv):
    dev = device()
    args = workload_args("gqa_ctx4096", 256)
    inp = make(device_=dev, poison=True, kv_layout="joint",
               **(dict(args, kv_dtype="fp8") if kv == "fp8" else args))
    seqs = sample_seqs(256, 16, seed=11)
    runs = [("auto", 0), ("mfma", 0), ("valu", 0), ("mfma", 512), ("valu", 1024), ("mfma", 64)]
    check_needles(inp, seqs, runs, boundaries=(64, 512, 1024, 2048, 3072), what=f"headline {kv}")


@pytest.mark.parametrize("kv", ["native", "fp8"])
def test_mqa_ragged_alibi_needles(kv):
    dev = device()
    args = workload_args("mqa_ragged_alibi", 256)
    inp = make(device_=dev, poison=True, kv_layout="joint",
               **(dict(args, kv_dtype="fp8") if kv == "fp8" else args))
    lens = inp.context_lens.cpu().numpy()
    # the sample: the longest and shortest sequences plus seeded ones
    seqs = sorted(set(sample_seqs(256, 14, seed=12)) | {int(np.argmax(lens)), int(np.argmin(lens))})
    parts = plan_of(inp, schedule="longest_first")
    assert parts.num_partitions > 1, "the MQA batch is expected to split"
    bounds = tuple(parts.partition_size * k for k in range(1, parts.num_partitions)) + (1024, 2048)
    # auto (partitions, longest first), in grid order; equal shares (needles at
    # their own cuts: tests/test_gpu_shares.py); one pass; the VALU engine
    runs = [("auto", 0), ("mfma", 0, "grid"), ("mfma", 0, "equal_shares"), ("mfma", -1),
            ("mfma", 1024), ("valu", 0)]
    check_needles(inp, seqs, runs, boundaries=bounds, what=f"mqa ragged alibi {kv}")
    # the grid order of the same split gives the same bits
    a = run(inp, engine="mfma", schedule="grid")
    b = run(inp, engine="mfma", schedule="longest_first")
    assert torch.equal(a, b)


@pytest.mark.parametrize("group,dtype", [(48, "f16"), (64, "bf16")])
@pytest.mark.parametrize("kv", ["native", "fp8"])
def test_table_window_needles(group, dtype, kv):
    """Block size 8: the staged loop's LDS window of 512 tile offsets covers
    4096 tokens, so these contexts refill it once or more mid-walk."""
    dev = device()
    lens = [4097, 9000, 12345, 600]
    inp = make(device_=dev, num_seqs=len(lens), num_heads=group, num_kv_heads=1, head_size=128,
               block_size=8, dtype=dtype, seed=8000 + group, context_lens=lens, alibi=True,
               poison=True, kv_dtype="fp8" if kv == "fp8" else None, kv_layout="joint")
    runs = [("mfma", -1), ("auto", 0), ("mfma", 8192), ("mfma", 2048)]
    check_needles(inp, list(range(len(lens))), runs, boundaries=(2048, 4096, 8192, 12288),
                  what=f"block 8 window G={group} {kv}")
