"""GPU tests of the longest-first schedule's start-order places: on the
LDS-staged kernel at one workgroup per CU (48-head groups), the workgroups
after the first round take their place in the unit order from a counter that
follows the order in the workspace, zeroed by the ordering kernel.  Whatever
the workspace held before, and however often it is reused, every unit must be
walked exactly once: the output equals the grid schedule's bit for bit (the
units are the same, only who walks them changes), and sampled rows meet the
oracle gate.
"""
import pytest
import torch

from decode_attention_paged_06_amd import (kv_layout_of, make_dims, make_opts, paged_attention_decode,
                                           paged_attention_plan)
from gpu_util import compare, device, make, oracle_ref, run, sample_seqs
from workloads import workload_args

pytestmark = pytest.mark.gpu

LONGEST = 2


def call(inp, ws, out):
    paged_attention_decode(out, inp.query, inp.key_cache, inp.value_cache, inp.block_tables,
                           inp.context_lens, inp.scale, inp.block_size, inp.alibi_slopes, workspace=ws,
                           k_scale=inp.k_scale, v_scale=inp.v_scale, schedule="longest_first")
    return out


@pytest.mark.parametrize("kv", [None, "fp8"])
def test_start_order_places_walk_every_unit_once(kv):
    dev = device()
    args = dict(workload_args("mqa_ragged_alibi", 256), kv_layout="joint")
    if kv:
        args["kv_dtype"] = kv
    inp = make(device_=dev, poison=True, **args)
    dims = make_dims(inp.query, inp.key_cache, inp.block_tables, inp.k_scale, inp.v_scale,
                     kv_layout_of(inp.key_cache, inp.value_cache))
    p = paged_attention_plan(dims, 1 << 40, make_opts(0, "auto", schedule="longest_first"))
    assert p.schedule == LONGEST and p.num_partitions > 1
    grid = run(inp, schedule="grid")
    for fill in (0x7f, 0xff, 0x00):  # whatever the counter held before the call
        ws = torch.full((p.workspace_bytes,), fill, dtype=torch.uint8, device=dev)
        for rep in range(2):  # and the same workspace again
            out = call(inp, ws, torch.full_like(inp.query, float("nan")))
            torch.cuda.synchronize()
            assert torch.equal(out, grid), f"fill {fill:#x}, call {rep}: differs from the grid schedule"
    seqs = sample_seqs(256, 16, seed=11)
    compare(out, oracle_ref(inp, seqs), inp.dtype, seqs, what=f"start-order places {kv}")


@pytest.mark.parametrize("case", ["hkv2_g48", "bs32_g40", "many_short"])
def test_start_order_places_other_shapes(case):
    """Two kv heads (two workgroups per unit, places counted over both), a
    40-head group on 32-token blocks, and many short sequences (most later
    units empty): bit-identical to the grid schedule and within the gate."""
    dev = device()
    shapes = {
        "hkv2_g48": dict(num_seqs=100, num_heads=96, num_kv_heads=2, head_size=128, block_size=16,
                         dtype="bf16", context_lens=(1, 6000), alibi=True),
        "bs32_g40": dict(num_seqs=400, num_heads=40, num_kv_heads=1, head_size=128, block_size=32,
                         dtype="f16", context_lens=(0, 5000)),
        "many_short": dict(num_seqs=220, num_heads=48, num_kv_heads=1, head_size=128, block_size=16,
                           dtype="f16", context_lens=(1, 300), max_blocks_per_seq=512),
    }
    inp = make(device_=dev, seed=71, poison=True, kv_layout="joint", **shapes[case])
    dims = make_dims(inp.query, inp.key_cache, inp.block_tables, inp.k_scale, inp.v_scale,
                     kv_layout_of(inp.key_cache, inp.value_cache))
    p = paged_attention_plan(dims, 1 << 40, make_opts(0, "auto", schedule="longest_first"))
    assert p.schedule == LONGEST and p.num_partitions > 1
    ws = torch.full((p.workspace_bytes,), 0x5a, dtype=torch.uint8, device=dev)
    out = call(inp, ws, torch.full_like(inp.query, float("nan")))
    torch.cuda.synchronize()
    assert torch.equal(out, run(inp, schedule="grid")), f"{case}: differs from the grid schedule"
    S = inp.query.shape[0]
    seqs = sample_seqs(S, 16, seed=12)
    compare(out, oracle_ref(inp, seqs), inp.dtype, seqs, what=f"start-order places {case}")
