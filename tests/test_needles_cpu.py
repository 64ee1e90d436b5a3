"""The needle construction (tests/needles.py) checked with the oracle on the
CPU: each planted query makes the exact output its chosen value row, with and
without ALiBi, for 16-bit and FP8 caches and small and large blocks."""
import numpy as np
import pytest

import needles
from gpu_util import oracle_ref
from workloads import decode_inputs


CASES = [
    # (heads, kv heads, dtype, block, lengths, alibi, kv dtype)
    (64, 8, "bf16", 16, [4096, 1000], False, None),
    (48, 1, "f16", 16, [8192, 300], True, None),
    (48, 1, "f16", 8, [9000], True, None),
    (16, 2, "bf16", 16, [700, 33], True, "fp8"),
]


@pytest.mark.parametrize("case", CASES)
def test_needles_force_their_value_row(case):
    Hq, Hkv, dtype, BS, lens, alibi, kvd = case
    inp = decode_inputs(num_seqs=len(lens), num_heads=Hq, num_kv_heads=Hkv, head_size=128,
                        block_size=BS, dtype=dtype, seed=7 + Hq + BS, context_lens=lens,
                        alibi=alibi, poison=True, kv_dtype=kvd)
    pos = {s: needles.positions_for(L, Hq, BS, boundaries=(256, 512, 4096), seed=s)
           for s, L in enumerate(lens)}
    plan = needles.plant(inp, pos)
    ref = oracle_ref(inp, plan["seqs"])
    for i, s in enumerate(plan["seqs"]):
        err = np.abs(ref[i] - plan["v"][s]).max()
        assert err < 1e-6 * max(1.0, np.abs(plan["v"][s]).max()), (s, err)
    # every special position is used
    assert 0 in pos[0] and lens[0] - 1 in pos[0] and 16 in pos[0]
