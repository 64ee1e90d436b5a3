"""GPU parity over seeded random configurations.

The targeted tests fix one or two parameters at a time; these draw whole
configurations at random (group size, head size, dtype, block size, cache
format and layout, ALiBi, engine, partition size, schedule, ragged lengths, and
new-token counts for the multi-query call) from a fixed seed, so combinations nobody
wrote down are checked against the fp64 oracle too.  Sizes stay small enough
for the oracle to finish in seconds.
"""
import numpy as np
import pytest
import torch

from gpu_util import compare, device, oracle_ref, run, to_device, make
from test_gpu_prefill import ref_prefill, run_prefill
from workloads import prefill_inputs

pytestmark = pytest.mark.gpu

GROUPS = [1, 2, 3, 4, 6, 8, 12, 16, 20, 32, 48, 64]
BLOCKS = [8, 16, 32, 64, 128, 256]


def draw_decode(rng):
    G = int(rng.choice(GROUPS))
    Hkv = int(rng.integers(1, max(2, 64 // G // 4) + 1)) if G < 64 else 1
    D = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["f16", "bf16"]))
    BS = int(rng.choice(BLOCKS))
    S = int(rng.integers(1, 7))
    lens = [int(x) for x in rng.integers(0, 900, size=S)]
    return dict(G=G, Hkv=Hkv, D=D, dtype=dtype, BS=BS, lens=lens,
                alibi=bool(rng.integers(0, 2)), fp8=bool(rng.integers(0, 4) == 0),
                engine=str(rng.choice(["auto", "valu", "mfma"])),
                ps=int(rng.choice([-1, 0, 0, 128, 256, 512])),
                schedule=str(rng.choice(["auto", "grid", "longest_first"])),
                layout=str(rng.choice(["separate", "joint"])))


@pytest.mark.parametrize("seed", range(48))
def test_random_decode(seed):
    dev = device()
    c = draw_decode(np.random.default_rng(1000 + seed))
    ps = c["ps"] if c["ps"] <= 0 else max(c["ps"], c["BS"])
    inp = to_device(make(num_seqs=len(c["lens"]), num_heads=c["G"] * c["Hkv"],
                         num_kv_heads=c["Hkv"], head_size=c["D"], block_size=c["BS"],
                         dtype=c["dtype"], seed=seed, context_lens=c["lens"], alibi=c["alibi"],
                         poison=True, kv_dtype="fp8" if c["fp8"] else None, kv_layout=c["layout"]), dev)
    ref = oracle_ref(inp)
    out = run(inp, engine=c["engine"], partition_size=ps, schedule=c["schedule"])
    compare(out, ref, c["dtype"], what=f"seed {seed}: {c}")


@pytest.mark.parametrize("seed", range(32))
def test_random_decode_equal_shares(seed):
    """Random staged configurations (groups of 17..64 heads) in equal shares:
    batches from one sequence to 40, lengths from 0, several kv heads."""
    dev = device()
    rng = np.random.default_rng(3000 + seed)
    G = int(rng.choice([20, 24, 32, 40, 48, 64]))
    Hkv = int(rng.integers(1, 4))
    D = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["f16", "bf16"]))
    BS = int(rng.choice(BLOCKS))
    S = int(rng.integers(1, 41))
    hi = int(rng.choice([30, 600, 3000]))
    lens = [int(x) for x in rng.integers(0, hi, size=S)]
    fp8 = bool(rng.integers(0, 3) == 0)
    alibi = bool(rng.integers(0, 2))
    layout = str(rng.choice(["separate", "joint"]))
    inp = to_device(make(num_seqs=S, num_heads=G * Hkv, num_kv_heads=Hkv, head_size=D, block_size=BS,
                         dtype=dtype, seed=seed, context_lens=lens, alibi=alibi, poison=True,
                         kv_dtype="fp8" if fp8 else None, kv_layout=layout), dev)
    seqs = list(range(S)) if S <= 12 else sorted(set(rng.choice(S, 12, replace=False).tolist()))
    ref = oracle_ref(inp, seqs)
    out = run(inp, schedule="equal_shares")
    what = f"seed {seed}: G={G} Hkv={Hkv} D={D} {dtype} BS={BS} S={S} fp8={fp8} alibi={alibi} {layout}"
    compare(out, ref, dtype, seqs, what=what)
    lens_np = np.asarray(lens)
    assert (out[torch.as_tensor(np.flatnonzero(lens_np == 0), device=out.device, dtype=torch.long)] == 0).all(), what


@pytest.mark.parametrize("seed", range(24))
def test_random_prefill(seed):
    dev = device()
    rng = np.random.default_rng(2000 + seed)
    G = int(rng.choice([1, 4, 8, 16, 48]))
    Hkv = 1 if G == 48 else int(rng.integers(1, 3))
    D = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["f16", "bf16"]))
    BS = int(rng.choice([8, 16, 64]))
    S = int(rng.integers(1, 5))
    lens = [int(x) for x in rng.integers(1, 400, size=S)]
    news = [int(rng.integers(0, min(L, 40) + 1)) for L in lens]
    if sum(news) == 0:
        news[0] = 1
    alibi = bool(rng.integers(0, 2))
    fp8 = bool(rng.integers(0, 4) == 0)
    ps = int(rng.choice([-1, 0, max(BS, 64)]))
    layout = str(rng.choice(["separate", "joint"]))
    inp, q, qs, max_q = prefill_inputs(new_tokens=news, seed=seed, device=dev, num_seqs=S,
                                       num_heads=G * Hkv, num_kv_heads=Hkv, head_size=D,
                                       block_size=BS, dtype=dtype, context_lens=lens,
                                       alibi=alibi, poison=True,
                                       kv_dtype="fp8" if fp8 else None, kv_layout=layout)
    ref = ref_prefill(inp, q, qs)
    compare(run_prefill(inp, q, qs, max_q, ps), ref, dtype,
            what=f"seed {seed}: G={G} Hkv={Hkv} D={D} {dtype} BS={BS} lens={lens} new={news} "
                 f"alibi={alibi} fp8={fp8} partition={ps} layout={layout}")
