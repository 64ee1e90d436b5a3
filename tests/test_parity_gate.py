"""The parity gate (tests/parity_gate.py) on the CPU: it admits a result with
the rounding a correct kernel performs and rejects the indexing mistakes that
max-abs alone lets through at long bf16 contexts.

Shape: the headline decode (64 query / 8 kv heads, D 128, block 16, bf16,
context 4096), a few sequences.  "Wrong" results are the oracle's own output
for wrongly indexed inputs (a context one tile short, a block-table entry
pointing at another sequence's block), rounded to bf16 as a kernel would.
"""
import numpy as np
import pytest

import oracle
import parity_gate
from workloads import decode_inputs, raw_u16

S, HQ, HKV, D, BS, L = 4, 64, 8, 128, 16, 4096


@pytest.fixture(scope="module")
def batch():
    inp = decode_inputs(num_seqs=S, num_heads=HQ, num_kv_heads=HKV, head_size=D, block_size=BS,
                        dtype="bf16", seed=3004, context_lens=L)
    q, kc, vc = raw_u16(inp.query), raw_u16(inp.key_cache), raw_u16(inp.value_cache)
    tables, lens = inp.block_tables.numpy().copy(), inp.context_lens.numpy().copy()
    ref = oracle.paged_decode(q, kc, vc, tables, lens, inp.scale, BS, dtype="bf16")
    return dict(q=q, kc=kc, vc=vc, tables=tables, lens=lens, scale=inp.scale, ref=ref)


def as_bf16(x):
    """x rounded to bf16 (RNE) and read back as float64: a kernel's final store."""
    return oracle.to_float64(oracle.round_to_storage(x, "bf16"), "bf16")


def rejected(got, ref, dtype="bf16"):
    try:
        parity_gate.check(got, ref, dtype, "planted")
    except AssertionError:
        return True
    return False


def simulated_matrix_core_result(b):
    """A correct kernel's arithmetic in the matrix-core engine's precisions:
    fp32 logits, weights exp(z - max) rounded to bf16, normaliser summed from
    the rounded weights, fp32 products and sums, output rounded to bf16."""
    q = oracle.to_float64(b["q"], "bf16").astype(np.float32)
    out = np.zeros((S, HQ, D))
    for s in range(S):
        K = oracle.to_float64(oracle.sequence_kv(b["kc"], b["tables"][s], L, BS), "bf16").astype(np.float32)
        V = oracle.to_float64(oracle.sequence_kv(b["vc"], b["tables"][s], L, BS), "bf16").astype(np.float32)
        for h in range(HQ):
            kvh = h // (HQ // HKV)
            z = (K[kvh] @ q[s, h]) * np.float32(b["scale"])
            p = np.exp(z - z.max()).astype(np.float32)
            p16 = oracle.to_float64(oracle.round_to_storage(p, "bf16"), "bf16").astype(np.float32)
            out[s, h] = (p16 @ V[kvh]) / p16.sum(dtype=np.float32)
    return as_bf16(out)


def test_correct_rounding_passes(batch):
    ref = batch["ref"]
    max_abs, rel, row = parity_gate.check(as_bf16(ref), ref, "bf16", "oracle rounded to bf16")
    assert rel < parity_gate.UNIT_ROUNDOFF["bf16"]


def test_simulated_matrix_core_arithmetic_passes(batch):
    ref = batch["ref"]
    parity_gate.check(simulated_matrix_core_result(batch), ref, "bf16", "bf16 weights, fp32 sums")


def test_dropped_tile_rejected_where_max_abs_is_blind(batch):
    b = batch
    short = b["lens"] - BS   # every sequence loses its final 16-token tile
    wrong = as_bf16(oracle.paged_decode(b["q"], b["kc"], b["vc"], b["tables"], short, b["scale"], BS,
                                        dtype="bf16"))
    # max-abs is of the order of its own bar (per sequence it lands on either
    # side of 1e-2 with the seed), relative L2 is several times its bound
    per_seq = [parity_gate.errors(wrong[s], b["ref"][s]) for s in range(S)]
    assert any(e[0] <= parity_gate.MAX_ABS["bf16"] for e in per_seq), "max-abs alone passes a sequence"
    assert all(e[1] > 5 * parity_gate.REL_L2["bf16"] for e in per_seq)
    assert all(rejected(wrong[s], b["ref"][s]) for s in range(S))


def test_dropped_tile_of_one_sequence_among_sixteen_rejected(batch):
    """One sequence's tile missing among 16 sampled ones (the GPU tests' sample size)."""
    b = batch
    ref16 = np.concatenate([b["ref"]] * 4)
    wrong = as_bf16(ref16).copy()
    short = b["lens"].copy()
    short[2] -= BS
    wrong[2] = as_bf16(oracle.paged_decode(b["q"], b["kc"], b["vc"], b["tables"], short, b["scale"], BS,
                                           dtype="bf16", seqs=[2]))[0]
    assert rejected(wrong, ref16)
    # and a single query head's row
    one = as_bf16(ref16).copy()
    one[2, 5] = wrong[2, 5]
    assert rejected(one, ref16)


def test_misplaced_tile_rejected(batch):
    b = batch
    tables = b["tables"].copy()
    j = L // BS // 2
    tables[0, j] = b["tables"][1, j]   # a block of sequence 1 read in place of sequence 0's
    wrong = b["ref"].copy()
    wrong[0] = oracle.paged_decode(b["q"], b["kc"], b["vc"], tables, b["lens"], b["scale"], BS,
                                   dtype="bf16", seqs=[0])[0]
    assert rejected(as_bf16(wrong), b["ref"])
    # the last tile misplaced (the table-walk end)
    tables = b["tables"].copy()
    tables[3, L // BS - 1] = b["tables"][0, 0]
    wrong = b["ref"].copy()
    wrong[3] = oracle.paged_decode(b["q"], b["kc"], b["vc"], tables, b["lens"], b["scale"], BS,
                                   dtype="bf16", seqs=[3])[0]
    assert rejected(as_bf16(wrong), b["ref"])


def test_swapped_heads_rejected(batch):
    """Two query heads of one group exchanged (a head-mapping slip inside a group)."""
    ref = batch["ref"]
    wrong = as_bf16(ref).copy()
    wrong[1, [3, 4]] = wrong[1, [4, 3]]
    assert rejected(wrong, ref)


def test_zero_rows_must_be_zero():
    ref = np.zeros((2, 3, 8))
    ref[1] = 1.0
    got = ref.copy()
    got[0, 1, 2] = 1e-6
    with pytest.raises(AssertionError):
        parity_gate.check(got, ref, "f16")
    parity_gate.check(ref.copy(), ref, "f16")


def test_fp16_bounds_are_tighter():
    assert parity_gate.REL_L2["f16"] == 2 * 2.0 ** -11
    assert parity_gate.ROW_REL_L2["bf16"] == 4 * 2.0 ** -8
    rng = np.random.default_rng(1)
    ref = rng.standard_normal((4, 8, 64)) * 0.05
    noisy = ref * (1 + 3 * 2.0 ** -11 * rng.choice([-1.0, 1.0], size=ref.shape))
    with pytest.raises(AssertionError):
        parity_gate.check(noisy, ref, "f16")
    parity_gate.check(noisy, ref, "bf16")
