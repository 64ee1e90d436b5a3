"""The parity gate of the GPU tests: a HIP output against the fp64 oracle.

Pure numpy (no GPU, no torch), so the gate itself is tested on the CPU
(tests/test_parity_gate.py) against oracle results with planted indexing
mistakes.

Three bounds, each checked on every comparison:

* max-abs per element: 2e-3 for fp16 outputs, 1e-2 for bf16 (the stated
  tolerance of the decode path);
* relative L2 over the whole compared output: 2 u;
* relative L2 per output row (the D elements of one query head of one query
  token): 4 u; a row whose reference is exactly zero (no context) must come
  back as zeros;

where u is the unit roundoff of the output format (round to nearest even):
2^-8 for bf16 (8 significant bits), 2^-11 for fp16 (11 bits).

Why these bounds hold for a correct kernel.  The GPU result differs from the
exact one by (i) the final rounding of each output element, at most u
relative per element and therefore at most u in relative L2 of any row or of
the whole output; (ii) on the matrix-core engine, the rounding of each softmax
weight p_t to the 16-bit operand type, a relative perturbation d_t with
|d_t| <= u.  Because the normaliser sums the same rounded weights, the result
stays a convex combination of value rows and its error is
sum_t d_t p_t (V_t - out) / sum_t p_t: a sum of many small terms of
independent sign, whose relative size against |out| is about u / 2 (it does
not grow with the context length: |out| and the error both scale as
1/sqrt(L_eff) for independent value rows); (iii) fp32 accumulation, orders of
magnitude below both.  A correct kernel thus lands near 0.6 u, and 2 u
(whole output) and 4 u (single row, where the sum in (ii) fluctuates more)
leave room for its spread.

What they catch that max-abs does not.  With a long flat softmax the outputs
are small (|out| ~ 1/sqrt(L)), so max-abs 1e-2 is a large fraction of the
signal: at 64 query / 8 kv heads, D 128, L 4096, bf16, dropping the final
16-token tile moves outputs by less than 1e-2 but changes each affected row
by about 5e-2 in relative L2, 13 u; reading one block from another sequence
does the same.  The CPU tests of this module check both.
"""
from __future__ import annotations

import numpy as np

MAX_ABS = {"f16": 2e-3, "bf16": 1e-2}
UNIT_ROUNDOFF = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
REL_L2 = {k: 2 * u for k, u in UNIT_ROUNDOFF.items()}
ROW_REL_L2 = {k: 4 * u for k, u in UNIT_ROUNDOFF.items()}


def errors(got: np.ndarray, ref: np.ndarray):
    """(max abs error, relative L2 over everything, largest per-row relative L2,
    index of that row, largest abs value in rows whose reference is zero)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.shape != ref.shape:
        raise ValueError(f"shapes differ: {got.shape} vs {ref.shape}")
    if got.size == 0:
        return 0.0, 0.0, 0.0, None, 0.0
    diff = got - ref
    max_abs = float(np.max(np.abs(diff)))
    ref_norm = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff)) / ref_norm if ref_norm > 0 else float(np.linalg.norm(diff) > 0) * np.inf
    D = ref.shape[-1]
    r2 = ref.reshape(-1, D)
    d2 = diff.reshape(-1, D)
    rn = np.linalg.norm(r2, axis=1)
    dn = np.linalg.norm(d2, axis=1)
    nz = rn > 0
    row_rel = np.zeros_like(rn)
    row_rel[nz] = dn[nz] / rn[nz]
    worst = int(np.argmax(row_rel)) if nz.any() else None
    zero_rows_abs = float(np.max(np.abs(d2[~nz]))) if (~nz).any() else 0.0
    return max_abs, rel, float(row_rel.max()) if nz.any() else 0.0, worst, zero_rows_abs


def check(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    """Assert the three bounds; returns (max_abs, rel_l2, worst_row_rel_l2)."""
    got = np.asarray(got, dtype=np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    max_abs, rel, row_rel, worst, zero_abs = errors(got, ref)
    print(f"  {what}: max_abs={max_abs:.3e} rel_l2={rel:.3e} worst_row_rel_l2={row_rel:.3e}",
          flush=True)
    assert max_abs <= MAX_ABS[dtype], f"{what}: max abs error {max_abs} > {MAX_ABS[dtype]}"
    assert rel <= REL_L2[dtype], f"{what}: relative L2 error {rel} > {REL_L2[dtype]}"
    if worst is not None:
        idx = np.unravel_index(worst, ref.shape[:-1])
        assert row_rel <= ROW_REL_L2[dtype], (
            f"{what}: row {tuple(int(i) for i in idx)} relative L2 error {row_rel} > {ROW_REL_L2[dtype]}")
    assert zero_abs == 0.0, f"{what}: a row with an all-zero reference is not zero ({zero_abs})"
    return max_abs, rel, row_rel
