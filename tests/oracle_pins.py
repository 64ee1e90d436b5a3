"""Pins of the CPU oracle against facts fixed outside it.

Each pin raises AssertionError on failure.  They look the oracle's helpers up
through the module at call time, so ``test_oracle_mutants.py`` can plant a
mistake in one helper and check that some pin catches it.

The pages print no worked example with values (only timings), so the pins are
mathematical: brute force on tiny inputs, a library routine on dense inputs,
closed forms, invariants and construction-time ground truth.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle.paged_attention as ora
from workloads import decode_inputs, raw_u16

RNG_SEED = 1234


def _rng(k=0):
    return np.random.default_rng(RNG_SEED + k)


def _tiny(dtype="bf16", seed=7, alibi=True, poison=True, Hq=6, Hkv=2, D=8, BS=4,
          lens=(1, 4, 5, 11, 0, 16)):
    inp = decode_inputs(num_seqs=len(lens), num_heads=Hq, num_kv_heads=Hkv, head_size=D,
                        block_size=BS, dtype=dtype, seed=seed, context_lens=list(lens),
                        alibi=alibi, poison=poison, max_blocks_per_seq=6)
    return inp


def _oracle_on(inp, **kw):
    return ora.paged_decode(raw_u16(inp.query), raw_u16(inp.key_cache), raw_u16(inp.value_cache),
                            inp.block_tables.numpy(), inp.context_lens.numpy(), inp.scale,
                            inp.block_size,
                            None if inp.alibi_slopes is None else inp.alibi_slopes.numpy(),
                            dtype=inp.dtype, **kw)


# --------------------------------------------------------------------------
# Brute force: pure Python loops, math.exp / math.fsum, the page's head_mapping
# --------------------------------------------------------------------------

def _brute_force(q, kc, vc, tables, lens, scale, BS, slopes):
    S, Hq, D = len(q), len(q[0]), len(q[0][0])
    Hkv = len(kc[0])
    G = Hq // Hkv
    head_mapping = [k for k in range(Hkv) for _ in range(G)]   # repeat_interleave
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(S)]
    for s in range(S):
        L = lens[s]
        if L <= 0:
            continue
        for h in range(Hq):
            kvh = head_mapping[h]
            logits = []
            for t in range(L):
                blk, off = tables[s][t // BS], t % BS
                z = scale * math.fsum(q[s][h][d] * kc[blk][kvh][off][d] for d in range(D))
                if slopes is not None:
                    z += slopes[h] * (t - (L - 1))
                logits.append(z)
            mx = max(logits)
            w = [math.exp(z - mx) for z in logits]
            den = math.fsum(w)
            for d in range(D):
                num = math.fsum(w[t] * vc[tables[s][t // BS]][kvh][t % BS][d] for t in range(L))
                out[s][h][d] = num / den
    return np.array(out)


def pin_brute_force():
    for dtype, alibi in (("bf16", True), ("f16", False)):
        inp = _tiny(dtype=dtype, alibi=alibi)
        f = lambda t: ora.to_float64(raw_u16(t), dtype).tolist()   # noqa: E731
        slopes = None if inp.alibi_slopes is None else [float(x) for x in inp.alibi_slopes.numpy()]
        ref = _brute_force(f(inp.query), f(inp.key_cache), f(inp.value_cache),
                           inp.block_tables.tolist(), inp.context_lens.tolist(),
                           inp.scale, inp.block_size, slopes)
        got = _oracle_on(inp)
        assert np.isfinite(got).all()
        assert np.max(np.abs(got - ref)) <= 1e-12, np.max(np.abs(got - ref))


# --------------------------------------------------------------------------
# Dense attention by a library routine, on K/V scattered by this test
# --------------------------------------------------------------------------

def _scatter_dense(rng, lens, Hkv, D, BS, extra_blocks=3):
    """Dense per-sequence K/V, placed into a shuffled pool by explicit loops."""
    nbs = [(L + BS - 1) // BS for L in lens]
    NB = sum(nbs) + extra_blocks
    perm = rng.permutation(NB)
    maxb = max(max(nbs), 1)
    tables = rng.integers(0, NB, size=(len(lens), maxb))
    kc = rng.standard_normal((NB, Hkv, BS, D))
    vc = rng.standard_normal((NB, Hkv, BS, D))
    dense_k, dense_v, slots = [], [], []
    pos = 0
    for s, (L, nb) in enumerate(zip(lens, nbs)):
        tables[s, :nb] = perm[pos:pos + nb]
        pos += nb
        dk = rng.standard_normal((Hkv, L, D))
        dv = rng.standard_normal((Hkv, L, D))
        sl = []
        for t in range(L):
            blk = tables[s, t // BS]
            kc[blk, :, t % BS, :] = dk[:, t, :]
            vc[blk, :, t % BS, :] = dv[:, t, :]
            sl.append(int(blk) * BS + t % BS)
        dense_k.append(dk)
        dense_v.append(dv)
        slots.append(sl)
    return kc, vc, tables, dense_k, dense_v, slots


def pin_dense_library():
    import torch.nn.functional as F
    rng = _rng(1)
    lens = [1, 7, 16, 33, 50]
    Hq, Hkv, D, BS = 8, 2, 16, 16
    kc, vc, tables, dk, dv, _ = _scatter_dense(rng, lens, Hkv, D, BS)
    q = rng.standard_normal((len(lens), Hq, D))
    slopes = np.array([2.0 ** (-8.0 * (i + 1) / Hq) for i in range(Hq)], dtype=np.float32)
    scale = 0.3
    for use_alibi in (False, True):
        got = ora.paged_decode(q, kc, vc, tables, np.array(lens), scale, BS,
                               slopes if use_alibi else None)
        for s, L in enumerate(lens):
            G = Hq // Hkv
            idx = torch.tensor([h // G for h in range(Hq)])
            K = torch.from_numpy(dk[s])[idx]          # [Hq, L, D]
            V = torch.from_numpy(dv[s])[idx]
            Q = torch.from_numpy(q[s])[:, None, :]    # [Hq, 1, D]
            mask = None
            if use_alibi:
                # bias slope * t: differs from the oracle's anchor by a per-row constant
                mask = torch.from_numpy(slopes.astype(np.float64))[:, None, None] * \
                    torch.arange(L, dtype=torch.float64)[None, None, :]
            ref = F.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=scale)[:, 0, :]
            err = np.max(np.abs(got[s] - ref.numpy()))
            assert err <= 1e-12, err


def pin_gather_by_construction():
    rng = _rng(2)
    lens = [3, 8, 17]
    Hkv, D, BS = 3, 8, 8
    _, _, tables, dk, dv, slots = _scatter_dense(rng, lens, Hkv, D, BS)
    NB = int(tables.max()) + 4
    # random 16-bit patterns (NaN / Inf encodings included) at the dense positions
    kc = rng.integers(0, 1 << 16, size=(NB, Hkv, BS, D), dtype=np.uint16)
    vc = rng.integers(0, 1 << 16, size=(NB, Hkv, BS, D), dtype=np.uint16)
    for s, sl in enumerate(slots):
        bk = rng.integers(0, 1 << 16, size=(len(sl), Hkv, D), dtype=np.uint16)
        bv = rng.integers(0, 1 << 16, size=(len(sl), Hkv, D), dtype=np.uint16)
        for i, slot in enumerate(sl):
            kc[slot // BS, :, slot % BS, :] = bk[i]
            vc[slot // BS, :, slot % BS, :] = bv[i]
        k_out, v_out = ora.gather_cached_kv(kc, vc, np.array(sl + [-1]), BS)
        assert np.array_equal(k_out[:-1], bk) and np.array_equal(v_out[:-1], bv)
        assert not k_out[-1].any() and not v_out[-1].any()


def pin_sequence_kv_by_construction():
    rng = _rng(3)
    lens = [1, 15, 16, 17, 40]
    Hkv, D, BS = 2, 4, 16
    kc, vc, tables, dk, dv, _ = _scatter_dense(rng, lens, Hkv, D, BS)
    for s, L in enumerate(lens):
        assert np.array_equal(ora.sequence_kv(kc, tables[s], L, BS), dk[s])
        assert np.array_equal(ora.sequence_kv(vc, tables[s], L, BS), dv[s])


# --------------------------------------------------------------------------
# Invariants and closed forms
# --------------------------------------------------------------------------

def pin_block_permutation():
    inp = _tiny(poison=False)
    base = _oracle_on(inp)
    rng = _rng(4)
    NB = inp.key_cache.shape[0]
    pi = rng.permutation(NB)
    kc = np.empty_like(raw_u16(inp.key_cache))
    vc = np.empty_like(kc)
    kc[pi] = raw_u16(inp.key_cache)
    vc[pi] = raw_u16(inp.value_cache)
    tables = pi[inp.block_tables.numpy()]
    got = ora.paged_decode(raw_u16(inp.query), kc, vc, tables, inp.context_lens.numpy(),
                           inp.scale, inp.block_size, inp.alibi_slopes.numpy(), dtype=inp.dtype)
    assert np.array_equal(got, base)


def pin_context_one():
    for alibi in (False, True):
        inp = decode_inputs(num_seqs=5, num_heads=8, num_kv_heads=4, head_size=16, block_size=8,
                            dtype="f16", seed=11, context_lens=1, alibi=alibi, poison=True,
                            max_blocks_per_seq=3)
        got = _oracle_on(inp)
        vc = ora.to_float64(raw_u16(inp.value_cache), "f16")
        for s in range(5):
            blk = int(inp.block_tables[s, 0])
            for h in range(8):
                assert np.array_equal(got[s, h], vc[blk, h // 2, 0])


def pin_identical_keys_mean():
    rng = _rng(5)
    L, Hkv, D, BS = 37, 1, 8, 16
    kc, vc, tables, dk, dv, _ = _scatter_dense(rng, [L], Hkv, D, BS)
    krow = rng.standard_normal(D)
    for t in range(L):
        kc[tables[0, t // BS], 0, t % BS] = krow
    q = rng.standard_normal((1, 3, D))
    got = ora.paged_decode(q, kc, vc, tables, np.array([L]), 0.7, BS)
    mean = dv[0][0].mean(axis=0)
    for h in range(3):
        assert np.max(np.abs(got[0, h] - mean)) <= 1e-14 * max(1.0, np.abs(mean).max())


def pin_identical_keys_alibi():
    rng = _rng(6)
    L, Hkv, D, BS = 29, 1, 8, 8
    kc, vc, tables, dk, dv, _ = _scatter_dense(rng, [L], Hkv, D, BS)
    krow = rng.standard_normal(D)
    for t in range(L):
        kc[tables[0, t // BS], 0, t % BS] = krow
    slopes = np.array([0.5, 0.125, 2.0 ** -7], dtype=np.float32)
    q = rng.standard_normal((1, 3, D))
    got = ora.paged_decode(q, kc, vc, tables, np.array([L]), 0.7, BS, slopes)
    for h in range(3):
        r = math.exp(-float(slopes[h]))
        w = np.array([r ** (L - 1 - t) * (1 - r) / (1 - r ** L) for t in range(L)])
        ref = w @ dv[0][0]
        assert np.max(np.abs(got[0, h] - ref)) <= 1e-13


def pin_needle():
    rng = _rng(7)
    lens = [40]
    Hkv, D, BS = 1, 16, 16
    kc, vc, tables, dk, dv, _ = _scatter_dense(rng, lens, Hkv, D, BS)
    K = dk[0][0]
    scale = 0.25
    for tstar in (0, BS - 1, BS, BS + 1, lens[0] - 1):
        ks = K[tstar]
        margins = ks @ ks - K @ ks
        margins[tstar] = np.inf
        if margins.min() <= 0:
            continue
        c = 60.0 / (scale * margins.min())
        q = (c * ks)[None, None, :]
        got = ora.paged_decode(q, kc, vc, tables, np.array(lens), scale, BS)
        assert np.max(np.abs(got[0, 0] - dv[0][0][tstar])) <= 1e-12


def pin_gqa_equals_repeated_mha():
    inp = _tiny(poison=False)     # Hq = 6, Hkv = 2, G = 3
    base = _oracle_on(inp)
    G = 3
    kc = np.repeat(raw_u16(inp.key_cache), G, axis=1)    # head h of the MHA cache = kv head h // G
    vc = np.repeat(raw_u16(inp.value_cache), G, axis=1)
    got = ora.paged_decode(raw_u16(inp.query), kc, vc, inp.block_tables.numpy(),
                           inp.context_lens.numpy(), inp.scale, inp.block_size,
                           inp.alibi_slopes.numpy(), dtype=inp.dtype)
    assert np.array_equal(got, base)


def pin_split_merge():
    inp = _tiny(poison=False)
    base = _oracle_on(inp)
    for ps in (1, 3, 4, 5, 16, 100):
        got = ora.paged_decode_partitioned(
            raw_u16(inp.query), raw_u16(inp.key_cache), raw_u16(inp.value_cache),
            inp.block_tables.numpy(), inp.context_lens.numpy(), inp.scale, inp.block_size, ps,
            inp.alibi_slopes.numpy(), dtype=inp.dtype)
        assert np.max(np.abs(got - base)) <= 1e-13


def pin_shift_and_linearity():
    rng = _rng(8)
    lens = [9, 21]
    Hkv, D, BS = 2, 8, 4
    kc, vc, tables, dk, dv, _ = _scatter_dense(rng, lens, Hkv, D, BS)
    q = rng.standard_normal((2, 4, D))
    slopes = np.array([0.1, 0.2, 0.3, 0.4], dtype=np.float32)
    base = ora.paged_decode(q, kc, vc, tables, np.array(lens), 0.5, BS, slopes)
    c = rng.standard_normal(D)
    # K + 1 c^T shifts every logit of a row by the same amount
    got = ora.paged_decode(q, kc + c, vc, tables, np.array(lens), 0.5, BS, slopes)
    assert np.max(np.abs(got - base)) <= 1e-12
    # V + 1 c^T adds c to every output row
    got = ora.paged_decode(q, kc, vc + c, tables, np.array(lens), 0.5, BS, slopes)
    assert np.max(np.abs(got - (base + c))) <= 1e-12
    # q * k with scale / k leaves the logits unchanged
    got = ora.paged_decode(q * 4.0, kc, vc, tables, np.array(lens), 0.125, BS, slopes)
    assert np.max(np.abs(got - base)) <= 1e-12


def pin_empty_context():
    inp = _tiny(poison=True)
    lens = inp.context_lens.clone()
    lens[:] = 0
    tables = np.full_like(inp.block_tables.numpy(), 10 ** 9)   # never read
    got = ora.paged_decode(raw_u16(inp.query), raw_u16(inp.key_cache), raw_u16(inp.value_cache),
                           tables, lens.numpy(), inp.scale, inp.block_size, None, dtype=inp.dtype)
    assert not got.any()


def pin_poison_ignored():
    dirty = _tiny(poison=True, seed=21)
    b = _oracle_on(dirty)
    assert np.isfinite(b).all()
    # replace every NaN slot (tails, unused blocks, the block unused table
    # entries point at) by finite values: the result must not move
    rng = _rng(9)
    kc = raw_u16(dirty.key_cache).copy()
    vc = raw_u16(dirty.value_cache).copy()
    for c in (kc, vc):
        nan = np.isnan(ora.to_float64(c, dirty.dtype))
        assert nan.any()
        c[nan] = rng.integers(0x3000, 0x4000, size=int(nan.sum()), dtype=np.uint16)
    a = ora.paged_decode(raw_u16(dirty.query), kc, vc, dirty.block_tables.numpy(),
                         dirty.context_lens.numpy(), dirty.scale, dirty.block_size,
                         dirty.alibi_slopes.numpy(), dtype=dirty.dtype)
    assert np.array_equal(a, b)


def pin_storage_formats():
    bf = np.array([0x3F80, 0xC000, 0x0001, 0x7F80, 0xFF80, 0x4049], dtype=np.uint16)
    want = [1.0, -2.0, 2.0 ** -133, math.inf, -math.inf, 3.140625]
    assert ora.to_float64(bf, "bf16").tolist() == want
    hf = np.array([0x3C00, 0x0001, 0x7BFF, 0xC400, 0x3555], dtype=np.uint16)
    want = [1.0, 2.0 ** -24, 65504.0, -4.0, 0.333251953125]
    assert ora.to_float64(hf, "f16").tolist() == want
    assert np.isnan(ora.to_float64(np.array([0x7FC0], np.uint16), "bf16")).all()
    # round-to-nearest-even at the bf16 half-way points around 1.0
    x = [1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20, -3.140625]
    assert ora.round_to_storage(x, "bf16").tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC049]
    x = [1.0, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 65520.0]
    assert ora.round_to_storage(x, "f16").tolist() == [0x3C00, 0x3C00, 0x3C02, 0x7C00]


def pin_cache_write_round_trip():
    """Written rows land where the layout says, others stay, negative slots skip."""
    rng = _rng(10)
    NB, Hkv, BS, D, T = 9, 3, 8, 4, 30
    kc = rng.integers(0, 1 << 16, size=(NB, Hkv, BS, D), dtype=np.uint16)
    vc = rng.integers(0, 1 << 16, size=(NB, Hkv, BS, D), dtype=np.uint16)
    k = rng.integers(0, 1 << 16, size=(T, Hkv, D), dtype=np.uint16)
    v = rng.integers(0, 1 << 16, size=(T, Hkv, D), dtype=np.uint16)
    slots = rng.permutation(NB * BS)[:T]
    slots[[3, 17]] = -1
    kc2, vc2 = ora.kv_cache_write(kc, vc, k, v, slots, BS)
    touched = np.zeros((NB, BS), dtype=bool)
    for i, slot in enumerate(slots):
        if slot < 0:
            continue
        b, o = divmod(int(slot), BS)          # block-major slot numbering
        assert np.array_equal(kc2[b, :, o, :], k[i]) and np.array_equal(vc2[b, :, o, :], v[i])
        touched[b, o] = True
    assert np.array_equal(kc2.transpose(0, 2, 1, 3)[~touched], kc.transpose(0, 2, 1, 3)[~touched])
    assert np.array_equal(vc2.transpose(0, 2, 1, 3)[~touched], vc.transpose(0, 2, 1, 3)[~touched])
    # the gather reads back exactly what was written
    kg, vg = ora.gather_cached_kv(kc2, vc2, slots, BS)
    ok = slots >= 0
    assert np.array_equal(kg[ok], k[ok]) and np.array_equal(vg[ok], v[ok])


def pin_fp8_format():
    """E4M3FN decoding: hand-worked codes and torch's float8_e4m3fn conversion."""
    want = {0x00: 0.0, 0x80: -0.0, 0x38: 1.0, 0xB8: -1.0, 0x7E: 448.0, 0x01: 2.0 ** -9,
            0x08: 2.0 ** -6, 0x07: 7 * 2.0 ** -9, 0x3C: 1.5, 0x54: 12.0, 0x41: 2.25}
    for code, val in want.items():
        got = ora.fp8_e4m3_value(code)
        assert got == val and math.copysign(1, got) == math.copysign(1, val), (code, got)
    assert math.isnan(ora.fp8_e4m3_value(0x7F)) and math.isnan(ora.fp8_e4m3_value(0xFF))
    codes = np.arange(256, dtype=np.uint8)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = ora.fp8_to_float64(codes)
    both_nan = np.isnan(lib) & np.isnan(ours)
    assert np.array_equal(lib[~both_nan], ours[~both_nan]) and both_nan.sum() == 2


def pin_fp8_cache_scales():
    """An fp8 cache with scales equals the float cache holding decoded * scale."""
    inp = decode_inputs(num_seqs=3, num_heads=4, num_kv_heads=2, head_size=16, block_size=8,
                        dtype="bf16", seed=5, context_lens=[3, 9, 17], alibi=True,
                        poison=True, kv_dtype="fp8", kv_scale=0.125)
    kraw = inp.key_cache.view(torch.uint8).numpy()
    vraw = inp.value_cache.view(torch.uint8).numpy()
    got = ora.paged_decode(raw_u16(inp.query), kraw, vraw, inp.block_tables.numpy(),
                           inp.context_lens.numpy(), inp.scale, 8, inp.alibi_slopes.numpy(),
                           dtype="bf16", k_scale=0.125, v_scale=0.25)
    kf = inp.key_cache.to(torch.float64).numpy() * 0.125    # library decoding of the bytes
    vf = inp.value_cache.to(torch.float64).numpy() * 0.25
    q = ora.to_float64(raw_u16(inp.query), "bf16")
    ref = ora.paged_decode(q, kf, vf, inp.block_tables.numpy(), inp.context_lens.numpy(),
                           inp.scale, 8, inp.alibi_slopes.numpy())
    assert np.isfinite(got).all() and np.array_equal(got, ref)


def _brute_prefill(q, kc, vc, tables, lens, qs, scale, BS, slopes):
    """Pure-Python causal attention: query i of s sees positions 0 .. L - n + i."""
    T, Hq, D = len(q), len(q[0]), len(q[0][0])
    Hkv = len(kc[0])
    head_mapping = [k for k in range(Hkv) for _ in range(Hq // Hkv)]
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(T)]
    for s in range(len(lens)):
        L, n = lens[s], qs[s + 1] - qs[s]
        for i in range(n):
            p = L - n + i
            for h in range(Hq):
                kvh = head_mapping[h]
                zs = []
                for t in range(p + 1):
                    blk, off = tables[s][t // BS], t % BS
                    z = scale * math.fsum(q[qs[s] + i][h][d] * kc[blk][kvh][off][d] for d in range(D))
                    if slopes is not None:
                        z += slopes[h] * (t - p)
                    zs.append(z)
                mx = max(zs)
                w = [math.exp(z - mx) for z in zs]
                den = math.fsum(w)
                for d in range(D):
                    out[qs[s] + i][h][d] = math.fsum(
                        w[t] * vc[tables[s][t // BS]][kvh][t % BS][d] for t in range(p + 1)) / den
    return np.array(out)


def _prefill_case(seed=13, lens=(5, 9, 1, 12), news=(3, 9, 1, 4), alibi=True, dtype="bf16"):
    inp = decode_inputs(num_seqs=len(lens), num_heads=6, num_kv_heads=2, head_size=8,
                        block_size=4, dtype=dtype, seed=seed, context_lens=list(lens),
                        alibi=alibi, poison=True)
    qs = np.concatenate([[0], np.cumsum(news)]).astype(np.int64)
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(int(qs[-1]), 6, 8, generator=g).to(inp.query.dtype)
    return inp, q, qs


def pin_prefill_brute_force():
    inp, q, qs = _prefill_case()
    f = lambda t: ora.to_float64(raw_u16(t), "bf16").tolist()   # noqa: E731
    slopes = [float(x) for x in inp.alibi_slopes.numpy()]
    ref = _brute_prefill(f(q), f(inp.key_cache), f(inp.value_cache), inp.block_tables.tolist(),
                         inp.context_lens.tolist(), qs.tolist(), inp.scale, 4, slopes)
    got = ora.paged_prefill(raw_u16(q), raw_u16(inp.key_cache), raw_u16(inp.value_cache),
                            inp.block_tables.numpy(), inp.context_lens.numpy(), qs, inp.scale, 4,
                            inp.alibi_slopes.numpy(), dtype="bf16")
    assert np.isfinite(got).all() and np.max(np.abs(got - ref)) <= 1e-12


def pin_prefill_last_token_is_decode():
    """Each sequence's last query row equals decode of that query over the whole context."""
    inp, q, qs = _prefill_case(alibi=True)
    got = ora.paged_prefill(raw_u16(q), raw_u16(inp.key_cache), raw_u16(inp.value_cache),
                            inp.block_tables.numpy(), inp.context_lens.numpy(), qs, inp.scale, 4,
                            inp.alibi_slopes.numpy(), dtype="bf16")
    last = raw_u16(q)[qs[1:] - 1]
    dec = ora.paged_decode(last, raw_u16(inp.key_cache), raw_u16(inp.value_cache),
                           inp.block_tables.numpy(), inp.context_lens.numpy(), inp.scale, 4,
                           inp.alibi_slopes.numpy(), dtype="bf16")
    assert np.array_equal(got[qs[1:] - 1], dec)


def pin_prefill_dense_causal_library():
    """Against SDPA with an explicit causal mask on dense K/V built by this test."""
    import torch.nn.functional as F
    rng = _rng(11)
    lens, news = [20, 7, 33], [6, 7, 1]
    Hq, Hkv, D, BS = 4, 2, 8, 8
    kc, vc, tables, dk, dv, _ = _scatter_dense(rng, lens, Hkv, D, BS)
    qs = np.concatenate([[0], np.cumsum(news)])
    q = rng.standard_normal((int(qs[-1]), Hq, D))
    got = ora.paged_prefill(q, kc, vc, tables, np.array(lens), qs, 0.4, BS)
    for s, (L, n) in enumerate(zip(lens, news)):
        idx = torch.tensor([h // (Hq // Hkv) for h in range(Hq)])
        K = torch.from_numpy(dk[s])[idx]
        V = torch.from_numpy(dv[s])[idx]
        Q = torch.from_numpy(q[qs[s]:qs[s] + n]).permute(1, 0, 2)       # [Hq, n, D]
        pos = torch.arange(L - n, L)[:, None]
        mask = torch.where(torch.arange(L)[None, :] <= pos, 0.0, float("-inf")).to(torch.float64)
        ref = F.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=0.4).permute(1, 0, 2)
        assert np.max(np.abs(got[qs[s]:qs[s] + n] - ref.numpy())) <= 1e-12


PINS = [
    pin_brute_force, pin_dense_library, pin_gather_by_construction,
    pin_sequence_kv_by_construction, pin_block_permutation, pin_context_one,
    pin_identical_keys_mean, pin_identical_keys_alibi, pin_needle, pin_gqa_equals_repeated_mha,
    pin_split_merge, pin_shift_and_linearity, pin_empty_context, pin_poison_ignored,
    pin_storage_formats, pin_cache_write_round_trip, pin_fp8_format, pin_fp8_cache_scales,
    pin_prefill_brute_force, pin_prefill_last_token_is_decode, pin_prefill_dense_causal_library,
]
