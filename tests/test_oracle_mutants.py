"""Plant plausible mistakes in the oracle (on the CPU) and check a pin catches each.

A pin suite that passes a wrong oracle pins nothing; every mutant below must
make at least one pin fail (or raise).
"""
import numpy as np
import pytest

import oracle.paged_attention as ora
from oracle_pins import PINS

_orig = {name: getattr(ora, name) for name in
         ("kv_head_of", "sequence_kv", "alibi_bias", "attend", "merge_partitions",
          "gather_cached_kv", "to_float64", "kv_cache_write", "fp8_to_float64",
          "query_position")}


def _kv_head_mod(h, Hq, Hkv):
    return h % Hkv


def _seq_drop_last(cache, row, L, BS):
    out = _orig["sequence_kv"](cache, row, L, BS)
    return out[:, :max(L - 1, 1)] if L > 1 else out * 0.5


def _seq_ignore_table(cache, row, L, BS):
    nb = (L + BS - 1) // BS
    return _orig["sequence_kv"](cache, np.arange(nb), L, BS)


def _seq_transposed_block(cache, row, L, BS):
    # reads the block as [BS, Hkv, D] instead of [Hkv, BS, D]
    nb = (L + BS - 1) // BS
    blocks = cache[np.asarray(row[:nb], dtype=np.int64)]
    Hkv, D = blocks.shape[1], blocks.shape[3]
    flat = blocks.reshape(nb, BS, Hkv, D).transpose(2, 0, 1, 3).reshape(Hkv, nb * BS, D)
    return flat[:, :L]


def _alibi_flipped(slope, L):
    return -_orig["alibi_bias"](slope, L)


def _alibi_off_by_one(slope, L):
    return float(slope) * (np.arange(L, dtype=np.float64) - L) * 1.5


def _attend_no_scale(q, K, V, scale, bias):
    return _orig["attend"](q, K, V, 1.0, bias)


def _attend_mean_norm(q, K, V, scale, bias):
    z = (K @ q) * scale + (0 if bias is None else bias)
    w = np.exp(z - z.max())
    return (w @ V) / len(w)


def _attend_kv_swapped(q, K, V, scale, bias):
    return _orig["attend"](q, V, K, scale, bias)


def _attend_bias_scaled(q, K, V, scale, bias):
    return _orig["attend"](q, K, V, scale, None if bias is None else bias * scale)


def _merge_no_rescale(stats):
    num = sum(l * o for _, l, o in stats)
    return num / sum(l for _, l, _ in stats)


def _gather_wrong_offset(kc, vc, slots, BS):
    slots = np.asarray(slots)
    shifted = np.where(slots >= 0, (slots // BS) * BS + (slots % BS + 1) % BS, slots)
    return _orig["gather_cached_kv"](kc, vc, shifted, BS)


def _gather_no_zero(kc, vc, slots, BS):
    k, v = _orig["gather_cached_kv"](kc, vc, slots, BS)
    neg = np.asarray(slots) < 0
    k[neg] = kc[0, :, 0, :]
    v[neg] = vc[0, :, 0, :]
    return k, v


def _to_f64_bf16_as_f16(raw, dtype):
    return _orig["to_float64"](raw, "f16")


def _write_offset_major(kc, vc, k, v, slots, BS):
    # treats the slot as offset-major (slot % NB, slot // NB): wrong numbering
    NB = kc.shape[0]
    kc2, vc2 = np.array(kc, copy=True), np.array(vc, copy=True)
    for i, slot in enumerate(np.asarray(slots).tolist()):
        if slot >= 0:
            kc2[slot % NB, :, slot // NB, :] = k[i]
            vc2[slot % NB, :, slot // NB, :] = v[i]
    return kc2, vc2


def _write_kv_swapped(kc, vc, k, v, slots, BS):
    return _orig["kv_cache_write"](kc, vc, v, k, slots, BS)


def _fp8_bias8(raw):
    return _orig["fp8_to_float64"](raw) / 2.0   # exponent bias 8 instead of 7


def _fp8_no_subnormals(raw):
    v = _orig["fp8_to_float64"](raw)
    return np.where((np.asarray(raw) & 0x78) == 0, 0.0, v)


def _position_off_by_one(L, n, i):
    return max(L - n + i - 1, 0)


def _position_first_token(L, n, i):
    return L - 1    # every new token sees the whole context (no causal mask)


MUTANTS = {
    "head_mapping_modulo": ("kv_head_of", _kv_head_mod),
    "drop_last_token": ("sequence_kv", _seq_drop_last),
    "ignore_block_table": ("sequence_kv", _seq_ignore_table),
    "transposed_block_layout": ("sequence_kv", _seq_transposed_block),
    "alibi_sign_flipped": ("alibi_bias", _alibi_flipped),
    "alibi_wrong_slope_scale": ("alibi_bias", _alibi_off_by_one),
    "missing_scale": ("attend", _attend_no_scale),
    "normalise_by_length": ("attend", _attend_mean_norm),
    "k_v_swapped": ("attend", _attend_kv_swapped),
    "bias_multiplied_by_scale": ("attend", _attend_bias_scaled),
    "merge_without_rescale": ("merge_partitions", _merge_no_rescale),
    "gather_wrong_offset": ("gather_cached_kv", _gather_wrong_offset),
    "gather_negative_slot_not_zeroed": ("gather_cached_kv", _gather_no_zero),
    "bf16_decoded_as_f16": ("to_float64", _to_f64_bf16_as_f16),
    "cache_write_offset_major": ("kv_cache_write", _write_offset_major),
    "cache_write_k_v_swapped": ("kv_cache_write", _write_kv_swapped),
    "fp8_exponent_bias_8": ("fp8_to_float64", _fp8_bias8),
    "fp8_subnormals_flushed": ("fp8_to_float64", _fp8_no_subnormals),
    "prefill_position_off_by_one": ("query_position", _position_off_by_one),
    "prefill_not_causal": ("query_position", _position_first_token),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(ora, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except Exception as e:   # AssertionError or any crash counts as caught
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin catches mutant {name}"
