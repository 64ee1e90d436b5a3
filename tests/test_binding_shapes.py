"""The Python binding rejects tensors whose shapes do not match before any
pointer reaches the C layer (which sees only pointers and would read or write
past an allocation).  Host tensors suffice: the shape checks come first."""
import pytest
import torch

from decode_attention_paged_06_amd import (gather_cached_kv, paged_attention_decode,
                                           paged_attention_prefill, paged_kv_cache_write)

S, HQ, HKV, D, BS, NB, MAXB = 3, 8, 2, 128, 16, 10, 4


def decode_args(**over):
    a = dict(out=torch.zeros(S, HQ, D, dtype=torch.bfloat16),
             query=torch.zeros(S, HQ, D, dtype=torch.bfloat16),
             key_cache=torch.zeros(NB, HKV, BS, D, dtype=torch.bfloat16),
             value_cache=torch.zeros(NB, HKV, BS, D, dtype=torch.bfloat16),
             block_tables=torch.zeros(S, MAXB, dtype=torch.int32),
             context_lens=torch.ones(S, dtype=torch.int32),
             scale=0.1, block_size=BS, alibi_slopes=None)
    a.update(over)
    return a


def test_well_shaped_host_tensors_reach_the_device_check():
    with pytest.raises(ValueError, match="device tensor"):
        paged_attention_decode(**decode_args())


@pytest.mark.parametrize("over,msg", [
    (dict(out=torch.zeros(S - 1, HQ, D, dtype=torch.bfloat16)), "out"),
    (dict(out=torch.zeros(S, HQ, 64, dtype=torch.bfloat16)), "out"),
    (dict(key_cache=torch.zeros(NB, HKV, BS, 64, dtype=torch.bfloat16),
          value_cache=torch.zeros(NB, HKV, BS, 64, dtype=torch.bfloat16)), "head_size"),
    (dict(value_cache=torch.zeros(NB + 1, HKV, BS, D, dtype=torch.bfloat16)), "key_cache"),
    (dict(block_tables=torch.zeros(S - 1, MAXB, dtype=torch.int32)), "block_tables"),
    (dict(block_tables=torch.zeros(S * MAXB, dtype=torch.int32)), "block_tables"),
    (dict(context_lens=torch.ones(S + 1, dtype=torch.int32)), "context_lens"),
    (dict(alibi_slopes=torch.ones(HQ - 1, dtype=torch.float32)), "alibi_slopes"),
])
def test_decode_shape_mismatch_raises(over, msg):
    with pytest.raises(ValueError, match=msg):
        paged_attention_decode(**decode_args(**over))


def test_prefill_shape_mismatch_raises():
    T = 5
    a = decode_args(out=torch.zeros(T, HQ, D, dtype=torch.bfloat16),
                    query=torch.zeros(T, HQ, D, dtype=torch.bfloat16))
    a["query_start_loc"] = torch.tensor([0, 2, 5], dtype=torch.int32)   # S + 1 = 4 needed
    a["max_query_len"] = 3
    with pytest.raises(ValueError, match="query_start_loc"):
        paged_attention_prefill(**a)
    a["query_start_loc"] = torch.tensor([0, 2, 4, 5], dtype=torch.int32)
    a["out"] = torch.zeros(T + 1, HQ, D, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="out"):
        paged_attention_prefill(**a)


@pytest.mark.parametrize("fn", [gather_cached_kv, paged_kv_cache_write])
def test_row_copy_shape_mismatch_raises(fn):
    kc = torch.zeros(NB, HKV, BS, D, dtype=torch.float16)
    vc = torch.zeros_like(kc)
    slots = torch.zeros(6, dtype=torch.int32)
    good = torch.zeros(6, HKV, D, dtype=torch.float16)
    for rows, msg in ((torch.zeros(5, HKV, D, dtype=torch.float16), "rows"),
                      (torch.zeros(6, HKV + 1, D, dtype=torch.float16), "rows"),
                      (torch.zeros(6, HKV, 64, dtype=torch.float16), "rows")):
        with pytest.raises(ValueError, match=msg):
            fn(rows, good, kc, vc, slots, BS) if fn is gather_cached_kv else fn(kc, vc, rows, good, slots, BS)
    with pytest.raises(ValueError, match="slot_mapping"):
        args = (good, good, kc, vc, slots.view(2, 3), BS)
        fn(*args) if fn is gather_cached_kv else fn(kc, vc, good, good, slots.view(2, 3), BS)
