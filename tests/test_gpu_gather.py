"""GPU parity of gather_cached_kv: bit-exact against the oracle's raw copy."""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_paged_06_amd import gather_cached_kv
from gpu_util import device
from workloads import gather_inputs, raw_u16

pytestmark = pytest.mark.gpu

CASES = [
    # tokens, kv heads, head size, block size, blocks, dtype, negative slots
    (64, 40, 128, 8, 1024, "f16", 0),     # the gather benchmark's shape, smallest batch
    (2048, 40, 128, 8, 1024, "f16", 0),   # ... and its largest
    (1000, 8, 128, 16, 4096, "bf16", 7),
    (333, 1, 64, 16, 64, "f16", 3),
    (17, 3, 8, 5, 11, "bf16", 2),
]


@pytest.mark.parametrize("case", CASES, ids=[f"T{c[0]}-H{c[1]}-D{c[2]}-BS{c[3]}" for c in CASES])
@pytest.mark.parametrize("random_bits", [False, True])
def test_gather_bit_exact(case, random_bits):
    dev = device()
    T, H, D, BS, NB, dtype, neg = case
    g = gather_inputs(num_tokens=T, num_kv_heads=H, head_size=D, block_size=BS, num_blocks=NB,
                      dtype=dtype, seed=T + H, random_bits=random_bits, num_negative=neg,
                      device=dev)
    ko = torch.empty((T, H, D), dtype=g.key_cache.dtype, device=dev)
    vo = torch.empty_like(ko)
    ko.view(torch.int16).fill_(0x5555)   # the kernel must overwrite every row
    vo.view(torch.int16).fill_(0x5555)
    gather_cached_kv(ko, vo, g.key_cache, g.value_cache, g.slot_mapping, BS)
    torch.cuda.synchronize()
    rk, rv = oracle.gather_cached_kv(raw_u16(g.key_cache), raw_u16(g.value_cache),
                                     g.slot_mapping.cpu().numpy(), BS)
    assert np.array_equal(raw_u16(ko), rk)
    assert np.array_equal(raw_u16(vo), rv)


WRITE_CASES = [
    # tokens, kv heads, head size, block size, blocks, dtype, negative slots
    (256, 8, 128, 16, 4096, "bf16", 0),    # one decode step of a 256-sequence batch
    (4096, 8, 128, 16, 1024, "bf16", 9),   # a prefill chunk
    (333, 40, 128, 8, 1024, "f16", 3),
    (17, 3, 8, 5, 11, "f16", 2),
]


@pytest.mark.parametrize("case", WRITE_CASES,
                         ids=[f"T{c[0]}-H{c[1]}-D{c[2]}-BS{c[3]}" for c in WRITE_CASES])
def test_cache_write_bit_exact_and_round_trip(case):
    from decode_attention_paged_06_amd import paged_kv_cache_write
    dev = device()
    T, H, D, BS, NB, dtype, neg = case
    g = gather_inputs(num_tokens=T, num_kv_heads=H, head_size=D, block_size=BS, num_blocks=NB,
                      dtype=dtype, seed=7 * T + H, random_bits=True, num_negative=neg, device=dev)
    gen = torch.Generator(device=dev).manual_seed(T)
    k = torch.randint(-32768, 32768, (T, H, D), generator=gen, dtype=torch.int32,
                      device=dev).to(torch.int16).view(g.key_cache.dtype)
    v = torch.randint(-32768, 32768, (T, H, D), generator=gen, dtype=torch.int32,
                      device=dev).to(torch.int16).view(g.key_cache.dtype)
    before_k, before_v = raw_u16(g.key_cache), raw_u16(g.value_cache)
    paged_kv_cache_write(g.key_cache, g.value_cache, k, v, g.slot_mapping, BS)
    torch.cuda.synchronize()
    rk, rv = oracle.kv_cache_write(before_k, before_v, raw_u16(k), raw_u16(v),
                                   g.slot_mapping.cpu().numpy(), BS)
    assert np.array_equal(raw_u16(g.key_cache), rk)
    assert np.array_equal(raw_u16(g.value_cache), rv)
    # reading the same slots back returns the written rows
    ko = torch.empty_like(k)
    vo = torch.empty_like(v)
    gather_cached_kv(ko, vo, g.key_cache, g.value_cache, g.slot_mapping, BS)
    torch.cuda.synchronize()
    ok = (g.slot_mapping >= 0).cpu().numpy()
    assert np.array_equal(raw_u16(ko)[ok], raw_u16(k)[ok])
    assert np.array_equal(raw_u16(vo)[ok], raw_u16(v)[ok])


def test_fp8_rows_copy_bit_exact():
    """Gather and cache write move FP8 bytes unchanged (NaN codes included)."""
    from decode_attention_paged_06_amd import paged_kv_cache_write
    dev = device()
    T, H, D, BS, NB = 300, 8, 128, 16, 64
    gen = torch.Generator(device=dev).manual_seed(5)
    kc = torch.randint(0, 256, (NB, H, BS, D), generator=gen, dtype=torch.int32,
                       device=dev).to(torch.uint8).view(torch.float8_e4m3fn)
    vc = torch.randint(0, 256, (NB, H, BS, D), generator=gen, dtype=torch.int32,
                       device=dev).to(torch.uint8).view(torch.float8_e4m3fn)
    slots = torch.randperm(NB * BS, generator=torch.Generator().manual_seed(2))[:T].to(torch.int32)
    slots[7] = -1
    slots = slots.to(dev)
    ko = torch.empty((T, H, D), dtype=torch.float8_e4m3fn, device=dev)
    vo = torch.empty_like(ko)
    gather_cached_kv(ko, vo, kc, vc, slots, BS)
    torch.cuda.synchronize()
    kb = kc.view(torch.uint8).cpu().numpy()
    vb = vc.view(torch.uint8).cpu().numpy()
    rk, rv = oracle.gather_cached_kv(kb, vb, slots.cpu().numpy(), BS)
    assert np.array_equal(ko.view(torch.uint8).cpu().numpy(), rk)
    assert np.array_equal(vo.view(torch.uint8).cpu().numpy(), rv)
    nk = torch.randint(0, 256, (T, H, D), generator=gen, dtype=torch.int32,
                       device=dev).to(torch.uint8).view(torch.float8_e4m3fn)
    nv = torch.randint(0, 256, (T, H, D), generator=gen, dtype=torch.int32,
                       device=dev).to(torch.uint8).view(torch.float8_e4m3fn)
    paged_kv_cache_write(kc, vc, nk, nv, slots, BS)
    torch.cuda.synchronize()
    wk, wv = oracle.kv_cache_write(kb, vb, nk.view(torch.uint8).cpu().numpy(),
                                   nv.view(torch.uint8).cpu().numpy(), slots.cpu().numpy(), BS)
    assert np.array_equal(kc.view(torch.uint8).cpu().numpy(), wk)
    assert np.array_equal(vc.view(torch.uint8).cpu().numpy(), wv)
