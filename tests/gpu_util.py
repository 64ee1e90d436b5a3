"""Helpers for the GPU parity tests: run the HIP path, run the oracle, compare."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from decode_attention_paged_06_amd import paged_attention_decode
import parity_gate
from workloads import decode_inputs, raw_bits, raw_u16

# Max-abs tolerances against the fp64 oracle: fp16 2e-3, bf16 1e-2 (with the
# relative L2 bounds of parity_gate applied on top by compare()).
TOL = parity_gate.MAX_ABS


def device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def make(device_="cpu", **kw):
    return decode_inputs(device=device_, **kw)


def to_device(inp, dev):
    """Move a batch to `dev`, keeping joint K/V caches joint (one tensor, two views)."""
    k, v = inp.key_cache, inp.value_cache
    if not (k.is_contiguous() and v.is_contiguous()):
        NB, Hkv, BS, D = k.shape
        assert v.data_ptr() == k.data_ptr() + BS * D * k.element_size(), "not a joint cache"
        kv = torch.as_strided(k, (NB, Hkv, 2, BS, D), (2 * Hkv * BS * D, 2 * BS * D, BS * D, D, 1)).to(dev)
        inp.key_cache, inp.value_cache = kv[:, :, 0], kv[:, :, 1]
    else:
        inp.key_cache, inp.value_cache = k.to(dev), v.to(dev)
    for name in ("query", "block_tables", "context_lens", "alibi_slopes"):
        t = getattr(inp, name)
        if t is not None:
            setattr(inp, name, t.to(dev))
    return inp


def run(inp, engine="auto", partition_size=0, out=None, schedule="auto"):
    if out is None:
        out = torch.full_like(inp.query, float("nan"))
    paged_attention_decode(out, inp.query, inp.key_cache, inp.value_cache, inp.block_tables,
                           inp.context_lens, inp.scale, inp.block_size, inp.alibi_slopes,
                           partition_size=partition_size, engine=engine,
                           k_scale=inp.k_scale, v_scale=inp.v_scale, schedule=schedule)
    torch.cuda.synchronize()
    return out


def oracle_ref(inp, seqs=None):
    """Oracle output for `seqs` (all by default), copying only their blocks to the host."""
    S = inp.query.shape[0]
    seqs = list(range(S)) if seqs is None else list(seqs)
    BS = inp.block_size
    lens = inp.context_lens.cpu().numpy()
    tables = inp.block_tables.cpu().numpy()
    maxb = tables.shape[1]
    # compact pool: the used blocks of the sampled sequences, in table order
    phys, rows = [], []
    for s in seqs:
        L = min(int(lens[s]), maxb * BS)
        nb = (L + BS - 1) // BS if L > 0 else 0
        rows.append(list(range(len(phys), len(phys) + nb)) + [0] * (maxb - nb))
        phys.extend(int(x) for x in tables[s, :nb])
    if not phys:
        phys = [0]
    idx = torch.tensor(phys, dtype=torch.long, device=inp.key_cache.device)
    kc = raw_bits(inp.key_cache.view(torch.uint8 if inp.key_cache.element_size() == 1 else torch.int16).index_select(0, idx).view(inp.key_cache.dtype))
    vc = raw_bits(inp.value_cache.view(torch.uint8 if inp.value_cache.element_size() == 1 else torch.int16).index_select(0, idx).view(inp.value_cache.dtype))
    q = raw_u16(inp.query.index_select(0, torch.tensor(seqs, device=inp.query.device)))
    lens_s = np.minimum(lens[seqs], maxb * BS)
    slopes = None if inp.alibi_slopes is None else inp.alibi_slopes.cpu().numpy()
    return oracle.paged_decode(q, kc, vc, np.array(rows), lens_s, inp.scale, BS, slopes,
                               dtype=inp.dtype, k_scale=inp.k_scale, v_scale=inp.v_scale)


def compare(got: torch.Tensor, ref: np.ndarray, dtype: str, seqs=None, what=""):
    """The parity gate (max-abs, whole-output and per-row relative L2; see
    parity_gate) of a device result against the oracle, on rows `seqs`."""
    g = got.float().cpu().numpy()
    if seqs is not None:
        g = g[list(seqs)]
    max_abs, rel, _ = parity_gate.check(g, ref, dtype, what)
    return max_abs, rel


def sample_seqs(S, k=16, seed=0):
    if S <= k:
        return list(range(S))
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, S - 1), size=k - 2, replace=False)
    return [0] + sorted(int(x) for x in mid) + [S - 1]
