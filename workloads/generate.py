"""Seeded synthetic inputs for paged decode attention and the paged-KV gather.

This module only draws random numbers and lays them out in the paged-cache
format; it performs none of the attention arithmetic.  Both the CPU oracle
tests and the GPU tests/bench build their inputs here, so the two sides see
identical bytes for identical seeds and devices.

Layout (the contract of the library in ``include/paged_attention.h``):
  query        [S, Hq, D]            fp16 or bf16
  key_cache    [NB, Hkv, BS, D]      fp16 or bf16 (or fp8)
  value_cache  [NB, Hkv, BS, D]      fp16 or bf16 (or fp8)
               two dense tensors, or (kv_layout="joint") the K and V views of
               one [NB, Hkv, 2, BS, D] tensor holding the same bytes
  block_tables [S, MAXB]             int32, physical block ids
  context_lens [S]                   int32
  alibi_slopes [Hq]                  fp32 (optional)

Randomness:
  * lengths, block assignment and table padding come from a CPU generator
    seeded with ``seed`` (identical on every device);
  * q/K/V values are N(0, 1) draws in fp32 from a generator on ``device``
    seeded with ``seed + 1``, then rounded to the storage dtype by torch's
    round-to-nearest-even conversion.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional, Sequence, Union

import numpy as np
import torch

DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}

LengthSpec = Union[int, tuple, Sequence[int]]


@dataclass
class DecodeInputs:
    query: torch.Tensor
    key_cache: torch.Tensor
    value_cache: torch.Tensor
    block_tables: torch.Tensor
    context_lens: torch.Tensor
    alibi_slopes: Optional[torch.Tensor]
    scale: float
    block_size: int
    dtype: str
    seed: int
    num_blocks_used: int
    poison_block: Optional[int] = None
    kv_dtype: str = ""
    k_scale: float = 1.0
    v_scale: float = 1.0
    meta: dict = field(default_factory=dict)

    @property
    def dims(self):
        S, Hq, D = self.query.shape
        NB, Hkv, BS, _ = self.key_cache.shape
        return dict(num_seqs=S, num_heads=Hq, num_kv_heads=Hkv, head_size=D,
                    block_size=BS, num_blocks=NB,
                    max_blocks_per_seq=self.block_tables.shape[1], dtype=self.dtype)


def alibi_slopes_geometric(num_heads: int) -> torch.Tensor:
    """Slopes 2^(-8 i / num_heads), i = 1..num_heads, stored as fp32."""
    return torch.tensor([2.0 ** (-8.0 * i / num_heads) for i in range(1, num_heads + 1)],
                        dtype=torch.float32)


def _lengths(spec: LengthSpec, num_seqs: int, gen: torch.Generator) -> torch.Tensor:
    if isinstance(spec, int):
        return torch.full((num_seqs,), spec, dtype=torch.int32)
    if isinstance(spec, tuple) and len(spec) == 2:
        lo, hi = spec
        return torch.randint(lo, hi + 1, (num_seqs,), generator=gen, dtype=torch.int64).to(torch.int32)
    lens = torch.tensor(list(spec), dtype=torch.int32)
    assert lens.numel() == num_seqs
    return lens


def _randn(shape, dtype: str, gen: torch.Generator, device, scale: float = 1.0) -> torch.Tensor:
    """N(0, 1) draws divided by `scale`, rounded to `dtype` (RNE; fp8 is E4M3FN).

    Draws in bounded chunks along dim 0 so that very large pools do not need a
    full-size fp32 temporary.
    """
    out = torch.empty(shape, dtype=DTYPES[dtype], device=device)
    if len(shape) == 0 or shape[0] == 0:
        return out
    row = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    step = max(1, (1 << 27) // max(row, 1))
    for i in range(0, shape[0], step):
        j = min(shape[0], i + step)
        x = torch.randn((j - i,) + tuple(shape[1:]), generator=gen, dtype=torch.float32,
                        device=device)
        if scale != 1.0:
            x = x / scale
        out[i:j] = x.to(DTYPES[dtype])
    return out


def decode_inputs(*, num_seqs: int, num_heads: int, num_kv_heads: int, head_size: int,
                  block_size: int, dtype: str, seed: int, context_lens: LengthSpec,
                  pool_blocks: Optional[int] = None, max_blocks_per_seq: Optional[int] = None,
                  alibi: bool = False, scale: Optional[float] = None, poison: bool = False,
                  device: Union[str, torch.device] = "cpu", kv_dtype: Optional[str] = None,
                  kv_scale: float = 0.0625, kv_layout: str = "separate") -> DecodeInputs:
    """Build one seeded decode batch.

    pool_blocks=None sizes the pool to fit exactly the blocks the sequences
    use (plus one all-NaN block when ``poison``).  Every used block is
    distinct; the assignment is a random permutation of the pool.

    kv_dtype="fp8" stores K and V as FP8 E4M3 with one scale per cache:
    the real value is code * kv_scale (draws are divided by kv_scale before
    rounding, so the real values stay ~N(0, 1)).

    kv_layout="joint" returns K and V as the two views of one [NB, Hkv, 2, BS,
    D] tensor (same values as "separate").

    poison=True writes NaN into every cache slot no valid token occupies
    (tail slots of each last block and all unused pool blocks) and points
    every unused table entry at an all-NaN block.  A kernel that reads
    anything outside the valid tokens then produces NaN.
    """
    device = torch.device(device)
    cpu = torch.Generator().manual_seed(seed)
    lens = _lengths(context_lens, num_seqs, cpu)
    nblk = [(int(L) + block_size - 1) // block_size for L in lens.tolist()]
    used = sum(nblk)
    maxb = max_blocks_per_seq if max_blocks_per_seq is not None else max(1, max(nblk, default=1))
    assert maxb >= max(nblk, default=0), "max_blocks_per_seq too small for the lengths"
    need = used + (1 if poison else 0)
    NB = pool_blocks if pool_blocks is not None else max(need, 1)
    assert NB >= need, "pool too small"

    perm = torch.randperm(NB, generator=cpu).to(torch.int32)
    poison_block = int(perm[used].item()) if poison else None
    tables = torch.randint(0, NB, (num_seqs, maxb), generator=cpu, dtype=torch.int64).to(torch.int32)
    if poison:
        tables.fill_(poison_block)
    pos = 0
    for s, nb in enumerate(nblk):
        tables[s, :nb] = perm[pos:pos + nb]
        pos += nb

    dev = torch.Generator(device=device).manual_seed(seed + 1)
    kv_dtype = kv_dtype or dtype
    kv_s = kv_scale if kv_dtype == "fp8" else 1.0
    q = _randn((num_seqs, num_heads, head_size), dtype, dev, device)
    kc = _randn((NB, num_kv_heads, block_size, head_size), kv_dtype, dev, device, kv_s)
    vc = _randn((NB, num_kv_heads, block_size, head_size), kv_dtype, dev, device, kv_s)

    if poison:
        nan = float("nan")
        used_mask = torch.zeros(NB, dtype=torch.bool)
        used_mask[perm[:used].long()] = True
        unused = (~used_mask).nonzero().flatten().to(device)
        kc[unused] = nan
        vc[unused] = nan
        for s, (L, nb) in enumerate(zip(lens.tolist(), nblk)):
            if nb == 0:
                continue
            last = int(tables[s, nb - 1])
            tail = L - (nb - 1) * block_size
            if tail < block_size:
                kc[last, :, tail:, :] = nan
                vc[last, :, tail:, :] = nan

    kc, vc = _lay_out(kc, vc, kv_layout)
    slopes = alibi_slopes_geometric(num_heads).to(device) if alibi else None
    if scale is None:
        scale = 1.0 / math.sqrt(head_size)
    return DecodeInputs(query=q, key_cache=kc, value_cache=vc,
                        block_tables=tables.to(device), context_lens=lens.to(device),
                        alibi_slopes=slopes, scale=float(scale), block_size=block_size,
                        dtype=dtype, seed=seed, num_blocks_used=used,
                        poison_block=poison_block, kv_dtype=kv_dtype, k_scale=kv_s,
                        v_scale=kv_s)


def _lay_out(kc: torch.Tensor, vc: torch.Tensor, kv_layout: str):
    """The caches as two dense tensors, or as the K and V views of one joint tensor."""
    if kv_layout == "separate":
        return kc, vc
    assert kv_layout == "joint", kv_layout
    kv = torch.stack([kc, vc], dim=2)   # [NB, Hkv, 2, BS, D], dense
    return kv[:, :, 0], kv[:, :, 1]


@dataclass
class GatherInputs:
    key_cache: torch.Tensor
    value_cache: torch.Tensor
    slot_mapping: torch.Tensor
    block_size: int
    dtype: str
    seed: int


def gather_inputs(*, num_tokens: int, num_kv_heads: int, head_size: int, block_size: int,
                  num_blocks: int, dtype: str, seed: int, random_bits: bool = False,
                  num_negative: int = 0, device: Union[str, torch.device] = "cpu",
                  kv_layout: str = "separate") -> GatherInputs:
    """Pool plus a slot mapping of distinct random slots.

    random_bits=True fills the pool with uniformly random 16-bit patterns
    (NaN and Inf encodings included) so a copy that converts values instead
    of moving bits is caught.  ``num_negative`` slots are set to -1.
    """
    device = torch.device(device)
    cpu = torch.Generator().manual_seed(seed)
    total = num_blocks * block_size
    assert num_tokens <= total
    slots = torch.randperm(total, generator=cpu)[:num_tokens].to(torch.int32)
    if num_negative:
        idx = torch.randperm(num_tokens, generator=cpu)[:num_negative]
        slots[idx] = -1
    shape = (num_blocks, num_kv_heads, block_size, head_size)
    dev = torch.Generator(device=device).manual_seed(seed + 1)
    if random_bits:
        kc = torch.randint(-32768, 32768, shape, generator=dev, dtype=torch.int32,
                           device=device).to(torch.int16).view(DTYPES[dtype])
        vc = torch.randint(-32768, 32768, shape, generator=dev, dtype=torch.int32,
                           device=device).to(torch.int16).view(DTYPES[dtype])
    else:
        kc = _randn(shape, dtype, dev, device)
        vc = _randn(shape, dtype, dev, device)
    kc, vc = _lay_out(kc, vc, kv_layout)
    return GatherInputs(key_cache=kc, value_cache=vc, slot_mapping=slots.to(device),
                        block_size=block_size, dtype=dtype, seed=seed)


def raw_u16(t: torch.Tensor) -> np.ndarray:
    """The storage bits of a 16-bit float tensor as a host uint16 array."""
    assert t.element_size() == 2
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def raw_bits(t: torch.Tensor) -> np.ndarray:
    """Storage bits of a 16-bit (uint16) or 8-bit (uint8) float tensor on the host."""
    if t.element_size() == 1:
        return t.detach().contiguous().cpu().view(torch.uint8).numpy()
    return raw_u16(t)


def prefill_inputs(*, new_tokens, seed: int, device: Union[str, torch.device] = "cpu",
                   **decode_kwargs):
    """A multi-query batch: decode_inputs for the caches plus packed new-token queries.

    new_tokens gives n_s per sequence (each <= its context length): the last
    n_s context tokens of sequence s are its new tokens.  Returns
    (inputs, query [T, Hq, D], query_start [S + 1] int32, max_query_len).
    """
    inp = decode_inputs(seed=seed, device=device, **decode_kwargs)
    news = [int(n) for n in new_tokens]
    lens = inp.context_lens.cpu().tolist()
    assert len(news) == len(lens) and all(0 <= n <= L for n, L in zip(news, lens))
    starts = torch.tensor([0] + list(np.cumsum(news)), dtype=torch.int32)
    g = torch.Generator(device=torch.device(device)).manual_seed(seed + 2)
    q = _randn((int(starts[-1]), inp.query.shape[1], inp.query.shape[2]), inp.dtype, g,
               torch.device(device))
    return inp, q, starts.to(device), max(news + [1])
