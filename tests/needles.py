"""Needle queries: q[s, h] = c K[s, kv(h), t*] puts (almost) all softmax weight
on one chosen token t*, so the exact output is V[s, kv(h), t*].  A kernel that
reads a wrong tile, a wrong row of a tile, a wrong block-table entry or a
wrong partition for that token is then off by an O(1) amount in that row,
whatever the context length -- the indexing pin of the decode path.

The strength c of each needle is set from the key itself and, with ALiBi, from
the bias the needle has to overcome: the needle's logit beats every other
token's by at least MARGIN (natural-log units), so its weight is at least
1 - L e^-MARGIN.  Works on CPU or device tensors (the inputs of
workloads.decode_inputs); only plain indexing, no attention arithmetic.
"""
from __future__ import annotations

import math

import numpy as np
import torch

MARGIN = 30.0


def _rows(cache: torch.Tensor, blocks, heads, offsets) -> torch.Tensor:
    """cache[blocks[i], heads[i], offsets[i], :] as float64 on the host."""
    dev = cache.device
    b = torch.as_tensor(blocks, dtype=torch.long, device=dev)
    h = torch.as_tensor(heads, dtype=torch.long, device=dev)
    o = torch.as_tensor(offsets, dtype=torch.long, device=dev)
    return cache[b, h, o].to(torch.float32).double().cpu()


def plant(inp, positions: dict) -> dict:
    """Write needle queries into inp.query for positions {s: [t* of head 0..Hq-1]}.

    Returns {"seqs": sorted sequences, "t": {s: [...]}, "v": {s: float64 [Hq, D]}}
    where v holds the value row each needle points at (times v_scale): the
    output the needle forces.
    """
    S, Hq, D = inp.query.shape
    Hkv = inp.key_cache.shape[1]
    G = Hq // Hkv
    BS = inp.block_size
    tables = inp.block_tables.cpu().numpy()
    lens = inp.context_lens.cpu().numpy()
    slopes = None if inp.alibi_slopes is None else inp.alibi_slopes.cpu().numpy().astype(np.float64)
    seqs = sorted(positions)
    blocks, heads, offs, where = [], [], [], []
    for s in seqs:
        ts = positions[s]
        assert len(ts) == Hq
        for h, t in enumerate(ts):
            assert 0 <= t < lens[s], (s, h, t, lens[s])
            blocks.append(int(tables[s, t // BS]))
            heads.append(h // G)
            offs.append(t % BS)
            where.append((s, h, t))
    K = _rows(inp.key_cache, blocks, heads, offs) * float(np.float32(inp.k_scale))
    V = _rows(inp.value_cache, blocks, heads, offs) * float(np.float32(inp.v_scale))
    q = torch.empty((len(where), D), dtype=torch.float64)
    for i, (s, h, t) in enumerate(where):
        k = K[i]
        n2 = float(k @ k)
        # other keys: k.K_t ~ N(0, |k|^2) for independent N(0, 1) keys; 6 sigma
        # covers any context here
        gain = inp.scale * (n2 - 6.0 * math.sqrt(n2))
        assert gain > 0, "key too short for a needle"
        bias_gap = 0.0 if slopes is None else slopes[h] * (int(lens[s]) - 1 - t)
        q[i] = k * ((MARGIN + bias_gap) / gain)
    sidx = torch.tensor([w[0] for w in where], dtype=torch.long, device=inp.query.device)
    hidx = torch.tensor([w[1] for w in where], dtype=torch.long, device=inp.query.device)
    inp.query[sidx, hidx] = q.to(inp.query.dtype).to(inp.query.device)
    vout = {s: np.zeros((Hq, D)) for s in seqs}
    for i, (s, h, t) in enumerate(where):
        vout[s][h] = V[i].numpy()
    return {"seqs": seqs, "t": {s: list(positions[s]) for s in seqs}, "v": vout}


def positions_for(L: int, Hq: int, block_size: int, boundaries=(), seed: int = 0) -> list:
    """One t* per query head: the edges of the first blocks and tiles, each
    partition boundary +-1, the last token, then seeded random positions;
    all clipped to [0, L)."""
    base = [0, 1, block_size - 1, block_size, block_size + 1, 15, 16, 17, L - 1, L - 2]
    for b in boundaries:
        base += [b - 1, b, b + 1]
    base = [t for t in dict.fromkeys(base) if 0 <= t < L]
    rng = np.random.default_rng(seed)
    while len(base) < Hq:
        base.append(int(rng.integers(0, L)))
    order = rng.permutation(Hq)
    return [base[i] for i in order] if len(base) == Hq else [base[i] for i in order[:Hq]]
