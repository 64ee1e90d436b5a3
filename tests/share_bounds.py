"""Where the equal-share schedule cuts the batch: the host-side reading of the
rule the decode kernel follows (decode_attention_paged_06_amd/csrc/launch.h:
workgroup b of G takes stream positions [floor(b T / G), floor((b + 1) T / G)) of
the batch's tiles, walked kv head by kv head, sequence by sequence).  Used to
plant needles right at the cuts."""
from __future__ import annotations

import bisect

import numpy as np

from decode_attention_paged_06_amd import kv_layout_of, make_dims, make_opts, paged_attention_plan
from decode_attention_paged_06_amd.ops import share_occupancy


def launched(inp):
    """(workgroups, piece cost) of an equal-share call on `inp` on the current device."""
    dims = make_dims(inp.query, inp.key_cache, inp.block_tables, inp.k_scale, inp.v_scale,
                     kv_layout_of(inp.key_cache, inp.value_cache))
    p = paged_attention_plan(dims, 1 << 40, make_opts(0, "auto", schedule="equal_shares"))
    table, dev, cost = share_occupancy(dims)
    return p.num_partitions // table * min(dev, table), cost


def cuts(lens, num_kv_heads: int, block_size: int, wgs: int, cost: int) -> dict:
    """{sequence: sorted token positions where a share's tiles start inside it}.

    Each sequence takes `cost` stream positions before its tiles; a share that
    starts among those positions starts the sequence's tiles at tile 0."""
    tt = min(16, block_size)
    tiles = [max(0, (int(L) + tt - 1) // tt) for L in lens]
    starts = np.concatenate([[0], np.cumsum([n + cost for n in tiles])]).astype(np.int64)
    t1 = int(starts[-1])
    total = t1 * num_kv_heads
    wgs = min(wgs, total)  # shares of at least one position
    out: dict = {}
    for b in range(1, wgs):
        x = b * total // wgs
        o = x % t1
        s = bisect.bisect_right(starts.tolist(), o) - 1
        t = max(0, int(o - starts[s] - cost))
        if t < tiles[s]:
            out.setdefault(s, set()).add(t * tt)
    return {s: sorted(v) for s, v in out.items()}
