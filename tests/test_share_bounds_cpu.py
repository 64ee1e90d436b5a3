"""The host-side reading of the equal-share cuts (tests/share_bounds.py, used
to plant needles at the cuts on the GPU) against a walk of the position
stream one position at a time."""
import numpy as np

import share_bounds


def brute(lens, hkv, bs, wgs, cost):
    tt = min(16, bs)
    tiles = [(int(L) + tt - 1) // tt for L in lens]
    total = sum(n + cost for n in tiles) * hkv
    g = min(wgs, total)
    starts = {b * total // g for b in range(1, g)}
    out, x = {}, 0
    for _ in range(hkv):
        for s, n in enumerate(tiles):
            for k in range(cost + n):
                if x in starts:
                    t = max(0, k - cost)
                    if t < n:
                        out.setdefault(s, set()).add(t * tt)
                x += 1
    return {s: sorted(v) for s, v in out.items()}


def test_cuts_match_a_walk_of_the_stream():
    rng = np.random.default_rng(0)
    for trial in range(40):
        S = int(rng.integers(1, 30))
        lens = rng.integers(0, 900, S)
        if trial % 5 == 0:
            lens[rng.integers(0, S)] = 0
        hkv = int(rng.integers(1, 4))
        bs = int(rng.choice([8, 16, 64]))
        wgs = int(rng.integers(1, 300))
        cost = int(rng.integers(1, 30))
        assert share_bounds.cuts(lens, hkv, bs, wgs, cost) == brute(lens, hkv, bs, wgs, cost), \
            (lens.tolist(), hkv, bs, wgs, cost)
