"""The bench's copy-throughput convention against numbers the gather page prints.

The page prints, per token count, a latency (rounded to 1 us) and a
throughput.  Reading A12: the throughput counts the K and V bytes of the
gathered rows once, in GiB/s.  Every printed pair must agree with that
convention to within the latency's rounding.
"""
import os

import bench

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "gather_benchmark_vllm_pr29.txt")


def rows():
    for line in open(GOLDEN):
        if line.strip() and not line.startswith("#"):
            t, ms, gbs = line.split()
            yield int(t), float(ms), float(gbs)


def test_printed_gather_throughput_matches_unit_convention():
    n = 0
    for tokens, ms, printed in rows():
        kv_bytes = bench.copy_bytes_once(tokens, num_kv_heads=40, head_size=128, elem_bytes=2)
        implied_ms = kv_bytes / (printed * 2 ** 30) * 1e3
        assert abs(implied_ms - ms) <= 0.0005 + 1e-9, (tokens, implied_ms, ms)
        # the decimal read+write figure the bench reports is 2 * 2^30 / 1e9 times larger
        assert abs(bench.pages_gib_per_s(tokens, 40, 128, 2, implied_ms * 1e-3) - printed) < 1e-6
        n += 1
    assert n == 6
