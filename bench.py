"""Benchmark: paged decode attention on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME --batch B]

A step is one paged_attention_decode call (validation, plan, decode kernel and,
for split plans, the partition-reduce kernel) over one synthetic batch already
resident in HBM.  Prints ONE JSON line on stdout.

value = algorithmic bytes per call / time per call (GB/s, decimal), where the
algorithmic bytes are K and V of every context token once per kv head, q in,
out back, one block-table entry per used block and the context lengths
(plus the slopes with ALiBi).

The caches are laid out joint by default (one [NB, Hkv, 2, BS, D] tensor: the
K and V tiles of each block and kv head side by side); --kv-layout separate
times two [NB, Hkv, BS, D] tensors.  Results are identical either way.

Caches are defeated by rotating over independent input sets whose combined
footprint is at least 2 GiB (the headline workload alone is 4.3 GB, so it
uses a single set).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, vendor peak
ROTATE_BYTES = 2 << 30          # >= 8x the 256 MB last-level cache
METRIC = "paged-attn decode µs/call + achieved HBM GB/s (% of peak), GQA 64q/8kv bf16"
# Context from the reference pages (A100-40GB-PCIE, bf16, 64q/8kv, ctx 4096,
# batch 256): FlashAttention decode 2583.970 us, paged attention V1 8771.168 us.
PAGES_US = {("gqa_ctx4096", 256): {"flash_attention_a100_us": 2583.970, "paged_v1_a100_us": 8771.168}}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--batch", type=int, default=None)
    ap.add_argument("--engine", default="auto", choices=["auto", "valu", "mfma"])
    ap.add_argument("--partition-size", type=int, default=0)
    ap.add_argument("--schedule", default="auto", choices=["auto", "grid", "longest_first", "equal_shares"],
                    help="layout of a split plan's work over workgroups (see pa_schedule)")
    ap.add_argument("--kv-dtype", default=None, choices=["fp8"],
                    help="store the K/V caches as FP8 E4M3 (scale 1/16) instead of the query type")
    ap.add_argument("--kv-layout", default="joint", choices=["joint", "separate"],
                    help="cache layout: one [NB, Hkv, 2, BS, D] tensor (K and V tiles of each "
                         "block and kv head side by side) or two [NB, Hkv, BS, D] tensors")
    ap.add_argument("--block-size", type=int, default=0,
                    help="override the workload's cache block size (tokens per block)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU time budget of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--hot", action="store_true",
                    help="time one input set over and over (no rotation): a labelled hot-cache "
                         "figure for workloads that fit the last-level cache")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the device-copy / streaming-read ceiling measured after the timed region")
    ap.add_argument("--graph", action="store_true",
                    help="also time the calls replayed from a HIP graph (GPU time without the "
                         "host launch path; matters for small, launch-bound batches)")
    ap.add_argument("--grid", action="store_true",
                    help="also time every workload and batch of the configuration list (on by "
                         "default for the headline invocation)")
    ap.add_argument("--no-grid", action="store_true", help="skip the configuration grid")
    ap.add_argument("--context", type=int, default=4096, help="context per sequence for --op prefill")
    ap.add_argument("--new-tokens", type=int, default=512, help="new tokens per sequence for --op prefill")
    ap.add_argument("--op", default="decode", choices=["decode", "gather", "cache_write", "prefill"],
                    help="decode (default), or one of the row-copy kernels at the gather "
                         "page's shapes (40 heads, D 128, block 8, 1024 blocks, fp16)")
    ap.add_argument("--tokens", type=int, default=2048, help="rows per call for --op gather/cache_write")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="instead of decoding, run --steps device-to-device copies of MIB MiB "
                         "(reference kernel for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def copy_bytes_once(num_tokens, num_kv_heads, head_size, elem_bytes):
    """K and V bytes of num_tokens rows, each counted once."""
    return 2 * num_tokens * num_kv_heads * head_size * elem_bytes


def pages_gib_per_s(num_tokens, num_kv_heads, head_size, elem_bytes, seconds):
    """The gather page's throughput convention: K+V bytes once, in GiB/s."""
    return copy_bytes_once(num_tokens, num_kv_heads, head_size, elem_bytes) / seconds / 2 ** 30


def cpu_baseline_copy(op, num_tokens, budget_s):
    """The oracle's row copy (numpy fancy indexing of raw words) at the same shapes."""
    import oracle
    from workloads import gather_inputs, raw_u16

    H, D, BS, NB = 40, 128, 8, 1024
    g = gather_inputs(num_tokens=num_tokens, num_kv_heads=H, head_size=D, block_size=BS,
                      num_blocks=NB, dtype="f16", seed=29, device="cpu")
    kc, vc, slots = raw_u16(g.key_cache), raw_u16(g.value_cache), g.slot_mapping.numpy()
    rows_k, rows_v = oracle.gather_cached_kv(kc, vc, slots, BS)
    calls = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        if op == "gather":
            oracle.gather_cached_kv(kc, vc, slots, BS)
        else:
            oracle.kv_cache_write(kc, vc, rows_k, rows_v, slots, BS)
        calls += 1
    dt = (time.perf_counter() - t0) / calls
    moved = 2 * copy_bytes_once(num_tokens, H, D, 2) + 4 * num_tokens
    return {"value": round(moved / dt / 1e9, 3), "unit": "GB/s read+write", "cores": 1,
            "host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{calls} full calls at the same shapes ({dt * 1e3:.1f} ms each, numpy)"}


def bench_copy(op, steps, warmup, num_tokens, cpu_seconds=0.0, kv_layout="separate"):
    """Time gather_cached_kv or paged_kv_cache_write at the gather page's shapes."""
    import torch

    from decode_attention_paged_06_amd import gather_cached_kv, paged_kv_cache_write
    from workloads import gather_inputs

    H, D, BS, NB = 40, 128, 8, 1024
    dev = torch.device("cuda:0")
    sets = []
    # rotate pools so the ~2 GiB working set defeats the 256 MB last-level cache
    for i in range(max(1, -(-ROTATE_BYTES // (2 * NB * H * BS * D * 2)))):
        g = gather_inputs(num_tokens=num_tokens, num_kv_heads=H, head_size=D, block_size=BS,
                          num_blocks=NB, dtype="f16", seed=29 + i, device=dev, kv_layout=kv_layout)
        rows = (torch.empty((num_tokens, H, D), dtype=torch.float16, device=dev),
                torch.empty((num_tokens, H, D), dtype=torch.float16, device=dev))
        sets.append((g, rows))

    def step(i):
        g, (a, b) = sets[i % len(sets)]
        if op == "gather":
            gather_cached_kv(a, b, g.key_cache, g.value_cache, g.slot_mapping, BS)
        else:
            paged_kv_cache_write(g.key_cache, g.value_cache, a, b, g.slot_mapping, BS)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # replay from a HIP graph: small copies are otherwise bound by the host launch path
    ncap = max(20, len(sets))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(ncap):
            step(i)
    graph.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // ncap)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3 / (reps * ncap)
    once = copy_bytes_once(num_tokens, H, D, 2)
    moved = 2 * once + 4 * num_tokens  # read and write every row, plus the slots
    print(json.dumps({"op": op, "num_tokens": num_tokens, "num_kv_heads": H, "head_size": D,
                      "block_size": BS, "num_blocks": NB, "dtype": "f16", "kv_layout": kv_layout,
                      "us_per_call": round(sec * 1e6, 3),
                      "GB/s_read_plus_write": round(moved / sec / 1e9, 2),
                      "pct_of_hbm_peak": round(100 * moved / sec / 1e9 / HBM_PEAK_GBPS, 2),
                      "pages_convention_GiB/s": round(pages_gib_per_s(num_tokens, H, D, 2, sec), 2),
                      "input_sets_rotated": len(sets),
                      **({"cpu_baseline": cpu_baseline_copy(op, num_tokens, cpu_seconds)}
                         if cpu_seconds > 0 else {})}), flush=True)


MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16/fp16 matrix peak
PREFILL_SETTLE_S = 0.3           # minimum untimed warm-up of the prefill timing


def cpu_baseline_prefill(context, new_tokens, budget_s, kv_dtype=None):
    """The fp64 oracle on a sample of the prefill workload: one sequence's last new tokens."""
    import oracle
    from workloads import prefill_inputs, raw_bits, raw_u16

    threads = _blas_threads()
    flops, rows, t_total = 0, 0, 0.0
    n = 1
    while t_total < budget_s and n <= new_tokens:
        inp, q, qs, _ = prefill_inputs(new_tokens=[n], seed=77, device="cpu", num_seqs=1,
                                       num_heads=64, num_kv_heads=8, head_size=128, block_size=16,
                                       dtype="bf16", context_lens=context, kv_dtype=kv_dtype)
        t0 = time.perf_counter()
        oracle.paged_prefill(raw_u16(q), raw_bits(inp.key_cache), raw_bits(inp.value_cache),
                             inp.block_tables.numpy(), inp.context_lens.numpy(), qs.numpy(),
                             inp.scale, 16, dtype="bf16", k_scale=inp.k_scale, v_scale=inp.v_scale)
        t_total += time.perf_counter() - t0
        flops += 4 * 64 * 128 * sum(context - n + i + 1 for i in range(n))
        rows += n
        n *= 2
    return {"value": round(flops / t_total / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{rows} query tokens (chunks of 1, 2, 4, ... new tokens of one sequence of "
                      f"{context} context tokens, {t_total:.1f} s, fp64 numpy)"}


def measure_prefill(steps, warmup, batch, context, new_tokens, partition_size, cpu_seconds=0.0,
                    kv_dtype=None, kv_layout="separate"):
    """Time causal multi-query attention: `new_tokens` queries per sequence over a
    `context`-token paged cache (GQA 64/8, D 128, bf16, block 16; FP8 E4M3 cache
    with kv_dtype="fp8")."""
    import torch

    from decode_attention_paged_06_amd import paged_attention_prefill
    from workloads import prefill_inputs

    dev = torch.device("cuda:0")
    inp, q, qs, max_q = prefill_inputs(new_tokens=[new_tokens] * batch, seed=77, device=dev,
                                       num_seqs=batch, num_heads=64, num_kv_heads=8,
                                       head_size=128, block_size=16, dtype="bf16",
                                       context_lens=context, kv_dtype=kv_dtype,
                                       kv_layout=kv_layout)
    out = torch.empty_like(q)

    def step():
        paged_attention_prefill(out, q, inp.key_cache, inp.value_cache, inp.block_tables,
                                inp.context_lens, qs, max_q, inp.scale, 16,
                                partition_size=partition_size, k_scale=inp.k_scale,
                                v_scale=inp.v_scale)

    # Warm-up: W calls, then more until PREFILL_SETTLE_S seconds of calls have
    # run: the shader clock ramps up over the first ~0.1 s of sustained matrix
    # work, and a timed region that starts earlier measures the ramp.
    t0 = time.perf_counter()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < PREFILL_SETTLE_S:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3 / steps
    # q.K and P.V multiply-adds over the visible (causal) keys of every query
    keys = sum(context - new_tokens + i + 1 for i in range(new_tokens)) * batch
    flops = 4 * 64 * 128 * keys
    return {"op": "prefill", "batch": batch, "context": context,
            "new_tokens": new_tokens, "kv_cache": kv_dtype or "bf16", "kv_layout": kv_layout,
            "steps": steps, "us_per_call": round(sec * 1e6, 2),
            "TFLOP/s": round(flops / sec / 1e12, 2),
            "pct_of_mfma_peak": round(100 * flops / sec / 1e12 / MFMA_BF16_PEAK_TFLOPS, 2),
            **({"cpu_baseline": cpu_baseline_prefill(context, new_tokens, cpu_seconds, kv_dtype)}
               if cpu_seconds > 0 else {})}


def bench_prefill(*args, **kw):
    print(json.dumps(measure_prefill(*args, **kw)), flush=True)


def calibrate_copy(mib, steps):
    import torch

    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").random_(0, 255)
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read_per_copy": n,
                      "bytes_written_per_copy": n, "copies": steps}), flush=True)


def device_ceiling(gib: int = 4, reps: int = 10, run_bytes: int = 8192):
    """What plain device-wide reading reaches on this GPU, as context for the
    kernel's fraction of the vendor peak: the library's read probe over `gib`
    GiB (the decode kernels' 16-byte non-temporal loads, reads only) in
    contiguous slices and as `run_bytes` runs at scattered positions (the
    paged pattern: one run per cache tile), and a device-to-device copy of
    1 GiB (the runtime's copy kernel, read and written)."""
    import torch

    from decode_attention_paged_06_amd.ops import stream_read_probe

    n = gib << 30
    big = torch.empty(n, dtype=torch.uint8, device="cuda:0").random_(0, 255)
    sink = stream_read_probe(big)
    src, dst = big[: 1 << 30], torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
    e = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    for _ in range(2):
        stream_read_probe(big, sink)
        stream_read_probe(big, sink, run_bytes=run_bytes)
        dst.copy_(src)
    torch.cuda.synchronize()
    e[0].record()
    for _ in range(reps):
        stream_read_probe(big, sink)
    e[1].record()
    e[2].record()
    for _ in range(reps):
        stream_read_probe(big, sink, run_bytes=run_bytes)
    e[3].record()
    e[4].record()
    for _ in range(reps):
        dst.copy_(src)
    e[5].record()
    torch.cuda.synchronize()
    read_s = e[0].elapsed_time(e[1]) * 1e-3 / reps
    runs_s = e[2].elapsed_time(e[3]) * 1e-3 / reps
    copy_s = e[4].elapsed_time(e[5]) * 1e-3 / reps
    del big, sink, src, dst
    torch.cuda.empty_cache()
    read_gbps = n / read_s / 1e9
    runs_gbps = n / runs_s / 1e9
    copy_gbps = 2 * (1 << 30) / copy_s / 1e9
    return {"stream_read_GB/s": round(read_gbps, 1),
            "stream_read_pct_of_peak": round(100 * read_gbps / HBM_PEAK_GBPS, 1),
            f"scattered_{run_bytes // 1024}KiB_runs_read_GB/s": round(runs_gbps, 1),
            f"scattered_{run_bytes // 1024}KiB_runs_read_pct_of_peak": round(100 * runs_gbps / HBM_PEAK_GBPS, 1),
            "copy_GB/s_read_plus_write": round(copy_gbps, 1),
            "copy_pct_of_peak": round(100 * copy_gbps / HBM_PEAK_GBPS, 1),
            "note": f"read probe over {gib} GiB (contiguous slices; {run_bytes} B runs at scattered "
                    f"positions) and torch copy_ of 1 GiB, {reps} each, after the timed region"}


PROFILE_DIR = os.path.join(ROOT, "profiles")


def recorded_traffic(kernel: str, workload: str, batch: int, kv: str = "native",
                     block_size: int = 16, kv_layout: str = "separate"):
    """HBM bytes per launch from a committed rocprofv3 PMC summary, or None.

    A summary under profiles/ ends with a JSON record of the scaled
    FETCH_SIZE + WRITE_SIZE traffic and a SHA-256 of the kernel's sources at
    the time the counters were taken; the figure is used only for the same
    workload, batch, cache format, block size and cache layout (a record
    without the last three is of a 16-bit cache with 16-token blocks in two
    separate tensors), and only while the sources still hash the same.
    """
    import glob
    import hashlib

    for path in sorted(glob.glob(os.path.join(PROFILE_DIR, "*.md"))):
        text = open(path).read()
        for line in text.splitlines():
            if not line.startswith('{"kernel"'):
                continue
            rec = json.loads(line)
            if (kernel not in rec["kernel"] or rec["workload"] != workload
                    or rec["batch"] != batch or rec.get("kv", "native") != kv
                    or rec.get("block_size", 16) != block_size
                    or rec.get("kv_layout", "separate") != kv_layout):
                continue
            h = hashlib.sha256()
            try:
                for f in rec["sources"]:
                    h.update(open(os.path.join(ROOT, f), "rb").read())
            except OSError:
                return None
            if h.hexdigest() == rec["sources_sha256"]:
                return rec["traffic_bytes_per_launch"]
    return None


def workload_label(name, args):
    return (f"{name}: {args['num_heads']}q/{args['num_kv_heads']}kv heads, D={args['head_size']}, "
            f"{args['dtype']}, block {args['block_size']}, batch {args['num_seqs']}, "
            f"context {args['context_lens']}" + (", ALiBi" if args.get("alibi") else "")
            + (f", {args['kv_dtype']} KV cache" if args.get("kv_dtype") else ""))


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl missing
        return 1


def cpu_baseline(args, budget_s):
    """The fp64 oracle on a bounded sample of the same workload, on the host cores."""
    import numpy as np

    import oracle
    from workloads import algorithmic_bytes, decode_inputs, raw_u16

    threads = _blas_threads()
    sample_args = dict(args)
    n = min(args["num_seqs"], 64)
    sample_args["num_seqs"] = n
    sample_args.pop("kv_layout", None)   # the oracle reads plain [NB, Hkv, BS, D] arrays
    inp = decode_inputs(device="cpu", **sample_args)
    q, kc, vc = raw_u16(inp.query), raw_u16(inp.key_cache), raw_u16(inp.value_cache)
    tables, lens = inp.block_tables.numpy(), inp.context_lens.numpy()
    slopes = None if inp.alibi_slopes is None else inp.alibi_slopes.numpy()
    # cycle over the sampled sequences until the time budget is spent
    done = []
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        for s in range(n):
            oracle.paged_decode(q, kc, vc, tables, lens, inp.scale, inp.block_size, slopes,
                                dtype=inp.dtype, seqs=[s])
            done.append(s)
            if time.perf_counter() - t0 > budget_s:
                break
    dt = time.perf_counter() - t0
    nbytes = algorithmic_bytes(context_lens=lens[done].tolist(), num_heads=args["num_heads"],
                               num_kv_heads=args["num_kv_heads"], head_size=args["head_size"],
                               block_size=args["block_size"], alibi=bool(args.get("alibi")))
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{len(done)} sequence decodes cycling over {n} of the {args['num_seqs']} "
                      f"sequences of the same workload ({dt:.1f} s wall, fp64 numpy)",
            "seconds_per_sequence": round(dt / len(done), 4)}


MAX_SETS = 1024   # cap on rotated input sets (tiny workloads: >= 1 GiB, 4x the last-level cache)
# The pages' A100 kernel-latency tables (bf16, 64q/8kv): paged V1, paged V2, FlashAttention, in us.
PAGES_TABLES_US = {
    ("gqa_ctx1024", 1): (37.541, 29.602, 27.675), ("gqa_ctx1024", 4): (68.585, 71.447, 27.433),
    ("gqa_ctx1024", 16): (162.237, 168.997, 67.681), ("gqa_ctx1024", 64): (687.938, 733.687, 214.041),
    ("gqa_ctx1024", 256): (2215.532, 2378.606, 680.123),
    ("gqa_ctx4096", 1): (137.858, 70.783, 28.557), ("gqa_ctx4096", 4): (223.438, 164.293, 62.104),
    ("gqa_ctx4096", 16): (716.780, 724.601, 238.730), ("gqa_ctx4096", 64): (2324.863, 2792.657, 772.266),
    ("gqa_ctx4096", 256): (8771.168, 9723.521, 2583.970),
}


def measure_decode(args, *, steps, warmup, engine="auto", partition_size=0, schedule="auto",
                   hot=False, graph=False, per_call=True):
    """Time paged_attention_decode on one synthetic workload (inputs resident in HBM).

    Input sets with the same lengths and shapes are rotated so their combined
    footprint is at least ROTATE_BYTES (at most MAX_SETS sets; one with
    hot=True).  Eager time: HIP events around `steps` back-to-back calls (and
    around each call when per_call).  graph=True also replays the calls from a
    HIP graph: device time without the host launch path.
    """
    import torch

    from decode_attention_paged_06_amd import (kv_layout_of, make_dims, make_opts,
                                               paged_attention_decode, paged_attention_plan)
    from workloads import algorithmic_bytes, algorithmic_flops, decode_inputs

    dev = torch.device("cuda:0")
    first = decode_inputs(device=dev, **args)
    lens = first.context_lens.cpu().tolist()
    nbytes = algorithmic_bytes(context_lens=lens, num_heads=args["num_heads"],
                               num_kv_heads=args["num_kv_heads"], head_size=args["head_size"],
                               block_size=args["block_size"], alibi=bool(args.get("alibi")),
                               kv_elem_bytes=first.key_cache.element_size())
    flops = algorithmic_flops(context_lens=lens, num_heads=args["num_heads"],
                              head_size=args["head_size"])
    footprint = sum(t.numel() * t.element_size() for t in
                    (first.query, first.key_cache, first.value_cache, first.block_tables))
    nsets = 1 if hot else min(MAX_SETS, max(1, -(-ROTATE_BYTES // footprint)))
    sets = [first]
    for i in range(1, nsets):
        # same lengths and shapes, fresh values and block assignment
        sets.append(decode_inputs(device=dev, **dict(args, seed=args["seed"] + 100000 * i,
                                                      context_lens=lens)))
    outs = [torch.empty_like(x.query) for x in sets]

    dims = make_dims(first.query, first.key_cache, first.block_tables, first.k_scale,
                     first.v_scale, kv_layout_of(first.key_cache, first.value_cache))
    opts = make_opts(partition_size, engine, schedule=schedule)
    plan = paged_attention_plan(dims, 1 << 40, opts)
    workspace = (torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)
                 if plan.workspace_bytes else None)

    def step(i):
        x = sets[i % nsets]
        paged_attention_decode(outs[i % nsets], x.query, x.key_cache, x.value_cache,
                               x.block_tables, x.context_lens, x.scale, x.block_size,
                               x.alibi_slopes, workspace=workspace,
                               partition_size=partition_size, engine=engine,
                               k_scale=x.k_scale, v_scale=x.v_scale, schedule=schedule)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps if per_call else 0)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(steps):
        if per_call:
            ev[i][0].record()
        step(i)
        if per_call:
            ev[i][1].record()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    res = {"nbytes": nbytes, "flops": flops, "plan": plan, "nsets": nsets, "wall": wall,
           "ms_per_step": t_start.elapsed_time(t_end) / steps,
           "per_call_ms": [x.elapsed_time(y) for x, y in ev]}

    if graph:
        # Capture one rotation of calls (at least 20) into a graph and replay it:
        # the GPU then runs the kernels back to back, so the time is the
        # device time of the calls without the host launch path.
        ncap = max(20, nsets)
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(ncap):
                step(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(ncap):
                step(i)
        g.replay()
        torch.cuda.synchronize()
        reps = max(1, steps // ncap)
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(reps):
            g.replay()
        g1.record()
        torch.cuda.synchronize()
        res["graph_us"] = g0.elapsed_time(g1) * 1e3 / (reps * ncap)
        del g
    del sets, outs, workspace, first
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def plan_fields(plan, engine="auto"):
    return {"engine": {0: "auto", 1: "valu", 2: "mfma"}[plan.engine] if engine == "auto" else engine,
            "num_partitions": plan.num_partitions, "partition_size": plan.partition_size,
            "schedule": {2: "longest_first", 3: "equal_shares"}.get(plan.schedule, "grid")}


def grid_rows(steps, warmup, kv_layout, headline=None):
    """Every named workload at every batch the pages' tables (and the MQA and
    MHA configurations) use: eager and graph-replay time per call, achieved
    GB/s and the fraction of the 8 TB/s peak, and the plan.  `headline`
    (workload, batch, measurement) is reused instead of measured again."""
    from workloads import WORKLOADS, workload_args

    rows = []
    for name, w in WORKLOADS.items():
        for batch in w["batches"]:
            args = dict(workload_args(name, batch), kv_layout=kv_layout)
            if headline is not None and (name, batch) == headline[:2]:
                r = headline[2]
            else:
                r = measure_decode(args, steps=steps, warmup=warmup, graph=True, per_call=False)
            us = r["ms_per_step"] * 1e3
            row = {"workload": name, "batch": batch, "kv_cache": args["dtype"],
                   "us_eager": round(us, 2),
                   "GB/s_eager": round(r["nbytes"] / (us * 1e-6) / 1e9, 1),
                   "frac_eager": round(r["nbytes"] / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
            if "graph_us" in r:
                g = r["graph_us"]
                row.update({"us_graph": round(g, 2),
                            "GB/s_graph": round(r["nbytes"] / (g * 1e-6) / 1e9, 1),
                            "frac_graph": round(r["nbytes"] / (g * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)})
            row.update({"bytes": r["nbytes"], "input_sets": r["nsets"], **plan_fields(r["plan"])})
            if (name, batch) in PAGES_TABLES_US:
                v1, v2, fa = PAGES_TABLES_US[(name, batch)]
                row["pages_a100_us"] = {"paged_v1": v1, "paged_v2": v2, "flash_attention": fa}
            rows.append(row)
            print(f"bench grid: {name} b={batch} eager {row['us_eager']} us, graph "
                  f"{row.get('us_graph')} us", file=sys.stderr, flush=True)
    return rows


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only (asked for --gpus {a.gpus}); the decode "
              "kernel has no cross-GPU path to measure", file=sys.stderr)
        sys.exit(2)
    if a.calibrate_copy:
        calibrate_copy(a.calibrate_copy, a.steps)
        return
    if a.op == "prefill":
        bench_prefill(a.steps, a.warmup, a.batch or 4, a.context, a.new_tokens, a.partition_size,
                      0.0 if a.no_cpu_baseline else min(a.cpu_seconds, 5.0), a.kv_dtype,
                      a.kv_layout)
        return
    if a.op != "decode":
        bench_copy(a.op, a.steps, a.warmup, a.tokens, 0.0 if a.no_cpu_baseline else min(a.cpu_seconds, 3.0),
                   a.kv_layout)
        return

    import torch

    from workloads import HEADLINE, workload_args

    name = a.workload or HEADLINE[0]
    batch = a.batch or HEADLINE[1]
    args = workload_args(name, batch)
    if a.kv_dtype:
        args["kv_dtype"] = a.kv_dtype
    args["kv_layout"] = a.kv_layout
    if a.block_size:
        args["block_size"] = a.block_size
        args.pop("pool_blocks", None)  # pool sized to fit the new block size
        args.pop("max_blocks_per_seq", None)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    # the grid runs with the default headline invocation (and on request)
    is_default = (a.workload is None and a.batch is None and not a.kv_dtype and not a.block_size
                  and a.engine == "auto" and a.partition_size == 0 and a.schedule == "auto"
                  and not a.hot)
    want_grid = (is_default and not a.no_grid) or a.grid

    m = measure_decode(args, steps=a.steps, warmup=a.warmup, engine=a.engine,
                       partition_size=a.partition_size, schedule=a.schedule, hot=a.hot,
                       graph=a.graph or want_grid)
    nbytes, flops, plan, nsets, wall = m["nbytes"], m["flops"], m["plan"], m["nsets"], m["wall"]
    per_call_ms = m["per_call_ms"]
    avg_ms = sum(per_call_ms) / len(per_call_ms)
    srt = sorted(per_call_ms)
    per_call_us = {"median": round(srt[len(srt) // 2] * 1e3, 2), "min": round(srt[0] * 1e3, 2),
                   "max": round(srt[-1] * 1e3, 2)}
    ms_per_step = m["ms_per_step"]
    gbps = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (avg_ms * 1e-3) / 1e9
    graph_us = m.get("graph_us")

    grid = None
    if want_grid:
        grid = grid_rows(max(20, min(a.steps, 100)), min(a.warmup, 10), a.kv_layout,
                         headline=(name, batch, m) if is_default else None)

    # the multi-query (prefill) shape: 4 sequences x 512 new tokens on 4096-token
    # contexts, GQA 64/8 bf16, with the default run's grid
    prefill = None
    if want_grid:
        prefill = measure_prefill(100, 10, 4, 4096, 512, 0, kv_layout=a.kv_layout)

    ceiling = None
    if not a.no_ceiling:
        try:
            # scattered runs the size of the workload's contiguous cache run: one
            # (block, kv head) tile of K and V in the joint layout, of K or V alone
            # in separate tensors (1 byte per element for an FP8 cache)
            elem = 1 if args.get("kv_dtype") == "fp8" else 2
            run = args["block_size"] * args["head_size"] * elem * (2 if a.kv_layout == "joint" else 1)
            ceiling = device_ceiling(run_bytes=max(1024, 1 << (run.bit_length() - 1)))
        except torch.cuda.OutOfMemoryError as e:  # context only: never fail the bench for it
            ceiling = {"error": f"not measured: {e.__class__.__name__}"}
            torch.cuda.empty_cache()

    kernel_name = "decode_mfma_kernel" if plan.engine == 2 else "decode_valu_kernel"
    context = PAGES_US.get((name, batch))

    result = {
        "metric": METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,   # value / cpu_baseline.value, filled in below
        "dtype": args["dtype"],
        "data": "synthetic",
        "config": {
            "workload": workload_label(name, args),
            "num_seqs": batch, "num_heads": args["num_heads"], "num_kv_heads": args["num_kv_heads"],
            "head_size": args["head_size"], "block_size": args["block_size"],
            "kv_cache": args.get("kv_dtype") or args["dtype"], "kv_layout": a.kv_layout,
            "context_lens": str(args["context_lens"]), "seed": args["seed"],
            **plan_fields(plan, a.engine),
            "input_sets_rotated": nsets,
            **({"hot_cache": True} if a.hot else {}),
        },
        "per_call_us": per_call_us,
        "us_per_call": round(ms_per_step * 1e3, 2),
        "pct_of_hbm_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 2),
        "algorithmic_bytes_per_call": nbytes,
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": recorded_traffic(kernel_name, name, batch, a.kv_dtype or "native",
                                        args["block_size"], a.kv_layout),
            "kernel": kernel_name,
            "kernel_avg_us": round(avg_ms * 1e3, 2),
            "flops_per_call": flops,
            "note": ("per-call HIP events on the launch stream; one decode kernel per call"
                     if plan.num_partitions == 1 else
                     "per-call HIP events include the partition-reduce kernel"),
        },
        "wall_s_timed_region": round(wall, 3),
    }
    if graph_us is not None:
        result["graph_replay"] = {"us_per_call": round(graph_us, 3),
                                  "GB/s": round(nbytes / (graph_us * 1e-6) / 1e9, 2),
                                  "pct_of_hbm_peak": round(100 * nbytes / (graph_us * 1e-6) / 1e9
                                                           / HBM_PEAK_GBPS, 2)}
    if grid is not None:
        result["grid"] = {"note": "every workload and batch of the configuration list, "
                                  f"{a.kv_layout} caches, auto plan; eager = HIP events around "
                                  "back-to-back calls, graph = replay of captured calls (device "
                                  "time without the host launch path); fractions of 8 TB/s; "
                                  "pages_a100_us: the pages' A100 table entries (context)",
                          "rows": grid}
    if prefill is not None:
        result["prefill"] = dict(prefill, note="causal multi-query call, GQA 64/8 bf16, "
                                 "TFLOP/s of the q.K and P.V products over the keys each query "
                                 "sees; peak = 2.5 PFLOP/s dense bf16")
    if ceiling is not None:
        result["device_ceiling"] = ceiling
    if context:
        result["pages_context"] = dict(context, note="A100 numbers from the reference pages "
                                       "(other hardware): context, not the baseline")
    if not a.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, a.cpu_seconds)
        # the stated baseline: the fp64 oracle on the host cores, same metric and unit
        result["vs_baseline"] = round(result["value"] / result["cpu_baseline"]["value"], 1)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
