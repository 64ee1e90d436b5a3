"""GPU parity: the HIP decode path against the fp64 oracle.

The gate (tests/parity_gate.py): max abs per element 2e-3 for fp16, 1e-2 for
bf16, plus relative L2 bounds over the whole output (2 u) and per output row
(4 u), u the output format's unit roundoff.  Integer facts (context length 1
returns V, relabelled blocks, determinism) are checked bit for bit.
"""
import numpy as np
import pytest
import torch

from gpu_util import TOL, compare, device, make, oracle_ref, run, sample_seqs, to_device
from workloads import WORKLOADS, raw_u16, workload_args

pytestmark = pytest.mark.gpu

ENGINES = ["valu", "mfma"]


# ---------------------------------------------------------------------------
# The named workloads at their full sizes, in the auto launch configuration
# (the one the bench times) and with each engine forced.  Sequences beyond 16
# are checked on a seeded sample, always including the first and the last.
# ---------------------------------------------------------------------------

WORKLOAD_CASES = [(name, b) for name, w in WORKLOADS.items() for b in w["batches"]]


@pytest.mark.parametrize("name,batch", WORKLOAD_CASES, ids=[f"{n}-b{b}" for n, b in WORKLOAD_CASES])
def test_workload_parity(name, batch):
    dev = device()
    args = workload_args(name, batch)
    inp = make(device_=dev, poison=True, **args)
    seqs = sample_seqs(batch, 16, seed=batch)
    ref = oracle_ref(inp, seqs)
    for engine in ["auto"] + ENGINES:
        out = run(inp, engine=engine)
        compare(out, ref, inp.dtype, seqs, what=f"{name} b={batch} engine={engine}")


# ---------------------------------------------------------------------------
# Split-context partitions: boundaries, ragged tails, every engine and dtype
# ---------------------------------------------------------------------------

BOUNDARY_LENS = [1, 15, 16, 17, 47, 48, 63, 64, 65, 127, 128, 129, 200, 511, 513, 1000]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("alibi", [False, True])
def test_partitions(dtype, engine, alibi):
    dev = device()
    inp = to_device(make(num_seqs=len(BOUNDARY_LENS), num_heads=16, num_kv_heads=2, head_size=128,
                         block_size=16, dtype=dtype, seed=77, context_lens=BOUNDARY_LENS,
                         alibi=alibi, poison=True), dev)
    ref = oracle_ref(inp)
    for ps in (-1, 0, 16, 32, 48, 64, 256):
        out = run(inp, engine=engine, partition_size=ps)
        compare(out, ref, dtype, what=f"{dtype} {engine} alibi={alibi} partition={ps}")


@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("group", [1, 2, 3, 8, 16, 20, 48, 64])
def test_group_sizes(engine, group):
    dev = device()
    Hkv = 2 if group <= 16 else 1
    inp = to_device(make(num_seqs=3, num_heads=group * Hkv, num_kv_heads=Hkv, head_size=128,
                         block_size=16, dtype="bf16", seed=100 + group, context_lens=[5, 130, 77],
                         alibi=True, poison=True), dev)
    ref = oracle_ref(inp)
    for ps in (-1, 64):
        compare(run(inp, engine=engine, partition_size=ps), ref, "bf16",
                what=f"G={group} {engine} partition={ps}")


@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("block_size", [8, 16, 32, 64, 256])
def test_block_sizes(engine, block_size):
    dev = device()
    lens = [1, 7, 8, 9, 31, 33, 255, 257, 600]
    for dtype, D in (("bf16", 128), ("f16", 64)):
        inp = to_device(make(num_seqs=len(lens), num_heads=16, num_kv_heads=2, head_size=D,
                             block_size=block_size, dtype=dtype, seed=block_size + D,
                             context_lens=lens, alibi=True, poison=True), dev)
        ref = oracle_ref(inp)
        for ps in (-1, 0, max(block_size, 128)):
            compare(run(inp, engine=engine, partition_size=ps), ref, dtype,
                    what=f"BS={block_size} D={D} {engine} partition={ps}")


@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("head_size", [64, 128])
def test_head_sizes_fp16(engine, head_size):
    dev = device()
    inp = to_device(make(num_seqs=5, num_heads=8, num_kv_heads=4, head_size=head_size,
                         block_size=16, dtype="f16", seed=9, context_lens=[1, 2, 33, 64, 250],
                         poison=True), dev)
    ref = oracle_ref(inp)
    for ps in (-1, 32):
        compare(run(inp, engine=engine, partition_size=ps), ref, "f16",
                what=f"D={head_size} {engine} partition={ps}")


# ---------------------------------------------------------------------------
# Closed forms, invariants and edge cases
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_context_one_returns_v_exactly(engine, dtype):
    dev = device()
    inp = to_device(make(num_seqs=6, num_heads=16, num_kv_heads=4, head_size=128, block_size=16,
                         dtype=dtype, seed=3, context_lens=1, alibi=True, poison=True,
                         max_blocks_per_seq=8), dev)
    vc = raw_u16(inp.value_cache)
    tables = inp.block_tables.cpu().numpy()
    for ps in (-1, 16):
        got = raw_u16(run(inp, engine=engine, partition_size=ps))
        for s in range(6):
            for h in range(16):
                assert np.array_equal(got[s, h], vc[tables[s, 0], h // 4, 0]), (s, h, ps)


@pytest.mark.parametrize("engine", ENGINES)
def test_empty_context_gives_zeros(engine):
    dev = device()
    inp = to_device(make(num_seqs=4, num_heads=8, num_kv_heads=1, head_size=128, block_size=16,
                         dtype="bf16", seed=4, context_lens=[0, 20, 0, 3], poison=True,
                         max_blocks_per_seq=4), dev)
    ref = oracle_ref(inp)
    for ps in (-1, 16):
        out = run(inp, engine=engine, partition_size=ps)
        assert not out[0].float().abs().sum().item() and not out[2].float().abs().sum().item()
        compare(out, ref, "bf16", what=f"empty {engine} partition={ps}")


@pytest.mark.parametrize("engine", ENGINES)
def test_deterministic_and_block_relabelling(engine):
    dev = device()
    inp = to_device(make(num_seqs=5, num_heads=32, num_kv_heads=4, head_size=128, block_size=16,
                         dtype="bf16", seed=12, context_lens=[300, 17, 1024, 64, 555],
                         alibi=True), dev)
    for ps in (-1, 128):
        a = raw_u16(run(inp, engine=engine, partition_size=ps))
        b = raw_u16(run(inp, engine=engine, partition_size=ps))
        assert np.array_equal(a, b), "two identical calls differ"
        # move every physical block to a new id: same bytes, same order of work
        NB = inp.key_cache.shape[0]
        pi = torch.randperm(NB, generator=torch.Generator().manual_seed(1)).to(dev)
        kc = torch.empty_like(inp.key_cache)
        vc = torch.empty_like(inp.value_cache)
        kc[pi] = inp.key_cache
        vc[pi] = inp.value_cache
        moved = make(num_seqs=1, num_heads=1, num_kv_heads=1, head_size=128, block_size=16,
                     dtype="bf16", seed=0, context_lens=1)
        moved.query, moved.key_cache, moved.value_cache = inp.query, kc, vc
        moved.block_tables = pi[inp.block_tables.long()].to(torch.int32).contiguous()
        moved.context_lens, moved.alibi_slopes, moved.scale = inp.context_lens, inp.alibi_slopes, inp.scale
        c = raw_u16(run(moved, engine=engine, partition_size=ps))
        assert np.array_equal(a, c), "relabelled blocks changed the result"


@pytest.mark.parametrize("engine", ENGINES)
def test_needle(engine):
    """q = c K[t*] puts all softmax weight on t*: out = V[t*] up to rounding."""
    dev = device()
    lens = [40, 300]
    inp = make(num_seqs=2, num_heads=8, num_kv_heads=1, head_size=128, block_size=16,
               dtype="f16", seed=21, context_lens=lens, poison=True)
    kc = inp.key_cache.float()
    tables = inp.block_tables
    for tstar in (0, 15, 16, 17, 39):
        for s in range(2):
            t = tstar if s == 0 else 255 - tstar
            k = kc[tables[s, t // 16], 0, t % 16]
            # 8 heads: 8 different needle strengths, all large
            for h in range(8):
                inp.query[s, h] = (k * (0.5 + 0.1 * h)).to(torch.float16)
        g = to_device(make(num_seqs=2, num_heads=8, num_kv_heads=1, head_size=128, block_size=16,
                           dtype="f16", seed=21, context_lens=lens, poison=True), dev)
        g.query = inp.query.to(dev)
        ref = oracle_ref(g)
        for ps in (-1, 32):
            compare(run(g, engine=engine, partition_size=ps), ref, "f16",
                    what=f"needle t*={tstar} {engine} partition={ps}")


def test_gqa_equals_repeated_mha():
    dev = device()
    G = 8
    gqa = to_device(make(num_seqs=3, num_heads=16, num_kv_heads=2, head_size=128, block_size=16,
                         dtype="bf16", seed=31, context_lens=[100, 7, 400], alibi=True), dev)
    mha = to_device(make(num_seqs=3, num_heads=16, num_kv_heads=2, head_size=128, block_size=16,
                         dtype="bf16", seed=31, context_lens=[100, 7, 400], alibi=True), dev)
    mha.key_cache = gqa.key_cache.repeat_interleave(G, dim=1).contiguous()
    mha.value_cache = gqa.value_cache.repeat_interleave(G, dim=1).contiguous()
    ref = oracle_ref(gqa)
    for engine in ENGINES:
        a = run(gqa, engine=engine)
        b = run(mha, engine=engine)
        compare(a, ref, "bf16", what=f"gqa {engine}")
        compare(b, ref, "bf16", what=f"repeated mha {engine}")
        assert float((a.float() - b.float()).abs().max()) <= TOL["bf16"]


def test_stream_argument_is_used():
    dev = device()
    inp = to_device(make(num_seqs=2, num_heads=8, num_kv_heads=2, head_size=128, block_size=16,
                         dtype="bf16", seed=41, context_lens=[500, 900]), dev)
    ref = oracle_ref(inp)
    s = torch.cuda.Stream()
    out = torch.empty_like(inp.query)
    from decode_attention_paged_06_amd import paged_attention_decode
    with torch.cuda.stream(s):
        paged_attention_decode(out, inp.query, inp.key_cache, inp.value_cache, inp.block_tables,
                               inp.context_lens, inp.scale, 16, None, stream=s, partition_size=64)
    s.synchronize()
    compare(out, ref, "bf16", what="side stream")


def test_side_stream_without_context_manager_owns_its_workspace():
    """stream=s while torch's current stream is another one, workspace=None:
    the binding's temporary workspace is recorded on s, so the allocator does
    not hand it to work on the current stream while the kernels on s run."""
    dev = device()
    inp = to_device(make(num_seqs=2, num_heads=64, num_kv_heads=8, head_size=128, block_size=16,
                         dtype="bf16", seed=42, context_lens=[4000, 3000]), dev)
    ref = oracle_ref(inp)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    from decode_attention_paged_06_amd import paged_attention_decode
    outs = []
    for _ in range(8):
        out = torch.empty_like(inp.query)
        paged_attention_decode(out, inp.query, inp.key_cache, inp.value_cache, inp.block_tables,
                               inp.context_lens, inp.scale, 16, None, stream=s, partition_size=128)
        # work on the current stream that would reuse a freed block at once
        junk = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
        junk.fill_(0xFF)
        outs.append(out)
    s.synchronize()
    for k, out in enumerate(outs):
        compare(out, ref, "bf16", what=f"side stream call {k}, binding-allocated workspace")


def test_concurrent_streams():
    """Calls in flight on two streams at once, each with its own workspace (a
    split GQA call and a longest-first MQA call), give what each gives alone."""
    dev = device()
    a = to_device(make(num_seqs=3, num_heads=64, num_kv_heads=8, head_size=128, block_size=16,
                       dtype="bf16", seed=43, context_lens=[2500, 40, 4000]), dev)
    b = to_device(make(num_seqs=24, num_heads=48, num_kv_heads=1, head_size=128, block_size=16,
                       dtype="f16", seed=44, context_lens=(64, 3000), alibi=True), dev)
    want = [run(a), run(b)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    ws = [torch.empty(32 << 20, dtype=torch.uint8, device=dev) for _ in range(2)]
    outs = [torch.full_like(x.query, float("nan")) for x in (a, b)]
    from decode_attention_paged_06_amd import paged_attention_decode
    for _ in range(10):
        for k, inp in enumerate((a, b)):
            with torch.cuda.stream(streams[k]):
                paged_attention_decode(outs[k], inp.query, inp.key_cache, inp.value_cache,
                                       inp.block_tables, inp.context_lens, inp.scale, 16,
                                       inp.alibi_slopes, stream=streams[k], workspace=ws[k])
    torch.cuda.synchronize()
    for k in range(2):
        assert torch.equal(outs[k], want[k]), f"stream {k} differs from its call alone"


# ---------------------------------------------------------------------------
# FP8 E4M3 caches (one scale per cache tensor)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("dtype,head_size", [("bf16", 128), ("f16", 128), ("f16", 64)])
def test_fp8_cache(engine, dtype, head_size):
    dev = device()
    lens = [1, 5, 16, 17, 100, 257, 700]
    for G, alibi in ((8, False), (1, True), (48, True)):
        Hkv = 2 if G < 48 else 1
        inp = to_device(make(num_seqs=len(lens), num_heads=G * Hkv, num_kv_heads=Hkv,
                             head_size=head_size, block_size=16, dtype=dtype, seed=G + head_size,
                             context_lens=lens, alibi=alibi, poison=True, kv_dtype="fp8",
                             kv_scale=0.0625), dev)
        ref = oracle_ref(inp)
        for ps in (-1, 0, 64):
            compare(run(inp, engine=engine, partition_size=ps), ref, dtype,
                    what=f"fp8 G={G} D={head_size} {dtype} {engine} partition={ps}")


@pytest.mark.parametrize("engine", ENGINES)
def test_fp8_context_one_is_exact(engine):
    """L = 1: out = decoded V * v_scale, exactly representable in bf16."""
    dev = device()
    inp = to_device(make(num_seqs=4, num_heads=8, num_kv_heads=2, head_size=128, block_size=16,
                         dtype="bf16", seed=8, context_lens=1, poison=True, kv_dtype="fp8",
                         kv_scale=0.125, max_blocks_per_seq=2), dev)
    got = run(inp, engine=engine, partition_size=-1).float().cpu().numpy()
    v = inp.value_cache.float().cpu().numpy() * 0.125
    tables = inp.block_tables.cpu().numpy()
    for s in range(4):
        for h in range(8):
            assert np.array_equal(got[s, h], v[tables[s, 0], h // 4, 0]), (s, h)


def test_fp8_workload_full_size():
    """The GQA ctx-4096 batch-64 workload with an fp8 cache, sampled against the oracle."""
    dev = device()
    args = workload_args("gqa_ctx4096", 64)
    inp = make(device_=dev, poison=True, kv_dtype="fp8", **args)
    seqs = sample_seqs(64, 12, seed=3)
    ref = oracle_ref(inp, seqs)
    for engine in ("auto", "valu"):
        compare(run(inp, engine=engine), ref, "bf16", seqs, what=f"fp8 gqa4096 b64 {engine}")


def test_fp8_mqa_workload_full_size():
    """The MQA 48/1 ragged ALiBi batch-256 workload with an fp8 cache (the staged
    path on tile pairs, split, longest first), sampled against the oracle."""
    dev = device()
    args = workload_args("mqa_ragged_alibi", 256)
    inp = make(device_=dev, poison=True, kv_dtype="fp8", **args)
    seqs = sample_seqs(256, 12, seed=4)
    ref = oracle_ref(inp, seqs)
    for schedule in ("auto", "grid"):
        compare(run(inp, schedule=schedule), ref, args["dtype"], seqs,
                what=f"fp8 mqa ragged b256 {schedule}")


# ---------------------------------------------------------------------------
# Groups of more than 16 heads: the head-tile waves of a token group share
# each K/V tile through an LDS ring and read tile source offsets from an LDS
# window (512 tiles of 16 tokens, 8 for 8-token blocks), refilled as the walk
# moves on.  Long contexts cross that window (4096 tokens at block size 8,
# 8192 otherwise; at block size 64 a window entry is a quarter block).
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("group", [20, 48, 64])
@pytest.mark.parametrize("kv", ["native", "fp8"])
@pytest.mark.parametrize("head_size", [64, 128])
def test_shared_tile_groups(group, kv, head_size):
    dev = device()
    dtype = "bf16" if head_size == 128 else "f16"
    for block_size, lens in ((8, [1, 9, 300, 4500]), (16, [17, 1000, 8300]), (64, [63, 65, 2000, 8500])):
        inp = to_device(make(num_seqs=len(lens), num_heads=group, num_kv_heads=1,
                             head_size=head_size, block_size=block_size, dtype=dtype,
                             seed=group + head_size + block_size, context_lens=lens, alibi=True,
                             poison=True, kv_dtype="fp8" if kv == "fp8" else None,
                             kv_scale=0.0625), dev)
        ref = oracle_ref(inp)
        for ps in (-1, 0, max(block_size, 128)):
            compare(run(inp, engine="mfma", partition_size=ps), ref, dtype,
                    what=f"G={group} {kv} D={head_size} BS={block_size} partition={ps}")


# ---------------------------------------------------------------------------
# Longest-first schedule of split units: only the order in which workgroups
# start changes, so the results are bit-identical to the grid order.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("group,Hkv", [(48, 1), (8, 2)])
def test_longest_first_schedule(group, Hkv):
    dev = device()
    inp = to_device(make(num_seqs=40, num_heads=group * Hkv, num_kv_heads=Hkv, head_size=128,
                         block_size=16, dtype="f16", seed=4040 + group, context_lens=(1, 3000),
                         alibi=True, poison=True), dev)
    seqs = sample_seqs(40, 12, seed=group)
    ref = oracle_ref(inp, seqs)
    for ps in (0, 128, 512):
        grid = run(inp, engine="mfma", partition_size=ps, schedule="grid")
        lpt = run(inp, engine="mfma", partition_size=ps, schedule="longest_first")
        assert torch.equal(grid, lpt), f"G={group} partition={ps}: schedules differ"
        compare(lpt, ref, "f16", seqs, what=f"longest-first G={group} partition={ps}")


# ---------------------------------------------------------------------------
# The reduce at every partition count it handles differently: batches of 4,
# 8, 16 and 32 partial-output loads, and more than 64 partitions (the (m, l)
# pairs then take several passes of one partition per lane).
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("engine", ENGINES)
def test_reduce_partition_counts(engine):
    dev = device()
    lens = [1, 40, 100, 130, 250, 520, 1100, 2200]
    inp = to_device(make(num_seqs=len(lens), num_heads=16, num_kv_heads=2, head_size=128,
                         block_size=16, dtype="bf16", seed=64, context_lens=lens, alibi=True,
                         poison=True), dev)
    ref = oracle_ref(inp)
    for ps in (16, 32, 64, 128, 256, 1024):  # up to 138 partitions of the longest sequence
        compare(run(inp, engine=engine, partition_size=ps), ref, "bf16",
                what=f"{engine} partition={ps}")


# ---------------------------------------------------------------------------
# Maximum sizes: the largest batch the ABI takes (65535 sequences, the grid's
# y limit; split and longest-first grids of ~200k units) and a 65536-token
# context (hundreds of partitions into one reduce).
# ---------------------------------------------------------------------------

def test_maximum_batch():
    dev = device()
    S = 65535
    inp = to_device(make(num_seqs=S, num_heads=16, num_kv_heads=2, head_size=64, block_size=16,
                         dtype="bf16", seed=51, context_lens=(1, 40)), dev)
    seqs = sample_seqs(S, 12, seed=5)
    ref = oracle_ref(inp, seqs)
    compare(run(inp), ref, "bf16", seqs, what="65535 sequences, one pass")
    compare(run(inp, partition_size=16), ref, "bf16", seqs, what="65535 sequences, split")
    compare(run(inp, partition_size=16, schedule="longest_first"), ref, "bf16", seqs,
            what="65535 sequences, split, longest first")


@pytest.mark.parametrize("block_size", [16, 256])
def test_maximum_context(block_size):
    dev = device()
    inp = to_device(make(num_seqs=1, num_heads=64, num_kv_heads=1, head_size=128,
                         block_size=block_size, dtype="bf16", seed=52, context_lens=65536,
                         alibi=True, poison=True), dev)
    ref = oracle_ref(inp)
    compare(run(inp), ref, "bf16", what=f"65536-token context, block {block_size}, auto plan")


@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_large_logits(engine, dtype):
    """q and K scaled by 16: logits in the thousands, a nearly one-hot softmax;
    the running max and rescale keep every weight finite, split or not."""
    dev = device()
    inp = to_device(make(num_seqs=4, num_heads=16, num_kv_heads=2, head_size=128, block_size=16,
                         dtype=dtype, seed=53, context_lens=[1, 300, 1000, 2500], alibi=True,
                         poison=True), dev)
    inp.query.mul_(16)
    inp.key_cache.mul_(16)
    ref = oracle_ref(inp)
    for ps in (-1, 128):
        compare(run(inp, engine=engine, partition_size=ps), ref, dtype,
                what=f"large logits {dtype} {engine} partition={ps}")
