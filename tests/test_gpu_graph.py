"""Decode and multi-query calls captured into a HIP graph and replayed.

A serving loop captures the attention call once and replays it every step.
The captured work must allocate nothing and record no memory fills, and each
replay must give exactly what an eager call gives on the same inputs (the
kernels are deterministic).  Between replays the test writes new query values
with ordinary eager work and synchronises, as a decode loop would.
"""
import pytest
import torch

from decode_attention_paged_06_amd import paged_attention_decode, paged_attention_prefill
from gpu_util import device, make, to_device
from workloads import prefill_inputs

pytestmark = pytest.mark.gpu

WS_BYTES = 64 << 20

DECODE_CASES = {
    # small batch, long context: split partitions + reduce
    "gqa_split": dict(num_seqs=2, num_heads=64, num_kv_heads=8, head_size=128, block_size=16,
                      dtype="bf16", context_lens=3000),
    # 48-head groups, ragged, ALiBi: equal shares of the staged decode + reduce
    "mqa_equal_shares": dict(num_seqs=32, num_heads=48, num_kv_heads=1, head_size=128,
                             block_size=16, dtype="f16", context_lens=(64, 4000), alibi=True),
    # the same cut into partitions: unit-order kernel + staged decode + reduce
    "mqa_longest_first": dict(num_seqs=32, num_heads=48, num_kv_heads=1, head_size=128,
                              block_size=16, dtype="f16", context_lens=(64, 4000), alibi=True,
                              schedule="longest_first"),
    # FP8 cache, one pass
    "gqa_fp8_single": dict(num_seqs=64, num_heads=64, num_kv_heads=8, head_size=128,
                           block_size=16, dtype="bf16", context_lens=700, kv_dtype="fp8"),
    # MHA on the VALU engine
    "mha_valu": dict(num_seqs=8, num_heads=40, num_kv_heads=40, head_size=128, block_size=16,
                     dtype="f16", context_lens=256),
}


def capture_and_check(call, query, what, lens=None, max_len=0):
    """Capture `call` into a graph and replay it four times, writing new query
    values (and, with `lens`, new context lengths up to `max_len`) between
    replays as a decode loop would; every replay must equal an eager call."""
    dev = query.device
    ws_g = torch.empty(WS_BYTES, dtype=torch.uint8, device=dev)
    ws_e = torch.empty(WS_BYTES, dtype=torch.uint8, device=dev)
    out_g = torch.full_like(query, float("nan"))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(out_g, ws_g)  # first call outside the capture (device attributes are cached)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(out_g, ws_g)
    gen = torch.Generator(device=dev).manual_seed(11)
    for rep in range(4):
        query.copy_(torch.randn(query.shape, generator=gen, device=dev).to(query.dtype))
        if lens is not None:  # the batch's lengths move between steps (within the plan's bound)
            lens.copy_(torch.randint(0, max_len + 1, lens.shape, generator=gen, device=dev,
                                     dtype=lens.dtype))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        out_e = torch.full_like(query, float("nan"))
        call(out_e, ws_e)
        torch.cuda.synchronize()
        assert torch.isfinite(out_g.float()).all(), f"{what} replay {rep}: non-finite output"
        assert torch.equal(out_g, out_e), f"{what} replay {rep}: differs from the eager call"


@pytest.mark.parametrize("case", list(DECODE_CASES))
def test_decode_graph_replay(case):
    dev = device()
    args = dict(DECODE_CASES[case])
    schedule = args.pop("schedule", "auto")
    inp = to_device(make(seed=31, poison=True, **args), dev)

    def call(out, ws):
        paged_attention_decode(out, inp.query, inp.key_cache, inp.value_cache, inp.block_tables,
                               inp.context_lens, inp.scale, inp.block_size, inp.alibi_slopes,
                               workspace=ws, k_scale=inp.k_scale, v_scale=inp.v_scale,
                               schedule=schedule)

    capture_and_check(call, inp.query, case)


@pytest.mark.parametrize("schedule", ["equal_shares", "longest_first"])
def test_decode_graph_replay_with_moving_lengths(schedule):
    """The split plan is fixed at capture (it depends only on the host-known
    bound max_blocks_per_seq * block_size); the device-side schedule -- the
    equal shares' tile prefix, the longest-first order -- is rebuilt from the
    lengths on every replay."""
    dev = device()
    inp = to_device(make(seed=33, num_seqs=24, num_heads=48, num_kv_heads=1, head_size=128,
                         block_size=16, dtype="f16", context_lens=(64, 4000), alibi=True), dev)
    max_len = inp.block_tables.shape[1] * inp.block_size

    def call(out, ws):
        paged_attention_decode(out, inp.query, inp.key_cache, inp.value_cache, inp.block_tables,
                               inp.context_lens, inp.scale, inp.block_size, inp.alibi_slopes,
                               workspace=ws, schedule=schedule)

    capture_and_check(call, inp.query, f"moving lengths, {schedule}", lens=inp.context_lens,
                      max_len=max_len)


def test_equal_shares_first_call_under_capture():
    """The first equal-share call of a configuration looks up the decode
    kernel's occupancy on the device; made under graph capture (a configuration
    -- bf16, head size 64, 33..48-head groups, FP8 cache -- that the tests
    before this one do not run), it must still capture and replay correctly."""
    dev = device()
    inp = to_device(make(seed=34, num_seqs=20, num_heads=40, num_kv_heads=1, head_size=64,
                         block_size=16, dtype="bf16", context_lens=(1, 3000), alibi=True,
                         kv_dtype="fp8"), dev)
    ws_g = torch.empty(WS_BYTES, dtype=torch.uint8, device=dev)
    out_g = torch.full_like(inp.query, float("nan"))
    args = (inp.query, inp.key_cache, inp.value_cache, inp.block_tables, inp.context_lens, inp.scale,
            inp.block_size, inp.alibi_slopes)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
        paged_attention_decode(out_g, *args, workspace=ws_g, k_scale=inp.k_scale, v_scale=inp.v_scale,
                               schedule="equal_shares")
    for rep in range(3):
        graph.replay()
        torch.cuda.synchronize()
        out_e = torch.full_like(inp.query, float("nan"))
        paged_attention_decode(out_e, *args, workspace=torch.empty_like(ws_g), k_scale=inp.k_scale,
                               v_scale=inp.v_scale, schedule="equal_shares")
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), f"replay {rep} differs from the eager call"


def test_prefill_graph_replay():
    dev = device()
    inp, q, qs, max_q = prefill_inputs(new_tokens=[40, 1, 300, 7], seed=32, device=dev,
                                       num_seqs=4, num_heads=32, num_kv_heads=4, head_size=128,
                                       block_size=16, dtype="bf16",
                                       context_lens=[100, 2000, 900, 7], alibi=True, poison=True)

    def call(out, ws):
        paged_attention_prefill(out, q, inp.key_cache, inp.value_cache, inp.block_tables,
                                inp.context_lens, qs, max_q, inp.scale, inp.block_size,
                                inp.alibi_slopes, workspace=ws, partition_size=256)

    capture_and_check(call, q, "prefill")
