"""Python binding with the C ABI's names: argument marshalling only.

torch supplies device memory and the current stream; every step of the
computation runs in the HIP kernels of libpagedattn.so.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib
from ._lib import (PA_BF16, PA_ENGINE_AUTO, PA_ENGINE_MFMA, PA_ENGINE_VALU, PA_F16, PA_FP8_E4M3,
                   PA_KV_FP8_E4M3, PA_KV_JOINT, PA_KV_NATIVE, PA_KV_SEPARATE, PA_SCHEDULE_AUTO,
                   PA_SCHEDULE_EQUAL_SHARES, PA_SCHEDULE_GRID,
                   PA_SCHEDULE_LONGEST_FIRST, PaDims, PaOpts, PaPlan, check, lib)

_DTYPE = {torch.float16: PA_F16, torch.bfloat16: PA_BF16, torch.float8_e4m3fn: PA_FP8_E4M3}
_ENGINE = {"auto": PA_ENGINE_AUTO, "valu": PA_ENGINE_VALU, "mfma": PA_ENGINE_MFMA}
_SCHEDULE = {"auto": PA_SCHEDULE_AUTO, "grid": PA_SCHEDULE_GRID,
             "longest_first": PA_SCHEDULE_LONGEST_FIRST, "equal_shares": PA_SCHEDULE_EQUAL_SHARES}


def joint_kv_cache(num_blocks: int, num_kv_heads: int, block_size: int, head_size: int,
                   dtype: torch.dtype, device) -> tuple:
    """Allocate a cache in the joint layout [NB, Hkv, 2, BS, D] (uninitialised).

    Returns (key_cache, value_cache): views [NB, Hkv, BS, D] of the K and V
    tiles, which every entry point accepts like two separate tensors.
    """
    kv = torch.empty((num_blocks, num_kv_heads, 2, block_size, head_size), dtype=dtype,
                     device=device)
    return kv[:, :, 0], kv[:, :, 1]


def kv_layout_of(key_cache: torch.Tensor, value_cache: torch.Tensor) -> int:
    """PA_KV_SEPARATE for two dense caches, PA_KV_JOINT for the two views of
    one [NB, Hkv, 2, BS, D] tensor; anything else is rejected."""
    if key_cache.shape != value_cache.shape or key_cache.dim() != 4:
        raise ValueError("key_cache and value_cache must both be [NB, Hkv, BS, D]")
    if key_cache.is_contiguous() and value_cache.is_contiguous():
        return PA_KV_SEPARATE
    NB, Hkv, BS, D = key_cache.shape
    joint = (2 * Hkv * BS * D, 2 * BS * D, D, 1)
    if (key_cache.stride() == joint and value_cache.stride() == joint and
            value_cache.data_ptr() == key_cache.data_ptr() + BS * D * key_cache.element_size()):
        return PA_KV_JOINT
    raise ValueError("caches must be two dense [NB, Hkv, BS, D] tensors or the K and V views "
                     "of one dense [NB, Hkv, 2, BS, D] tensor")


def make_dims(query: torch.Tensor, key_cache: torch.Tensor, block_tables: torch.Tensor,
              k_scale: float = 1.0, v_scale: float = 1.0,
              kv_layout: int = PA_KV_SEPARATE) -> PaDims:
    S, Hq, D = query.shape
    NB, Hkv, BS, D2 = key_cache.shape
    fp8 = key_cache.dtype == torch.float8_e4m3fn
    return PaDims(S, Hq, Hkv, D, BS, NB, block_tables.shape[1], _DTYPE[query.dtype],
                  PA_KV_FP8_E4M3 if fp8 else PA_KV_NATIVE, float(k_scale), float(v_scale),
                  int(kv_layout))


def make_opts(partition_size: int = 0, engine: str = "auto", num_cus: int = 0,
              schedule: str = "auto") -> PaOpts:
    return PaOpts(int(partition_size), _ENGINE[engine], int(num_cus), _SCHEDULE[schedule])


def _stream_ptr(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _require(t: torch.Tensor, name: str, dtype=None, dense: bool = True):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dense and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _shape_error(msg: str):
    raise ValueError(msg)


def _check_attention_shapes(out, query, key_cache, value_cache, block_tables, context_lens,
                            alibi_slopes, num_seqs: int, query_start_loc=None):
    """Shapes the C layer cannot see (it gets pointers): every tensor must
    match the query and the caches, or the kernels would read or write past
    an allocation."""
    if query.dim() != 3:
        _shape_error(f"query must be [tokens, num_heads, head_size], got {tuple(query.shape)}")
    if tuple(out.shape) != tuple(query.shape):
        _shape_error(f"out {tuple(out.shape)} must have the query's shape {tuple(query.shape)}")
    if key_cache.dim() != 4 or tuple(key_cache.shape) != tuple(value_cache.shape):
        _shape_error("key_cache and value_cache must both be [num_blocks, num_kv_heads, block_size, "
                     f"head_size], got {tuple(key_cache.shape)} and {tuple(value_cache.shape)}")
    if key_cache.shape[3] != query.shape[2]:
        _shape_error(f"cache head_size {key_cache.shape[3]} differs from the query's {query.shape[2]}")
    if block_tables.dim() != 2 or block_tables.shape[0] < num_seqs:
        _shape_error(f"block_tables must be [num_seqs, max_blocks_per_seq] with at least {num_seqs} "
                     f"rows, got {tuple(block_tables.shape)}")
    if context_lens.dim() != 1 or context_lens.shape[0] != num_seqs:
        _shape_error(f"context_lens must hold {num_seqs} entries, got {tuple(context_lens.shape)}")
    if alibi_slopes is not None and (alibi_slopes.dim() != 1 or
                                     alibi_slopes.shape[0] != query.shape[1]):
        _shape_error(f"alibi_slopes must hold one slope per query head ({query.shape[1]}), got "
                     f"{tuple(alibi_slopes.shape)}")
    if query_start_loc is not None and (query_start_loc.dim() != 1 or
                                        query_start_loc.shape[0] != num_seqs + 1):
        _shape_error(f"query_start_loc must hold num_seqs + 1 = {num_seqs + 1} entries, got "
                     f"{tuple(query_start_loc.shape)}")


def _check_row_copy_shapes(rows_k, rows_v, key_cache, value_cache, slot_mapping):
    """[T, Hkv, D] row arrays against the caches and the slot list."""
    if key_cache.dim() != 4 or tuple(key_cache.shape) != tuple(value_cache.shape):
        _shape_error("key_cache and value_cache must both be [num_blocks, num_kv_heads, block_size, "
                     f"head_size], got {tuple(key_cache.shape)} and {tuple(value_cache.shape)}")
    if slot_mapping.dim() != 1:
        _shape_error(f"slot_mapping must be 1-D, got {tuple(slot_mapping.shape)}")
    want = (slot_mapping.shape[0], key_cache.shape[1], key_cache.shape[3])
    for t, n in ((rows_k, "key rows"), (rows_v, "value rows")):
        if tuple(t.shape) != want:
            _shape_error(f"{n} must be [num_tokens, num_kv_heads, head_size] = {want}, got "
                         f"{tuple(t.shape)}")


def _owned_workspace(nbytes: int, device, stream):
    """A temporary workspace for one call.  The kernels run on `stream`; when
    that is not torch's current stream the allocation is recorded on it, so
    the caching allocator does not hand the memory to other work before the
    call's kernels on `stream` are done with it."""
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    ptr = _stream_ptr(stream)
    if ptr != torch.cuda.current_stream(device).cuda_stream:
        ws.record_stream(stream if isinstance(stream, torch.cuda.Stream)
                         else torch.cuda.ExternalStream(ptr, device=device))
    return ws


# The (dims, opts) structures of recent decode calls, by everything they hold:
# a serving loop repeats one configuration every step, and building the ctypes
# structures costs more than the lookup.  The library only reads them.
_decode_struct_cache: dict = {}


def _decode_structs(out, query, key_cache, value_cache, block_tables, context_lens, alibi_slopes,
                    k_scale, v_scale, partition_size, engine, schedule):
    """Checks every tensor of a decode call; returns its (dims, opts)."""
    _check_attention_shapes(out, query, key_cache, value_cache, block_tables, context_lens,
                            alibi_slopes, query.shape[0] if query.dim() == 3 else 0)
    qdt = query.dtype
    _require(out, "out", qdt)
    _require(query, "query", qdt)
    kdt = key_cache.dtype
    kv_dtype = kdt if kdt == torch.float8_e4m3fn else qdt
    _require(key_cache, "key_cache", kv_dtype, dense=False)
    _require(value_cache, "value_cache", kv_dtype, dense=False)
    layout = kv_layout_of(key_cache, value_cache)
    _require(block_tables, "block_tables", torch.int32)
    _require(context_lens, "context_lens", torch.int32)
    if alibi_slopes is not None:
        _require(alibi_slopes, "alibi_slopes", torch.float32)
    if qdt not in _DTYPE:
        raise ValueError(f"unsupported dtype {qdt}")
    k_scale, v_scale, partition_size = float(k_scale), float(v_scale), int(partition_size)
    key = (query.shape, key_cache.shape, block_tables.shape[1], qdt, kdt, k_scale, v_scale, layout,
           partition_size, engine, schedule)
    structs = _decode_struct_cache.get(key)
    if structs is None:
        structs = (make_dims(query, key_cache, block_tables, k_scale, v_scale, layout),
                   make_opts(partition_size, engine, schedule=schedule))
        if len(_decode_struct_cache) >= 64:
            _decode_struct_cache.clear()
        _decode_struct_cache[key] = structs
    return structs


def paged_attention_plan(dims: PaDims, workspace_bytes: int, opts: Optional[PaOpts] = None) -> PaPlan:
    plan = PaPlan()
    check(lib().paged_attention_plan(ctypes.byref(dims), workspace_bytes,
                                     ctypes.byref(opts) if opts else None, ctypes.byref(plan)))
    return plan


def paged_attention_workspace_bytes(dims: PaDims, opts: Optional[PaOpts] = None) -> int:
    return int(lib().paged_attention_workspace_bytes(ctypes.byref(dims),
                                                     ctypes.byref(opts) if opts else None))


def paged_attention_decode(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
                           value_cache: torch.Tensor, block_tables: torch.Tensor,
                           context_lens: torch.Tensor, scale: float, block_size: int,
                           alibi_slopes: Optional[torch.Tensor] = None, stream=None,
                           workspace: Optional[torch.Tensor] = None, partition_size: int = 0,
                           engine: str = "auto", k_scale: float = 1.0,
                           v_scale: float = 1.0, schedule: str = "auto") -> torch.Tensor:
    """Enqueue paged decode attention; writes and returns ``out`` ([S, Hq, D]).

    Caches hold the query's dtype, or torch.float8_e4m3fn with the real values
    code * k_scale / code * v_scale.  ``workspace`` (uint8 device tensor) is
    allocated with torch when omitted and the plan needs one.
    """
    dims, opts = _decode_structs(out, query, key_cache, value_cache, block_tables, context_lens,
                                 alibi_slopes, k_scale, v_scale, partition_size, engine, schedule)
    if workspace is None:
        nbytes = paged_attention_workspace_bytes(dims, opts)
        if nbytes:
            workspace = _owned_workspace(nbytes, query.device, stream)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _require(workspace, "workspace")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    check(lib().paged_attention_decode(
        out.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
        block_tables.data_ptr(), context_lens.data_ptr(), float(scale), int(block_size),
        alibi_slopes.data_ptr() if alibi_slopes is not None else None, _stream_ptr(stream),
        ctypes.byref(dims), ws_ptr, ws_bytes, ctypes.byref(opts)))
    return out


def paged_attention_decode_noalloc(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
                                   value_cache: torch.Tensor, block_tables: torch.Tensor,
                                   context_lens: torch.Tensor, scale: float, block_size: int,
                                   alibi_slopes: Optional[torch.Tensor] = None, stream=None,
                                   partition_size: int = 0, engine: str = "auto",
                                   k_scale: float = 1.0, v_scale: float = 1.0,
                                   schedule: str = "auto") -> torch.Tensor:
    """paged_attention_decode without a workspace: the split partials go to the
    library's per-GPU scratch (see paged_attention_decode_noalloc in the C
    header; calls that overlap on one GPU race).  Allocates nothing."""
    dims, opts = _decode_structs(out, query, key_cache, value_cache, block_tables, context_lens,
                                 alibi_slopes, k_scale, v_scale, partition_size, engine, schedule)
    check(lib().paged_attention_decode_noalloc(
        out.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
        block_tables.data_ptr(), context_lens.data_ptr(), float(scale), int(block_size),
        alibi_slopes.data_ptr() if alibi_slopes is not None else None, _stream_ptr(stream),
        ctypes.byref(dims), ctypes.byref(opts)))
    return out


def make_prefill_dims(query: torch.Tensor, key_cache: torch.Tensor, block_tables: torch.Tensor,
                      num_seqs: int, k_scale: float = 1.0, v_scale: float = 1.0,
                      kv_layout: int = PA_KV_SEPARATE) -> PaDims:
    dims = make_dims(query, key_cache, block_tables, k_scale, v_scale, kv_layout)
    dims.num_seqs = int(num_seqs)
    return dims


def paged_attention_prefill(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
                            value_cache: torch.Tensor, block_tables: torch.Tensor,
                            context_lens: torch.Tensor, query_start_loc: torch.Tensor,
                            max_query_len: int, scale: float, block_size: int,
                            alibi_slopes: Optional[torch.Tensor] = None, stream=None,
                            workspace: Optional[torch.Tensor] = None, partition_size: int = 0,
                            k_scale: float = 1.0, v_scale: float = 1.0) -> torch.Tensor:
    """Enqueue causal multi-query attention for packed new tokens; returns ``out``."""
    _check_attention_shapes(out, query, key_cache, value_cache, block_tables, context_lens,
                            alibi_slopes, context_lens.shape[0] if context_lens.dim() == 1 else -1,
                            query_start_loc)
    _require(out, "out", query.dtype)
    _require(query, "query", query.dtype)
    kv_dtype = torch.float8_e4m3fn if key_cache.dtype == torch.float8_e4m3fn else query.dtype
    _require(key_cache, "key_cache", kv_dtype, dense=False)
    _require(value_cache, "value_cache", kv_dtype, dense=False)
    layout = kv_layout_of(key_cache, value_cache)
    _require(block_tables, "block_tables", torch.int32)
    _require(context_lens, "context_lens", torch.int32)
    _require(query_start_loc, "query_start_loc", torch.int32)
    if alibi_slopes is not None:
        _require(alibi_slopes, "alibi_slopes", torch.float32)
    S = context_lens.shape[0]
    T = query.shape[0]
    dims = make_prefill_dims(query, key_cache, block_tables, S, k_scale, v_scale, layout)
    opts = make_opts(partition_size, "auto")
    if workspace is None:
        nbytes = int(lib().paged_attention_prefill_workspace_bytes(
            ctypes.byref(dims), T, int(max_query_len), ctypes.byref(opts)))
        if nbytes:
            workspace = _owned_workspace(nbytes, query.device, stream)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _require(workspace, "workspace")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    check(lib().paged_attention_prefill(
        out.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
        block_tables.data_ptr(), context_lens.data_ptr(), query_start_loc.data_ptr(), T,
        int(max_query_len), float(scale), int(block_size),
        alibi_slopes.data_ptr() if alibi_slopes is not None else None, _stream_ptr(stream),
        ctypes.byref(dims), ws_ptr, ws_bytes, ctypes.byref(opts)))
    return out


def gather_cached_kv(key_out: torch.Tensor, value_out: torch.Tensor, key_cache: torch.Tensor,
                     value_cache: torch.Tensor, slot_mapping: torch.Tensor, block_size: int,
                     stream=None):
    """Enqueue the bit-exact gather of cache rows into key_out/value_out ([T, Hkv, D])."""
    _check_row_copy_shapes(key_out, value_out, key_cache, value_cache, slot_mapping)
    for t, n in ((key_out, "key_out"), (value_out, "value_out")):
        _require(t, n, key_cache.dtype)
    for t, n in ((key_cache, "key_cache"), (value_cache, "value_cache")):
        _require(t, n, key_cache.dtype, dense=False)
    layout = kv_layout_of(key_cache, value_cache)
    _require(slot_mapping, "slot_mapping", torch.int32)
    NB, Hkv, BS, D = key_cache.shape
    check(lib().gather_cached_kv(
        key_out.data_ptr(), value_out.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
        slot_mapping.data_ptr(), slot_mapping.shape[0], Hkv, D, int(block_size), NB,
        _DTYPE[key_cache.dtype], layout, _stream_ptr(stream)))
    return key_out, value_out


def paged_kv_cache_write(key_cache: torch.Tensor, value_cache: torch.Tensor, key: torch.Tensor,
                         value: torch.Tensor, slot_mapping: torch.Tensor, block_size: int,
                         stream=None):
    """Enqueue the bit-exact store of key/value rows ([T, Hkv, D]) into their cache slots."""
    _check_row_copy_shapes(key, value, key_cache, value_cache, slot_mapping)
    for t, n in ((key, "key"), (value, "value")):
        _require(t, n, key_cache.dtype)
    for t, n in ((key_cache, "key_cache"), (value_cache, "value_cache")):
        _require(t, n, key_cache.dtype, dense=False)
    layout = kv_layout_of(key_cache, value_cache)
    _require(slot_mapping, "slot_mapping", torch.int32)
    NB, Hkv, BS, D = key_cache.shape
    check(lib().paged_kv_cache_write(
        key_cache.data_ptr(), value_cache.data_ptr(), key.data_ptr(), value.data_ptr(),
        slot_mapping.data_ptr(), slot_mapping.shape[0], Hkv, D, int(block_size), NB,
        _DTYPE[key_cache.dtype], layout, _stream_ptr(stream)))
    return key_cache, value_cache


def stream_read_probe(src: torch.Tensor, sink: Optional[torch.Tensor] = None, stream=None,
                      run_bytes: int = 0):
    """Enqueue one read of ``src``'s bytes (a measurement aid; see
    pa_stream_read_probe): contiguous slices, or runs of ``run_bytes`` at
    scattered positions.  Returns the sink tensor (allocated when omitted)."""
    _require(src, "src")
    nbytes = src.numel() * src.element_size()
    need = int(lib().pa_stream_read_sink_bytes(nbytes))
    if sink is None:
        sink = torch.empty(max(need, 16), dtype=torch.uint8, device=src.device)
    _require(sink, "sink")
    check(lib().pa_stream_read_probe(src.data_ptr(), nbytes, int(run_bytes), sink.data_ptr(),
                                     sink.numel() * sink.element_size(), _stream_ptr(stream)))
    return sink


def share_occupancy(dims: PaDims):
    """(workgroups per CU the planner assumes, what the device's occupancy
    calculator reports, the piece cost in stream positions) for the
    equal-share decode kernel of these dims (a measurement aid; see
    pa_share_occupancy)."""
    t, d, c = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)
    check(lib().pa_share_occupancy(ctypes.byref(dims), ctypes.byref(t), ctypes.byref(d), ctypes.byref(c)))
    return t.value, d.value, c.value


__all__ = ["paged_attention_decode", "paged_attention_decode_noalloc", "paged_attention_plan", "paged_attention_workspace_bytes",
           "paged_attention_prefill", "make_prefill_dims", "gather_cached_kv", "paged_kv_cache_write",
           "make_dims", "make_opts", "joint_kv_cache", "kv_layout_of", "stream_read_probe", "share_occupancy", "_lib"]
