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
                   PA_SCHEDULE_GRID,
                   PA_SCHEDULE_LONGEST_FIRST, PaDims, PaOpts, PaPlan, check, lib)

_DTYPE = {torch.float16: PA_F16, torch.bfloat16: PA_BF16, torch.float8_e4m3fn: PA_FP8_E4M3}
_ENGINE = {"auto": PA_ENGINE_AUTO, "valu": PA_ENGINE_VALU, "mfma": PA_ENGINE_MFMA}
_SCHEDULE = {"auto": PA_SCHEDULE_AUTO, "grid": PA_SCHEDULE_GRID,
             "longest_first": PA_SCHEDULE_LONGEST_FIRST}


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
    _require(out, "out", query.dtype)
    _require(query, "query", query.dtype)
    kv_dtype = torch.float8_e4m3fn if key_cache.dtype == torch.float8_e4m3fn else query.dtype
    _require(key_cache, "key_cache", kv_dtype, dense=False)
    _require(value_cache, "value_cache", kv_dtype, dense=False)
    layout = kv_layout_of(key_cache, value_cache)
    _require(block_tables, "block_tables", torch.int32)
    _require(context_lens, "context_lens", torch.int32)
    if alibi_slopes is not None:
        _require(alibi_slopes, "alibi_slopes", torch.float32)
    if query.dtype not in _DTYPE:
        raise ValueError(f"unsupported dtype {query.dtype}")
    dims = make_dims(query, key_cache, block_tables, k_scale, v_scale, layout)
    opts = make_opts(partition_size, engine, schedule=schedule)
    if workspace is None:
        nbytes = paged_attention_workspace_bytes(dims, opts)
        if nbytes:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=query.device)
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
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=query.device)
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


__all__ = ["paged_attention_decode", "paged_attention_plan", "paged_attention_workspace_bytes",
           "paged_attention_prefill", "make_prefill_dims", "gather_cached_kv", "paged_kv_cache_write",
           "make_dims", "make_opts", "joint_kv_cache", "kv_layout_of", "stream_read_probe", "_lib"]
