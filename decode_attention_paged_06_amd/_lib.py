"""ctypes declarations of the C ABI in include/paged_attention.h.

Loading fails loudly when libpagedattn.so has not been built: there is no
fallback implementation anywhere in this package.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpagedattn.so")

PA_F16, PA_BF16, PA_FP8_E4M3 = 0, 1, 2
PA_KV_NATIVE, PA_KV_FP8_E4M3 = 0, 1
PA_KV_SEPARATE, PA_KV_JOINT = 0, 1
PA_ENGINE_AUTO, PA_ENGINE_VALU, PA_ENGINE_MFMA = 0, 1, 2
PA_SCHEDULE_AUTO, PA_SCHEDULE_GRID, PA_SCHEDULE_LONGEST_FIRST, PA_SCHEDULE_EQUAL_SHARES = 0, 1, 2, 3
# PA_NOALLOC_SCRATCH_BYTES of include/paged_attention.h
NOALLOC_SCRATCH_BYTES = 32 << 20
STATUS = {0: "PA_OK", 1: "PA_ERR_INVALID_ARG", 2: "PA_ERR_UNSUPPORTED", 3: "PA_ERR_ALIGNMENT",
          4: "PA_ERR_WORKSPACE", 5: "PA_ERR_LAUNCH", 6: "PA_ERR_DEVICE"}

# Every symbol include/paged_attention.h declares.
EXPORTS = ("paged_attention_decode", "paged_attention_decode_noalloc", "paged_attention_workspace_bytes", "paged_attention_plan",
           "paged_attention_prefill", "paged_attention_prefill_workspace_bytes",
           "paged_attention_prefill_plan", "gather_cached_kv", "paged_kv_cache_write",
           "pa_status_string", "pa_last_error")
# The measurement aids of csrc/measure.h (exported, not part of the public header).
MEASURE_EXPORTS = ("pa_stream_read_probe", "pa_stream_read_sink_bytes", "pa_share_occupancy")


class PaDims(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_size", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("kv_format", ctypes.c_int32), ("k_scale", ctypes.c_float),
                ("v_scale", ctypes.c_float), ("kv_layout", ctypes.c_int32)]


class PaOpts(ctypes.Structure):
    _fields_ = [("partition_size", ctypes.c_int32), ("engine", ctypes.c_int32),
                ("num_cus", ctypes.c_int32), ("schedule", ctypes.c_int32)]


class PaPlan(ctypes.Structure):
    _fields_ = [("num_partitions", ctypes.c_int32), ("partition_size", ctypes.c_int32),
                ("engine", ctypes.c_int32), ("schedule", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_size_t)]


class PagedAttentionError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m decode_attention_paged_06_amd.build` "
                          "(or __graft_entry__.build()) first")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    L.paged_attention_decode.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_float, i32, vp, vp,
                                         ctypes.POINTER(PaDims), vp, sz, ctypes.POINTER(PaOpts)]
    L.paged_attention_decode.restype = ctypes.c_int
    L.paged_attention_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_float, i32, vp,
                                                 vp, ctypes.POINTER(PaDims), ctypes.POINTER(PaOpts)]
    L.paged_attention_decode_noalloc.restype = ctypes.c_int
    L.paged_attention_workspace_bytes.argtypes = [ctypes.POINTER(PaDims), ctypes.POINTER(PaOpts)]
    L.paged_attention_workspace_bytes.restype = sz
    L.paged_attention_plan.argtypes = [ctypes.POINTER(PaDims), sz, ctypes.POINTER(PaOpts),
                                       ctypes.POINTER(PaPlan)]
    L.paged_attention_plan.restype = ctypes.c_int
    L.paged_attention_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, ctypes.c_float,
                                          i32, vp, vp, ctypes.POINTER(PaDims), vp, sz,
                                          ctypes.POINTER(PaOpts)]
    L.paged_attention_prefill.restype = ctypes.c_int
    L.paged_attention_prefill_workspace_bytes.argtypes = [ctypes.POINTER(PaDims), i32, i32,
                                                          ctypes.POINTER(PaOpts)]
    L.paged_attention_prefill_workspace_bytes.restype = sz
    L.paged_attention_prefill_plan.argtypes = [ctypes.POINTER(PaDims), i32, i32, sz,
                                               ctypes.POINTER(PaOpts), ctypes.POINTER(PaPlan)]
    L.paged_attention_prefill_plan.restype = ctypes.c_int
    L.gather_cached_kv.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp]
    L.gather_cached_kv.restype = ctypes.c_int
    L.paged_kv_cache_write.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp]
    L.paged_kv_cache_write.restype = ctypes.c_int
    L.pa_stream_read_probe.argtypes = [vp, sz, sz, vp, sz, vp]
    L.pa_stream_read_probe.restype = ctypes.c_int
    L.pa_stream_read_sink_bytes.argtypes = [sz]
    L.pa_stream_read_sink_bytes.restype = sz
    L.pa_share_occupancy.argtypes = [ctypes.POINTER(PaDims), ctypes.POINTER(i32), ctypes.POINTER(i32),
                                     ctypes.POINTER(i32)]
    L.pa_share_occupancy.restype = ctypes.c_int
    L.pa_status_string.argtypes = [ctypes.c_int]
    L.pa_status_string.restype = ctypes.c_char_p
    L.pa_last_error.argtypes = []
    L.pa_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def check(status: int) -> None:
    if status != 0:
        raise PagedAttentionError(status, lib().pa_last_error().decode())
