"""The C-ABI library on the CPU: exports, planner, validation and error paths.

No call here reaches a kernel launch: every decode/gather call is made with
arguments the host layer must reject first.
"""
import ctypes
import os
import re
import subprocess
import sys

import pytest

from decode_attention_paged_06_amd import _lib
from decode_attention_paged_06_amd._lib import PaDims, PaOpts, PaPlan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "paged_attention.h")
MEASURE_HEADER = os.path.join(ROOT, "decode_attention_paged_06_amd", "csrc", "measure.h")

OK, INVALID, UNSUPPORTED, ALIGN, WORKSPACE = 0, 1, 2, 3, 4


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def header_functions(path=None):
    text = open(path or HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(L):
    declared = header_functions()
    assert set(declared) == set(_lib.EXPORTS), declared
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared:
        assert name in exported, name
        assert getattr(L, name) is not None
    # the measurement aid lives in an internal header, exported for the bench only
    internal = header_functions(MEASURE_HEADER)
    assert set(internal) == set(_lib.MEASURE_EXPORTS), internal
    for name in internal:
        assert name in exported, name


def test_product_package_does_not_load_the_oracle():
    code = ("import sys; sys.path.insert(0, %r); import decode_attention_paged_06_amd as p; "
            "p._lib.lib(); assert not any(m == 'oracle' or m.startswith('oracle.') "
            "for m in sys.modules), 'oracle imported'" % ROOT)
    subprocess.run([sys.executable, "-c", code], check=True)
    for dirpath, _, files in os.walk(os.path.join(ROOT, "decode_attention_paged_06_amd")):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                src = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle", src, re.M), f


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", "/nonexistent/libpagedattn.so")
    with pytest.raises(ImportError):
        _lib.lib()


def dims(S=256, Hq=64, Hkv=8, D=128, BS=16, NB=65536, MAXB=256, dtype=1):
    return PaDims(S, Hq, Hkv, D, BS, NB, MAXB, dtype)


def plan(L, d, ws=1 << 40, ps=0, engine=0, cus=256, schedule=0):
    p = PaPlan()
    st = L.paged_attention_plan(ctypes.byref(d), ws, ctypes.byref(PaOpts(ps, engine, cus, schedule)),
                                ctypes.byref(p))
    return st, p


def test_plan_large_batch_is_single_pass(L):
    st, p = plan(L, dims())
    assert st == OK and p.num_partitions == 1 and p.workspace_bytes == 0
    assert p.engine == 2  # GQA group of 8 runs on the matrix cores


def test_plan_small_batch_splits(L):
    for S in (1, 4, 16):
        st, p = plan(L, dims(S=S))
        assert st == OK and p.num_partitions > 1
        assert p.partition_size % 16 == 0
        assert p.num_partitions * p.partition_size >= 256 * 16
        assert (p.num_partitions - 1) * p.partition_size < 256 * 16
        rows = S * 64 * p.num_partitions
        assert p.workspace_bytes >= rows * 128 * 4 + rows * 8


def test_plan_engine_choice(L):
    assert plan(L, dims(Hq=40, Hkv=40, S=8))[1].engine == 1   # MHA: vector ALU path
    assert plan(L, dims(Hq=48, Hkv=1))[1].engine == 2          # MQA: matrix cores
    assert plan(L, dims(), engine=1)[1].engine == 1
    assert plan(L, dims(), engine=7)[0] == INVALID


def test_plan_forced_partitions(L):
    st, p = plan(L, dims(S=256), ps=-1)
    assert st == OK and p.num_partitions == 1
    st, p = plan(L, dims(S=256), ps=512)
    assert st == OK and p.num_partitions == 8 and p.partition_size == 512
    st, p = plan(L, dims(MAXB=4), ps=64)
    assert st == OK and p.num_partitions == 1
    assert plan(L, dims(), ps=40)[0] == INVALID
    assert plan(L, dims(), ps=-5)[0] == INVALID
    assert plan(L, dims(S=2), ps=256, ws=1024)[0] == WORKSPACE


def test_plan_shrinks_to_workspace(L):
    st, full = plan(L, dims(S=1))
    assert st == OK and full.num_partitions > 2
    st, p = plan(L, dims(S=1), ws=full.workspace_bytes // 3)
    assert st == OK and 1 <= p.num_partitions < full.num_partitions
    assert p.workspace_bytes <= full.workspace_bytes // 3
    st, p = plan(L, dims(S=1), ws=0)
    assert st == OK and p.num_partitions == 1


def test_workspace_bytes_matches_plan(L):
    for S in (1, 4, 64, 256):
        d = dims(S=S)
        o = PaOpts(0, 0, 256, 0)
        assert L.paged_attention_workspace_bytes(ctypes.byref(d), ctypes.byref(o)) == \
            plan(L, d)[1].workspace_bytes
    bad = dims(Hq=63)
    assert L.paged_attention_workspace_bytes(ctypes.byref(bad), None) == 0


@pytest.mark.parametrize("field,value,code", [
    ("num_heads", 63, INVALID),          # 63 % 8 != 0 (head_mapping needs a multiple)
    ("num_heads", 0, INVALID),
    ("num_kv_heads", 0, INVALID),
    ("head_size", 96, UNSUPPORTED),
    ("block_size", 12, UNSUPPORTED),     # not a power of two
    ("block_size", 4, UNSUPPORTED),      # below the smallest built tile
    ("block_size", 512, UNSUPPORTED),
    ("dtype", 7, UNSUPPORTED),
    ("num_blocks", 0, INVALID),
    ("max_blocks_per_seq", 0, INVALID),
    ("num_seqs", -1, INVALID),
])
def test_plan_rejects_bad_dims(L, field, value, code):
    d = dims()
    setattr(d, field, value)
    assert plan(L, d)[0] == code
    assert L.pa_last_error().decode()


def test_fp8_cache_validation(L):
    d = dims()
    d.kv_format = 1                      # FP8 E4M3 caches need positive finite scales
    assert plan(L, d)[0] == INVALID
    d.k_scale, d.v_scale = 0.5, float("inf")
    assert plan(L, d)[0] == INVALID
    d.v_scale = 0.25
    assert plan(L, d)[0] == OK
    d.kv_format = 3
    assert plan(L, d)[0] == UNSUPPORTED
    g = L.gather_cached_kv               # fp8 rows of head size 8 are 8 bytes: not 16-byte rows
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 8, 16, 10, 2, 0, None) == UNSUPPORTED
    assert g(None, None, None, None, None, 0, 8, 16, 16, 10, 2, 0, None) == OK


def test_prefill_validation(L):
    d = dims(S=4)
    o = PaOpts(-1, 1, 256, 0)      # the VALU engine cannot run multi-query calls
    pf = L.paged_attention_prefill
    args = lambda **k: (k.get("out", FAKE), FAKE, FAKE, FAKE, FAKE, FAKE, k.get("qs", FAKE),  # noqa: E731
                        k.get("T", 100), k.get("maxq", 40), ctypes.c_float(0.1), 16, None, None,
                        ctypes.byref(d), None, 0, ctypes.byref(k.get("opts", PaOpts(-1, 0, 256, 0))))
    assert pf(*args(opts=o)) == UNSUPPORTED
    assert pf(*args(qs=None)) == INVALID
    assert pf(*args(T=-1)) == INVALID
    assert pf(*args(maxq=70000)) == INVALID
    assert pf(*args(qs=FAKE + 2)) == ALIGN
    assert pf(*args(T=0)) == OK and pf(*args(maxq=0)) == OK
    p = PaPlan()
    assert L.paged_attention_prefill_plan(ctypes.byref(dims(S=1, MAXB=256)), 512, 512, 1 << 40,
                                          ctypes.byref(PaOpts(0, 0, 256, 0)), ctypes.byref(p)) == OK
    assert p.engine == 2
    rows = 512 * 64 * p.num_partitions
    assert p.workspace_bytes == (0 if p.num_partitions == 1 else
                                 ((rows * 128 * 4 + 255) // 256) * 256 + rows * 8)


def test_plan_rejects_group_above_limit(L):
    assert plan(L, dims(Hq=128, Hkv=1))[0] == UNSUPPORTED


FAKE = 0x10000  # never dereferenced: each call below fails validation first


def decode(L, d, out=FAKE, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, cl=FAKE, scale=0.1, bs=16, alibi=None,
           ws=None, ws_bytes=0, ps=-1):
    return L.paged_attention_decode(out, q, k, v, bt, cl, ctypes.c_float(scale), bs, alibi, None,
                                    ctypes.byref(d) if d is not None else None, ws, ws_bytes,
                                    ctypes.byref(PaOpts(ps, 0, 256, 0)))


def test_decode_validation(L):
    assert decode(L, None) == INVALID
    assert decode(L, dims(Hq=60)) == INVALID
    assert decode(L, dims(), bs=8) == INVALID                 # argument vs dims mismatch
    assert decode(L, dims(), scale=float("nan")) == INVALID
    assert decode(L, dims(), scale=float("inf")) == INVALID
    assert decode(L, dims(), q=None) == INVALID
    assert decode(L, dims(), cl=None) == INVALID
    assert decode(L, dims(), out=FAKE + 8) == ALIGN
    assert decode(L, dims(), k=FAKE + 2) == ALIGN
    assert decode(L, dims(), bt=FAKE + 2) == ALIGN
    assert decode(L, dims(), alibi=FAKE + 1) == ALIGN
    assert decode(L, dims(), ps=64) == WORKSPACE              # forced split, no workspace
    assert decode(L, dims(S=1), ps=64, ws=FAKE + 16, ws_bytes=1 << 30) == ALIGN
    assert "workspace" in L.pa_last_error().decode()
    # nothing to do: succeeds without touching any pointer or device
    assert decode(L, dims(S=0), out=None, q=None, k=None, v=None, bt=None, cl=None) == OK
    assert L.pa_last_error().decode() == ""


def test_gather_validation(L):
    g = L.gather_cached_kv
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 128, 16, 10, 5, 0, None) == UNSUPPORTED
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 12, 16, 10, 0, 0, None) == UNSUPPORTED
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, -1, 8, 128, 16, 10, 0, 0, None) == INVALID
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 0, 128, 16, 10, 0, 0, None) == INVALID
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 128, 0, 10, 0, 0, None) == INVALID
    assert g(None, FAKE, FAKE, FAKE, FAKE, 4, 8, 128, 16, 10, 0, 0, None) == INVALID
    assert g(FAKE + 4, FAKE, FAKE, FAKE, FAKE, 4, 8, 128, 16, 10, 0, 0, None) == ALIGN
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE + 2, 4, 8, 128, 16, 10, 0, 0, None) == ALIGN
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, 64, 128, 16, 10, 0, 0, None) == INVALID
    # 2^31 16-byte pieces (2^24 tokens x 8 heads x 16 pieces), and just below 2^32: the
    # kernels' 32-bit grid-stride counters could wrap around, so both are refused
    for n in (1 << 24, (1 << 25) - 1):
        assert g(FAKE, FAKE, FAKE, FAKE, FAKE, n, 8, 128, 16, 10, 0, 0, None) == INVALID
        assert "too large" in L.pa_last_error().decode()
        assert L.paged_kv_cache_write(FAKE, FAKE, FAKE, FAKE, FAKE, n, 8, 128, 16, 10, 0, 0,
                                      None) == INVALID
    assert g(None, None, None, None, None, 0, 8, 128, 16, 10, 0, 0, None) == OK


def test_cache_write_validation(L):
    w = L.paged_kv_cache_write
    assert w(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 128, 16, 10, 9, 0, None) == UNSUPPORTED
    assert w(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 100, 16, 10, 0, 0, None) == UNSUPPORTED
    assert w(FAKE, FAKE, FAKE, FAKE, FAKE, -2, 8, 128, 16, 10, 0, 0, None) == INVALID
    assert w(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 128, 16, 0, 0, 0, None) == INVALID
    assert w(FAKE, None, FAKE, FAKE, FAKE, 4, 8, 128, 16, 10, 0, 0, None) == INVALID
    assert w(FAKE, FAKE, FAKE + 8, FAKE, FAKE, 4, 8, 128, 16, 10, 0, 0, None) == ALIGN
    assert w(FAKE, FAKE, FAKE, FAKE, FAKE + 1, 4, 8, 128, 16, 10, 0, 0, None) == ALIGN
    assert w(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 128, 1 << 20, 1 << 12, 0, 0, None) == INVALID
    assert w(None, None, None, None, None, 0, 8, 128, 16, 10, 1, 0, None) == OK


def test_kv_layout_validation(L):
    d = dims()
    d.kv_layout = 2                      # neither separate nor joint
    assert plan(L, d)[0] == INVALID
    tile = 16 * 128 * 2                  # block_size * head_size * 2 bytes
    d = dims()
    d.kv_layout = 1                      # joint: value tiles must follow key tiles
    assert plan(L, d)[0] == OK
    assert decode(L, d, k=FAKE, v=FAKE + 2 * tile) == INVALID
    assert "joint" in L.pa_last_error().decode()
    assert decode(L, d, k=FAKE + 4 * tile, v=FAKE) == INVALID
    g, w = L.gather_cached_kv, L.paged_kv_cache_write
    for f in (g, w):
        assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 128, 16, 10, 0, 7, None) == INVALID
        assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 128, 16, 10, 0, 1, None) == INVALID
        assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 128, 16, 10, 1, 1, None) == INVALID
        assert f(None, None, None, None, None, 0, 8, 128, 16, 10, 0, 1, None) == OK


def test_plan_block_sizes(L):
    for bs, maxb in ((8, 512), (32, 128), (256, 16)):
        st, p = plan(L, dims(S=1, BS=bs, MAXB=maxb))
        assert st == OK and p.num_partitions > 1 and p.partition_size % bs == 0
        assert p.partition_size >= 64           # one-head-tile decode: 64-token minimum
        assert p.num_partitions * p.partition_size >= maxb * bs


def test_plan_one_tile_targets_one_group_per_cu(L):
    # GQA 64/8 (one 16-head tile): about one workgroup per CU, partitions of
    # 64+ tokens; 256 CUs
    for S, maxb, P in ((1, 256, 32), (4, 256, 8), (16, 256, 2), (1, 64, 16), (4, 64, 8),
                       (16, 64, 2), (64, 256, 1)):
        st, p = plan(L, dims(S=S, MAXB=maxb))
        assert st == OK and p.engine == 2 and p.num_partitions == P, (S, maxb, p.num_partitions)
    # a 48-head group (three tiles) cut into partitions keeps two workgroups per CU
    st, p = plan(L, dims(S=64, Hq=48, Hkv=1, MAXB=256), schedule=2)
    assert st == OK and p.num_partitions == 8
    # over an FP8 cache: two per CU, partitions of 128+ tokens
    for S, maxb, P in ((1, 256, 32), (4, 256, 16), (16, 256, 4), (1, 64, 8), (4, 64, 8),
                       (16, 64, 4), (64, 256, 1)):
        d = dims(S=S, MAXB=maxb)
        d.kv_format, d.k_scale, d.v_scale = 1, 0.5, 0.5
        st, p = plan(L, d)
        assert st == OK and p.engine == 2 and p.num_partitions == P, (S, maxb, p.num_partitions)


def test_plan_multi_tile_partitions(L):
    # 48-head MQA, batch 256, contexts up to 8192: two partitions per sequence
    # when the work is cut into partitions
    st, p = plan(L, dims(S=256, Hq=48, Hkv=1, MAXB=512), schedule=2)
    assert st == OK and p.engine == 2 and p.num_partitions == 2 and p.partition_size == 4096


def test_plan_equal_shares(L):
    GRID, LONGEST, SHARES = 1, 2, 3
    mqa = dims(S=64, Hq=48, Hkv=1, MAXB=512)
    # auto, fewer items than workgroup slots: equal shares, one 12-wave workgroup
    # per CU (its LDS ring holds one)
    st, p = plan(L, mqa)
    assert st == OK and p.schedule == SHARES and p.engine == 2
    assert p.num_partitions == 256 and p.partition_size == 0
    # workspace: fp32 partials of 48 heads x (64 items + 256 workgroups) slots, (m, l)
    # pairs, the tile prefix
    slots, rows = 64 + 256, 48
    assert p.workspace_bytes >= slots * rows * (128 * 4 + 8) + 65 * 4
    # as many items as workgroup slots: longest-first partitions; on request, shares
    st, q = plan(L, dims(S=256, Hq=48, Hkv=1, MAXB=512))
    assert st == OK and q.schedule == LONGEST and q.num_partitions == 2
    st, q = plan(L, dims(S=256, Hq=48, Hkv=1, MAXB=512), schedule=SHARES)
    assert st == OK and q.schedule == SHARES and q.num_partitions == 256
    o = PaOpts(0, 0, 256, 0)
    assert L.paged_attention_workspace_bytes(ctypes.byref(mqa), ctypes.byref(o)) == p.workspace_bytes
    # a workspace too small for the shares falls back to partitions that fit
    st, q = plan(L, mqa, ws=p.workspace_bytes - 1)
    assert st == OK and q.schedule != SHARES and q.workspace_bytes < p.workspace_bytes
    # 32-head groups (4-wave workgroups, two per CU by LDS), 64-head groups (four):
    # 256 items are fewer than their workgroup slots
    st, p = plan(L, dims(S=256, Hq=32, Hkv=1, MAXB=512))
    assert st == OK and p.schedule == SHARES and p.num_partitions == 2 * 256
    st, p = plan(L, dims(S=256, Hq=64, Hkv=1, MAXB=512))
    assert st == OK and p.schedule == SHARES and p.num_partitions == 4 * 256
    # requested: even where the auto plan makes one pass
    st, p = plan(L, dims(S=1024, Hq=48, Hkv=1, MAXB=64))
    assert st == OK and p.schedule == GRID and p.num_partitions == 1
    st, p = plan(L, dims(S=1024, Hq=48, Hkv=1, MAXB=64), schedule=SHARES)
    assert st == OK and p.schedule == SHARES and p.num_partitions == 256
    # not for one head tile, nor for more than 2048 sequences, nor with a forced partition size
    st, p = plan(L, dims(S=4), schedule=SHARES)
    assert st == OK and p.schedule == GRID
    st, p = plan(L, dims(S=2048, Hq=48, Hkv=1, MAXB=4), schedule=SHARES)
    assert st == OK and p.schedule == SHARES
    st, p = plan(L, dims(S=2049, Hq=48, Hkv=1, MAXB=4), schedule=SHARES)
    assert st == OK and p.schedule != SHARES
    st, p = plan(L, mqa, ps=1024, schedule=SHARES)
    assert st == OK and p.schedule == LONGEST and p.partition_size == 1024


def test_plan_schedule(L):
    GRID, LONGEST = 1, 2
    mqa = dims(S=256, Hq=48, Hkv=1, MAXB=512)
    st, p = plan(L, mqa, schedule=LONGEST)                 # split, > 16 heads: longest first
    assert st == OK and p.num_partitions > 1 and p.schedule == LONGEST
    st, g = plan(L, mqa, schedule=GRID)
    assert st == OK and g.schedule == GRID and g.num_partitions == p.num_partitions
    # the unit order (one int32 per (sequence, partition)) and the start counter of
    # the later workgroups sit after the partials (256-byte aligned)
    order_at = (g.workspace_bytes + 255) // 256 * 256
    assert p.workspace_bytes == order_at + (256 * p.num_partitions + 1) * 4
    st, p = plan(L, dims(S=4))                             # split GQA: grid order unless asked
    assert st == OK and p.num_partitions > 1 and p.schedule == GRID
    st, p = plan(L, dims(S=4), schedule=LONGEST)
    assert st == OK and p.schedule == LONGEST
    st, p = plan(L, dims(S=256), schedule=LONGEST)         # single pass: nothing to order
    assert st == OK and p.num_partitions == 1 and p.schedule == GRID and p.workspace_bytes == 0
    st, p = plan(L, dims(S=4, Hq=8, Hkv=8), schedule=LONGEST)  # VALU engine keeps the grid
    assert st == OK and p.engine == 1 and p.schedule == GRID
    assert plan(L, dims(), schedule=4)[0] == INVALID
    assert plan(L, dims(), schedule=-1)[0] == INVALID
    d = dims(S=256, Hq=48, Hkv=1, MAXB=512)
    o = PaOpts(0, 0, 256, LONGEST)
    assert L.paged_attention_workspace_bytes(ctypes.byref(d), ctypes.byref(o)) == \
        plan(L, d, schedule=LONGEST)[1].workspace_bytes


def test_status_strings(L):
    for code in range(7):
        assert L.pa_status_string(code).decode()
    assert L.pa_status_string(99).decode() == "unknown status"


def test_last_error_is_per_thread(L):
    """Concurrent callers each read their own failure message (the foreign calls
    release the interpreter lock, so the threads do run in the library at once)."""
    import threading

    L.pa_last_error.restype = ctypes.c_char_p
    failures = []

    def worker(t):
        bad = dims(Hq=64 + t, Hkv=8)  # not a multiple: the message names 64 + t
        good = dims(S=256)
        for _ in range(2000):
            st, _ = plan(L, bad)
            msg = L.pa_last_error().decode()
            if st != INVALID or f"({64 + t})" not in msg:
                failures.append((t, st, msg))
                return
            st, _ = plan(L, good)
            if st != OK or L.pa_last_error().decode() != "":
                failures.append((t, st, "not cleared"))
                return

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(1, 7)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not failures, failures[:3]


def test_binding_detects_cache_layout():
    import torch

    from decode_attention_paged_06_amd import kv_layout_of

    NB, Hkv, BS, D = 5, 3, 16, 64
    k = torch.zeros((NB, Hkv, BS, D), dtype=torch.float16)
    v = torch.zeros_like(k)
    assert kv_layout_of(k, v) == 0
    kv = torch.zeros((NB, Hkv, 2, BS, D), dtype=torch.bfloat16)
    assert kv_layout_of(kv[:, :, 0], kv[:, :, 1]) == 1
    with pytest.raises(ValueError):       # V tiles must follow K tiles
        kv_layout_of(kv[:, :, 1], kv[:, :, 0])
    kv16 = torch.zeros((NB, Hkv, 2, BS, D), dtype=torch.float16)
    with pytest.raises(ValueError):       # one dense, one strided
        kv_layout_of(k, kv16[:, :, 1])
    kv2 = torch.zeros((NB, 2, Hkv, BS, D), dtype=torch.float16)
    with pytest.raises(ValueError):       # [NB, 2, Hkv, BS, D] is not a supported layout
        kv_layout_of(kv2[:, 0], kv2[:, 1])
    with pytest.raises(ValueError):
        kv_layout_of(k, v[:, :, :8])


def test_stream_read_probe_validation(L):
    p = L.pa_stream_read_probe
    assert L.pa_stream_read_sink_bytes(0) == 0
    assert L.pa_stream_read_sink_bytes(16 * 2048) == 16            # one workgroup per 32 KB
    assert L.pa_stream_read_sink_bytes(1 << 32) == 16 * 4096      # grid capped at 4096 workgroups
    assert p(FAKE, 24, 0, FAKE, 1 << 20, None) == INVALID           # not a multiple of 16
    assert p(None, 1024, 0, FAKE, 1 << 20, None) == INVALID
    assert p(FAKE + 8, 1024, 0, FAKE, 1 << 20, None) == ALIGN
    assert p(FAKE, 1 << 20, 0, FAKE, 16, None) == INVALID           # sink too small
    assert p(FAKE, 1 << 20, 1000, FAKE, 1 << 20, None) == INVALID   # runs: powers of two >= 1 KB
    assert p(FAKE, 3 << 13, 1 << 13, FAKE, 1 << 20, None) == INVALID  # run count not a power of two
    assert p(None, 0, 0, None, 0, None) == OK
