"""CPU oracle for paged decode attention and the paged-KV gather.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP library.

What it computes (plain definitions, float64, on the exact values of the
16-bit inputs):

* Decode attention for a single new query token per head, over K/V vectors
  kept in fixed-size physical cache blocks and reached through a per-sequence
  block table ("single_query_cached_kv_attention", vLLM PR #420; paged KV
  cache as used in vLLM PR #2744):

      out[s, h] = softmax(scale * K_s[kvh] q[s, h] + bias_h) V_s[kvh]

  over the context tokens t = 0 .. L_s - 1 of sequence s.

* GQA/MQA head mapping: query head h reads KV head h // (Hq / Hkv), the
  ``head_mapping = repeat_interleave(arange(num_kv_heads), num_queries_per_kv)``
  of the review suggestion in vLLM PR #452 ("Optimize MQA Kernel"), with
  Hq % Hkv == 0 asserted there.

* Optional ALiBi bias (the ``use_alibi`` switch of the kernel-latency
  benchmark in vLLM PR #2744): bias_h(t) = slope_h * (t - (L - 1)).  The pages
  give no formula; this is the usual linear distance penalty anchored at the
  query position.  Any per-row constant gives the same softmax.

* gather_cached_kv (vLLM PR #29, "Memcpy kernel for flash attention"): copy
  the K/V rows of a list of cache slots into contiguous [T, Hkv, D] arrays,
  bit for bit.  slot = physical_block * block_size + offset; a negative slot
  yields a zero row.

* kv_cache_write: the cache operation that stores each new token's K/V rows
  into its slot before attention runs (the cache op whose cost at block size
  256 vLLM PR #2744 discusses), bit for bit; a negative slot is skipped.

Readings of points the pages leave open (cache layout [NB, Hkv, BS, D], the
new token already in the cache at position L - 1, L <= 0 giving zeros) are
listed with the rest of the design notes; every function below states the one
it relies on.

Parity pins for every function live in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

# ----------------------------------------------------------------------------
# 16-bit storage formats
# ----------------------------------------------------------------------------


def to_float64(raw, dtype: str) -> np.ndarray:
    """Exact float64 values of fp16 ('f16') or bf16 ('bf16') storage bits.

    bf16 is the upper half of an IEEE binary32 word, so its value is the
    binary32 whose low 16 bits are zero.  fp16 is IEEE binary16.
    """
    raw = np.asarray(raw)
    if raw.dtype != np.uint16:
        raise TypeError("expected raw uint16 storage bits")
    if dtype == "f16":
        return raw.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (raw.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def fp8_e4m3_value(code: int) -> float:
    """Value of one FP8 E4M3 code (OCP "E4M3FN": bias 7, no infinities, 0x7F/0xFF NaN).

    The pages name an fp8 KV cache without fixing a format; this is the reading
    taken (the format gfx950's conversion instructions implement).
    """
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:
        return sign * man * 2.0 ** -9              # subnormal: man/8 * 2^(1-7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


_FP8_TABLE = np.array([fp8_e4m3_value(c) for c in range(256)], dtype=np.float64)


def fp8_to_float64(raw) -> np.ndarray:
    """Exact float64 values of FP8 E4M3 storage bytes (uint8)."""
    raw = np.asarray(raw)
    if raw.dtype != np.uint8:
        raise TypeError("expected raw uint8 storage bytes")
    return _FP8_TABLE[raw]


def round_to_storage(x, dtype: str) -> np.ndarray:
    """Round float64 values to the 16-bit format with round-to-nearest-even.

    Used only to state the output rounding the GPU path performs; the oracle
    itself reports float64.
    """
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f16":
        with np.errstate(over="ignore"):
            return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        with np.errstate(over="ignore"):
            f = x.astype(np.float32)
        bits = f.view(np.uint32).astype(np.uint64)
        nan = np.isnan(f)
        lsb = (bits >> np.uint64(16)) & np.uint64(1)
        rounded = ((bits + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
        rounded[nan] = 0x7FC0
        return rounded
    raise ValueError(f"unknown dtype {dtype!r}")


# ----------------------------------------------------------------------------
# Pieces of the definition (kept separate so each can be read against the pages)
# ----------------------------------------------------------------------------


def kv_head_of(h: int, num_heads: int, num_kv_heads: int) -> int:
    """KV head read by query head h (vLLM PR #452, head_mapping suggestion)."""
    if num_heads % num_kv_heads != 0:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    return h // (num_heads // num_kv_heads)


def sequence_kv(cache: np.ndarray, table_row: np.ndarray, L: int, block_size: int) -> np.ndarray:
    """Logical K (or V) rows of one sequence, [Hkv, L, D].

    Token t lives in physical block table_row[t // block_size] at offset
    t % block_size; cache layout is [num_blocks, Hkv, block_size, D].  Only the
    first ceil(L / block_size) table entries are read, and slots at or past L
    in the last block are dropped.
    """
    nb = (L + block_size - 1) // block_size
    phys = np.asarray(table_row[:nb], dtype=np.int64)
    blocks = cache[phys]                       # [nb, Hkv, BS, D]
    Hkv, D = blocks.shape[1], blocks.shape[3]
    return blocks.transpose(1, 0, 2, 3).reshape(Hkv, nb * block_size, D)[:, :L]


def alibi_bias(slope: float, L: int) -> np.ndarray:
    """slope * (t - (L - 1)) for t = 0 .. L - 1 (zero at the query's own position)."""
    return float(slope) * (np.arange(L, dtype=np.float64) - (L - 1))


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
           bias: Optional[np.ndarray]) -> np.ndarray:
    """softmax(scale * K q + bias) V for one query vector; K, V are [L, D]."""
    z = (K @ q) * float(scale)
    if bias is not None:
        z = z + bias
    w = np.exp(z - z.max())
    return (w @ V) / w.sum()


# ----------------------------------------------------------------------------
# The operations
# ----------------------------------------------------------------------------


def _as_f64(x, dtype):
    x = np.asarray(x)
    if x.dtype == np.uint8:
        return fp8_to_float64(x)
    return to_float64(x, dtype) if x.dtype == np.uint16 else x.astype(np.float64)


def paged_decode(query, key_cache, value_cache, block_tables, context_lens, scale: float,
                 block_size: int, alibi_slopes=None, dtype: Optional[str] = None,
                 seqs=None, k_scale: float = 1.0, v_scale: float = 1.0) -> np.ndarray:
    """Paged decode attention, float64 result [S, Hq, D] (or [len(seqs), Hq, D]).

    query [S, Hq, D]; key_cache/value_cache [NB, Hkv, BS, D]; block_tables
    [S, MAXB] int; context_lens [S] int; alibi_slopes [Hq] float32 or None.
    16-bit inputs are passed as raw uint16 storage bits together with
    ``dtype``; float inputs are used as given.  An FP8 E4M3 cache is passed as
    raw uint8 bytes: its value is the decoded byte times ``k_scale`` (keys) or
    ``v_scale`` (values), one fp32 scale per cache tensor.  ``seqs`` restricts
    the work to a subset of sequences (rows are returned in that order).

    L <= 0 yields a zero row (a sequence with no context has nothing to
    attend to).
    """
    q_all = np.asarray(query)
    S, Hq, D = q_all.shape
    NB, Hkv, BS, D2 = np.asarray(key_cache).shape
    if D2 != D or BS != block_size:
        raise ValueError("shape mismatch")
    tables = np.asarray(block_tables)
    lens = np.asarray(context_lens)
    slopes = None if alibi_slopes is None else np.asarray(alibi_slopes, dtype=np.float32)
    order = range(S) if seqs is None else list(seqs)
    out = np.zeros((len(order), Hq, D), dtype=np.float64)
    for row, s in enumerate(order):
        L = int(lens[s])
        if L <= 0:
            continue
        q = _as_f64(q_all[s], dtype)
        K = _as_f64(sequence_kv(key_cache, tables[s], L, block_size), dtype) * float(np.float32(k_scale))
        V = _as_f64(sequence_kv(value_cache, tables[s], L, block_size), dtype) * float(np.float32(v_scale))
        for h in range(Hq):
            kvh = kv_head_of(h, Hq, Hkv)
            bias = None if slopes is None else alibi_bias(float(slopes[h]), L)
            out[row, h] = attend(q[h], K[kvh], V[kvh], scale, bias)
    return out


def partition_stats(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                    bias: Optional[np.ndarray], lo: int, hi: int):
    """(m, l, o) of tokens [lo, hi): max logit, sum of exp(z - m), normalised output."""
    z = (K[lo:hi] @ q) * float(scale)
    if bias is not None:
        z = z + bias[lo:hi]
    m = z.max()
    w = np.exp(z - m)
    return m, w.sum(), (w @ V[lo:hi]) / w.sum()


def merge_partitions(stats):
    """Combine per-partition (m, l, o) into the full softmax-weighted output.

    With M = max m_p and w_p = l_p exp(m_p - M), the full result is
    sum_p w_p o_p / sum_p w_p.  This is an exact identity of the softmax, the
    split-context reading of the pages' "Paged attention V2" column.
    """
    M = max(m for m, _, _ in stats)
    w = [l * math.exp(m - M) for m, l, _ in stats]
    num = sum(wp * o for wp, (_, _, o) in zip(w, stats))
    return num / sum(w)


def paged_decode_partitioned(query, key_cache, value_cache, block_tables, context_lens,
                             scale: float, block_size: int, partition_size: int,
                             alibi_slopes=None, dtype: Optional[str] = None) -> np.ndarray:
    """paged_decode computed per context partition of ``partition_size`` tokens and merged."""
    q_all = np.asarray(query)
    S, Hq, D = q_all.shape
    Hkv = np.asarray(key_cache).shape[1]
    tables = np.asarray(block_tables)
    lens = np.asarray(context_lens)
    slopes = None if alibi_slopes is None else np.asarray(alibi_slopes, dtype=np.float32)
    out = np.zeros((S, Hq, D), dtype=np.float64)
    for s in range(S):
        L = int(lens[s])
        if L <= 0:
            continue
        q = _as_f64(q_all[s], dtype)
        K = _as_f64(sequence_kv(key_cache, tables[s], L, block_size), dtype)
        V = _as_f64(sequence_kv(value_cache, tables[s], L, block_size), dtype)
        for h in range(Hq):
            kvh = kv_head_of(h, Hq, Hkv)
            bias = None if slopes is None else alibi_bias(float(slopes[h]), L)
            stats = [partition_stats(q[h], K[kvh], V[kvh], scale, bias, lo,
                                     min(lo + partition_size, L))
                     for lo in range(0, L, partition_size)]
            out[s, h] = merge_partitions(stats)
    return out


def gather_cached_kv(key_cache_raw, value_cache_raw, slot_mapping, block_size: int):
    """Raw-bit copy of cache rows for each slot: ([T, Hkv, D], [T, Hkv, D]) uint16.

    Row i is cache[slot_i // block_size, :, slot_i % block_size, :] (vLLM PR #29,
    the gather benchmark's parameters: tokens, heads, head size, block size,
    pool size).  A negative slot gives a zero row.
    """
    kc = np.asarray(key_cache_raw)
    vc = np.asarray(value_cache_raw)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    T = slots.shape[0]
    Hkv, D = kc.shape[1], kc.shape[3]
    k_out = np.zeros((T, Hkv, D), dtype=kc.dtype)
    v_out = np.zeros((T, Hkv, D), dtype=vc.dtype)
    for i, slot in enumerate(slots.tolist()):
        if slot < 0:
            continue
        k_out[i] = kc[slot // block_size, :, slot % block_size, :]
        v_out[i] = vc[slot // block_size, :, slot % block_size, :]
    return k_out, v_out


def kv_cache_write(key_cache_raw, value_cache_raw, key_raw, value_raw, slot_mapping,
                   block_size: int):
    """Caches after storing token i's rows at slot_mapping[i]: (key_cache, value_cache) copies.

    key/value [T, Hkv, D] raw 16-bit words; caches [NB, Hkv, BS, D].  Row i goes
    to block slot // block_size, offset slot % block_size; a negative slot leaves
    the caches untouched.  Slots are distinct (two tokens never share a slot).
    """
    kc = np.array(key_cache_raw, copy=True)
    vc = np.array(value_cache_raw, copy=True)
    k = np.asarray(key_raw)
    v = np.asarray(value_raw)
    for i, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64).tolist()):
        if slot < 0:
            continue
        kc[slot // block_size, :, slot % block_size, :] = k[i]
        vc[slot // block_size, :, slot % block_size, :] = v[i]
    return kc, vc


def query_position(L: int, n: int, i: int) -> int:
    """Position of new token i when the last n of L context tokens are new."""
    return L - n + i


def paged_prefill(query, key_cache, value_cache, block_tables, context_lens, query_start,
                  scale: float, block_size: int, alibi_slopes=None, dtype: Optional[str] = None,
                  k_scale: float = 1.0, v_scale: float = 1.0) -> np.ndarray:
    """Causal multi-query attention over the paged cache, float64 [T, Hq, D].

    Sequence s owns query rows query_start[s] .. query_start[s+1] - 1 (T rows in
    all); they are its last n_s = query_start[s+1] - query_start[s] context
    tokens, already stored in the cache (reading taken for running the
    FlashAttention cache call on prefill chunks, vLLM PR #2744 discussion).
    Query i of s sits at position p = L_s - n_s + i and attends to positions
    0 .. p; the ALiBi bias is slope * (t - p).  With n_s = 1 this is exactly
    paged_decode.
    """
    q_all = np.asarray(query)
    T, Hq, D = q_all.shape
    Hkv = np.asarray(key_cache).shape[1]
    tables = np.asarray(block_tables)
    lens = np.asarray(context_lens)
    qs = np.asarray(query_start)
    slopes = None if alibi_slopes is None else np.asarray(alibi_slopes, dtype=np.float32)
    out = np.zeros((T, Hq, D), dtype=np.float64)
    for s in range(len(lens)):
        L = int(lens[s])
        first, n = int(qs[s]), int(qs[s + 1]) - int(qs[s])
        if n <= 0 or L <= 0:
            continue
        if n > L:
            raise ValueError("a sequence has more new tokens than context")
        K = _as_f64(sequence_kv(key_cache, tables[s], L, block_size), dtype) * float(np.float32(k_scale))
        V = _as_f64(sequence_kv(value_cache, tables[s], L, block_size), dtype) * float(np.float32(v_scale))
        for i in range(n):
            p = query_position(L, n, i)
            q = _as_f64(q_all[first + i], dtype)
            for h in range(Hq):
                kvh = kv_head_of(h, Hq, Hkv)
                bias = None if slopes is None else alibi_bias(float(slopes[h]), p + 1)
                out[first + i, h] = attend(q[h], K[kvh, :p + 1], V[kvh, :p + 1], scale, bias)
    return out
