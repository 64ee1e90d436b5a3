// Device helpers shared by the gfx950 decode kernels: 16-bit storage formats,
// DPP cross-lane moves, exp2 and the online-softmax merge.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pa {

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Running-max sentinel.  Finite on purpose: masked scores take this value, so
// "sentinel - sentinel" is 0, never NaN; a state that only ever saw masked
// tokens is wiped by the exp2(sentinel - finite) = 0 rescale on the first
// real token or at the merge.
constexpr float kNegBig = -1.0e30f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Maximum of two logits or running maxima, all of which lie below kPosBig
// (masked scores are kNegBig; real logits are orders of magnitude smaller):
// the median of the two and that ceiling, one v_med3_f32 with none of the
// quieting steps that the IEEE maximum of arbitrary inputs (fmaxf) costs.
constexpr float kPosBig = 1.0e30f;
__device__ __forceinline__ float score_max(float a, float b) {
  return __builtin_amdgcn_fmed3f(a, b, kPosBig);
}
// Maximum of three logits, one v_max3_f32 (the compiler would quiet each
// input of an fmaxf chain first).
__device__ __forceinline__ float score_max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// ---- 16-bit storage formats -------------------------------------------------

struct F16 {
  static constexpr uint32_t kOnes = 0x3C003C00u;  // (1, 1) packed
  // value of the low / high half of a packed pair
  static __device__ __forceinline__ float lo(uint32_t u) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xffffu));
  }
  static __device__ __forceinline__ float hi(uint32_t u) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16));
  }
  // a.x * b.x + a.y * b.y + c, products exact, fp32 accumulate
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b),
                                  c, false);
  }
  // round-to-nearest-even pack of two floats (x in the low half)
  static __device__ __forceinline__ uint32_t pack(float x, float y) {
    f16x2_t v = {(_Float16)x, (_Float16)y};
    return __builtin_bit_cast(uint32_t, v);
  }
};

struct BF16 {
  static constexpr uint32_t kOnes = 0x3F803F80u;  // (1, 1) packed
  static __device__ __forceinline__ float lo(uint32_t u) { return __uint_as_float(u << 16); }
  static __device__ __forceinline__ float hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
  }
  static __device__ __forceinline__ uint32_t pack(float x, float y) {
    bf16x2_t v = {(__bf16)x, (__bf16)y};
    return __builtin_bit_cast(uint32_t, v);
  }
};

// Two 16-bit halves from two words: (lo half of a | lo half of b << 16) etc.
__device__ __forceinline__ uint32_t pack_lo_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// ---- cross-lane moves ---------------------------------------------------------

// DPP controls (gfx9 encoding)
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowMirror = 0x140;    // lane i <- lane 15-i within a row of 16
constexpr int kDppRowHalfMirror = 0x141;// lane i <- lane 7-i within each half row

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of N lanes (N = 8 or 16); every lane of the group
// receives the group total.  Four (three) DPP-fused adds, no LDS.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 8 || N == 16, "group of 8 or 16 lanes");
  if constexpr (N == 16) x += dpp<kDppRowMirror>(x);
  x += dpp<kDppRowHalfMirror>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppQuadXor1>(x);
  return x;
}

__device__ __forceinline__ float shfl_xor(float x, int mask) {
  const int lane = threadIdx.x & 63;
  return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __float_as_int(x)));
}

// Reductions over the four lanes l % 16 + 16 k (k = 0..3) with the gfx950
// lane-swap instructions (the maxima are of logits / running maxima, see
// score_max): permlane32_swap pairs lane l with l ^ 32 and
// permlane16_swap pairs it with l ^ 16.  Plain VALU moves, no LDS round trip;
// every lane of a group ends with the same value (max and + are commutative).
__device__ __forceinline__ float xor32_pair_max(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return score_max(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float xor16_pair_max(float x) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return score_max(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float column_max4(float x) { return xor16_pair_max(xor32_pair_max(x)); }
__device__ __forceinline__ float column_sum4(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(s[0]) + __uint_as_float(s[1]);
  const auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

// True if any lane of the wave has `p` set.
__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// Inclusive prefix sum over the 64 lanes of a wave: lane i gets x_0 + .. + x_i.
__device__ __forceinline__ int wave_prefix_sum(int x) {
  const int lane = (int)(threadIdx.x & 63);
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}

// ---- loads --------------------------------------------------------------------

// Streaming loads of K/V: every byte is read exactly once per call, so these
// are issued with the non-temporal hint (no reuse expected in the caches).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 load_nt(const uint2* p) {
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(v.x, v.y);
}

// Buffer resource (V#) over `bytes` bytes at a wave-uniform `base`: loads
// through it take the base from SGPRs and a 32-bit per-lane byte offset from
// one VGPR, and return zero (instead of faulting) past `bytes`.  Word 3 is the
// gfx9 raw-buffer configuration.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
// STREAM selects the non-temporal hint: right when one wave consumes the bytes
// (they are never read again), wrong when sibling waves re-read the same lines
// through the caches (the hint makes the caches drop them).
template <bool STREAM>
__device__ __forceinline__ uint4 buffer_load(rsrc_t r, uint32_t off, uint4*) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, STREAM ? 2 : 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
template <bool STREAM>
__device__ __forceinline__ uint2 buffer_load(rsrc_t r, uint32_t off, uint2*) {
  const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, STREAM ? 2 : 0);
  return make_uint2(v.x, v.y);
}

__device__ __forceinline__ uint32_t buffer_load_b32(rsrc_t r, uint32_t off, bool stream) {
  return stream ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 2)
                : (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}

// ---- LDS staging ----------------------------------------------------------------
//
// Buffer bytes are copied straight into LDS by the buffer-load-to-LDS
// instruction, 16 bytes per lane: lane l's bytes land at +16 l from the
// wave-uniform LDS destination; past the buffer bound the transfer writes
// zeros.  Two uses: a per-lane 16-byte piece (LdsPiece: a wave reading it back
// from the same lane position gets what a direct load would have given it),
// and a whole contiguous run copied as is (lds_copy_run: 1 KB per transfer,
// read back at the offsets a direct load would have used).
//
// The transfers are issued from inline assembly, so the compiler does not
// count them when it places its own waits (which only makes those waits
// stricter); the issuing wave waits for them with wait_vmcnt and a barrier
// publishes them to the other waves.  The statements keep their place among
// the kernel's memory accesses.  M0, which holds the LDS destination, is
// restored afterwards; an LDS transfer may not read M0 in the cycle after a
// scalar write to it (one wait state on this GPU family), hence the s_nop.
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ uint32_t lds_address(void* p) {
  return (uint32_t)(uintptr_t)(lds_void_t*)p;
}
__device__ __forceinline__ void lds_load16(rsrc_t r, uint32_t off, void* dst) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %1, %3, 0 offen nt lds\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off), "s"(lds_address(dst)), "s"(r)
      : "memory");
}

struct LdsPiece {
  static constexpr int kTransfers = 1;
  static constexpr int kBytes = 64 * 16;
  static __device__ __forceinline__ void copy(rsrc_t r, uint32_t off, char* dst) {
    lds_load16(r, off, dst);
  }
  static __device__ __forceinline__ uint4 read(const char* src, int lane) {
    return *reinterpret_cast<const uint4*>(src + 16 * lane);
  }
};

// Bytes 0 .. BYTES - 1 of the buffer to dst (BYTES 1, 2 or 4 KB; one transfer
// per KB).  The run is contiguous at both ends, so one M0 set-up serves all its
// transfers: the instruction's immediate offset advances the memory and the
// LDS address alike (measured: FP8 MQA 111.5 -> 109.1 us, prefill 611 -> 621
// TFLOP/s against an M0 set-up per transfer).
template <int BYTES>
__device__ __forceinline__ void lds_copy_run(rsrc_t r, char* dst, int lane) {
  static_assert(BYTES == 1024 || BYTES == 2048 || BYTES == 4096, "1, 2 or 4 transfers");
  const uint32_t off = 16u * lane;
  uint32_t saved;
  if constexpr (BYTES == 4096) {
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
        "buffer_load_dwordx4 %1, %3, 0 offen offset:0 nt lds\n\t"
        "buffer_load_dwordx4 %1, %3, 0 offen offset:1024 nt lds\n\t"
        "buffer_load_dwordx4 %1, %3, 0 offen offset:2048 nt lds\n\t"
        "buffer_load_dwordx4 %1, %3, 0 offen offset:3072 nt lds\n\ts_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(off), "s"(lds_address(dst)), "s"(r)
        : "memory");
  } else if constexpr (BYTES == 2048) {
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
        "buffer_load_dwordx4 %1, %3, 0 offen offset:0 nt lds\n\t"
        "buffer_load_dwordx4 %1, %3, 0 offen offset:1024 nt lds\n\ts_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(off), "s"(lds_address(dst)), "s"(r)
        : "memory");
  } else {
    lds_load16(r, off, dst);
  }
}

// A 4 KB run of 16 rows of 256 bytes to dst, with each lane's source offset
// in transfer c (rows 4 c .. 4 c + 3) given by voff[c]: transfer c's lane l
// still lands at dst + 1024 c + 16 l, so the caller's offsets choose which
// 16-byte piece of its row each LDS position holds (a swizzle).  One M0
// set-up; the immediate offsets step memory and LDS by 1 KB per transfer.
template <bool NT = true>
__device__ __forceinline__ void lds_copy_rows_swizzled(rsrc_t r, char* dst, const uint32_t* voff) {
  uint32_t saved;
  if constexpr (NT) {
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %5\n\ts_nop 0\n\t"
        "buffer_load_dwordx4 %1, %6, 0 offen offset:0 nt lds\n\t"
        "buffer_load_dwordx4 %2, %6, 0 offen offset:1024 nt lds\n\t"
        "buffer_load_dwordx4 %3, %6, 0 offen offset:2048 nt lds\n\t"
        "buffer_load_dwordx4 %4, %6, 0 offen offset:3072 nt lds\n\ts_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "s"(lds_address(dst)), "s"(r)
        : "memory");
  } else {
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %5\n\ts_nop 0\n\t"
        "buffer_load_dwordx4 %1, %6, 0 offen offset:0 lds\n\t"
        "buffer_load_dwordx4 %2, %6, 0 offen offset:1024 lds\n\t"
        "buffer_load_dwordx4 %3, %6, 0 offen offset:2048 lds\n\t"
        "buffer_load_dwordx4 %4, %6, 0 offen offset:3072 lds\n\ts_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "s"(lds_address(dst)), "s"(r)
        : "memory");
  }
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier that the compiler may not move LDS accesses across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---- FP8 E4M3 caches ----------------------------------------------------------

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two FP8 E4M3 codes (bytes 0-1, or 2-3 when HI, of w) as the compute format's
// packed pair.  Exact: every E4M3 value is representable in fp16 and bf16.
template <typename Fmt, bool HI>
__device__ __forceinline__ uint32_t fp8x2_to(uint32_t w) {
  const f32x2_t f = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
  return Fmt::pack(f.x, f.y);
}

// How a cache stores 8 (or 4) consecutive elements of a row and how they become
// the 16-bit compute format.  Native caches hold the compute format already.
// K rows are read 16 bytes per lane; kKSteps is the number of 8-element q.K
// operands one such read holds (1 for 16-bit caches, 2 for FP8), and split()
// hands them out.
template <typename Fmt, bool FP8>
struct KVStore {
  static constexpr int kBytes = 2;  // bytes per element
  static constexpr int kKSteps = 1;
  using Raw8 = uint4;
  using Raw4 = uint2;
  static __device__ __forceinline__ void split(uint4 w, Raw8* k) { k[0] = w; }
  static __device__ __forceinline__ uint4 to16(uint4 r) { return r; }
  static __device__ __forceinline__ uint2 to16(uint2 r) { return r; }
  template <bool STREAM>
  static __device__ __forceinline__ Raw8 load8(rsrc_t rs, uint32_t off) {
    return buffer_load<STREAM>(rs, off, (uint4*)nullptr);
  }
  template <bool STREAM>
  static __device__ __forceinline__ Raw4 load4(rsrc_t rs, uint32_t off) {
    return buffer_load<STREAM>(rs, off, (uint2*)nullptr);
  }
};

template <typename Fmt>
struct KVStore<Fmt, true> {
  static constexpr int kBytes = 1;
  static constexpr int kKSteps = 2;
  using Raw8 = uint2;
  using Raw4 = uint32_t;
  static __device__ __forceinline__ void split(uint4 w, Raw8* k) {
    k[0] = make_uint2(w.x, w.y);
    k[1] = make_uint2(w.z, w.w);
  }
  static __device__ __forceinline__ uint4 to16(uint2 r) {
    return make_uint4(fp8x2_to<Fmt, false>(r.x), fp8x2_to<Fmt, true>(r.x),
                      fp8x2_to<Fmt, false>(r.y), fp8x2_to<Fmt, true>(r.y));
  }
  static __device__ __forceinline__ uint2 to16(uint32_t r) {
    return make_uint2(fp8x2_to<Fmt, false>(r), fp8x2_to<Fmt, true>(r));
  }
  template <bool STREAM>
  static __device__ __forceinline__ Raw8 load8(rsrc_t rs, uint32_t off) {
    return buffer_load<STREAM>(rs, off, (uint2*)nullptr);
  }
  template <bool STREAM>
  static __device__ __forceinline__ Raw4 load4(rsrc_t rs, uint32_t off) {
    return buffer_load_b32(rs, off, STREAM);
  }
};

}  // namespace pa
