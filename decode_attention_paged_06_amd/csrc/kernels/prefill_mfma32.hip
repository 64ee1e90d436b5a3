// Causal multi-query (prefill) attention over the paged cache on the gfx950
// 32 x 32 matrix tiles.
//
// Operation (the multi-query call of the C ABI): new token i of sequence s,
// at position p = L - n + i, attends to cached positions 0 .. p:
//   out[row, h] = softmax_t(scale q[row, h].K[t] + alibi_h (t - p)) . V[t]
// over the K/V of its kv head, reached through the block table.
//
// Decomposition.  A workgroup of 4 waves owns 128 query rows of one
// (sequence, kv head) -- row i G + g is new token i, query head g of the
// group -- and walks the keys they see in steps of 32 (two 16-row cache
// tiles), staged once per step through an LDS ring of three slots that all
// four waves fill (a quarter each) and read.  Wave w owns rows 32 w ..
// 32 w + 31 and computes, per step,
//   S^T[key, row]  = sum_d K[key, d] Q[row, d]     8 x v_mfma_f32_32x32x16 (D / 16)
//   O^T[d, row]   += sum_key V[key, d] P[row, key]  8 x v_mfma_f32_32x32x16 (4 d-blocks x 2)
// Register layouts (lane = 32 jj + n):
//   Q operand, k-step s : Q[row n][dims 16 s + 8 jj .. + 7]   (in registers all along)
//   K operand, k-step s : K[key n][dims 16 s + 8 jj .. + 7]   (from LDS)
//   S^T, register r     : key 8 (r / 4) + 4 jj + r % 4, row n -- so a lane holds
//                         16 keys of one row (half of them; lane n + 32 has
//                         the rest), and its maximum is a tree of in-lane
//                         three-input maxima
//   P operand, half h   : the lane's S registers 8 h .. 8 h + 7 as weights, i.e.
//                         keys 16 h + 8 e' + 4 jj + v (e' = 0, 1; v = 0..3)
//   V^T operand, block b, half h : V[those keys][dims 32 b + n], taken with two
//                         LDS transpose reads (keys 4 at a time)
//   O^T block b, reg r  : dims 32 b + 8 (r / 4) + 4 jj + r % 4 of row n
// The contraction order of each product is a permutation shared by both
// operands, which is what lets S feed P.V without any data movement.
//
// LDS: a step's 32 key rows of K (8 KB) then of V (8 KB), 256 bytes per row,
// each row's 16-byte pieces XOR-swizzled (K: by row % 16; V: by 5 (row % 4),
// i.e. 0, 5, 10, 15) so that the lanes one LDS cycle serves -- 128 or 256
// bytes' worth -- of a K read (rows n, pieces 2 s + jj) or of a V transpose
// read (4 rows, 4 pieces) never share a bank.  The swizzle is
// applied by the buffer-to-LDS copies themselves: each lane fetches the
// piece that belongs at its fixed LDS position.
//
// Softmax: fp32 online softmax in log2 units against a per-row reference max
// that moves only when a step's max exceeds it by more than 8 (weights stay
// below 2^8, the rescale is rare; each lane tests its own half of the row,
// and the two halves are combined only on a step that moves the max); P is
// rounded to the 16-bit type for the matrix product and l sums the same
// rounded weights.  Built for 16-bit
// caches, head size 128 and cache blocks of at least 16 tokens; other
// multi-query calls run on the general kernel.
#include <type_traits>

#include "../launch.h"
#include "device_common.h"

namespace pa {

namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <typename Fmt>
struct Mfma32;
template <>
struct Mfma32<F16> {
  static __device__ __forceinline__ f32x16_t mma(uint4 a, uint4 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
};
template <>
struct Mfma32<BF16> {
  static __device__ __forceinline__ f32x16_t mma(uint4 a, uint4 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};

constexpr int kD = 128;                        // head size
constexpr int kW = 4;                          // waves per workgroup
constexpr int kRows = 32 * kW;                 // query rows per workgroup
static_assert(kRows == kPrefillRows, "the host sizes the row chunks with kPrefillRows");
constexpr int kKeys = 32;                      // keys per step
constexpr int kRowBytes = kD * 2;              // 256
constexpr int kKBytes = kKeys * kRowBytes;     // 8 KB of K per step
constexpr int kSlotBytes = 2 * kKBytes;        // K then V
constexpr int kSlots = 3;                      // ring slots
constexpr int kRingBytes = kSlots * kSlotBytes;
constexpr int kQBytes = kRows * kRowBytes;     // 32 KB: the query rows, before the ring
constexpr int kLdsBytes = kRingBytes > kQBytes ? kRingBytes : kQBytes;
constexpr int kWindow = 512;                   // tile source offsets kept in LDS
constexpr int kTransfersPerWave = 4;           // 1 KB copies per wave per step (a quarter)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.f;

// 16 rows of 256 bytes to dst (rows 4 c .. 4 c + 3 by transfer c) where lane
// l of transfer c fetches the source bytes at voff[c] (+ 1 KB c) for LDS
// position dst + 1 KB c + 16 l.
__device__ __forceinline__ void copy_tile(rsrc_t r, char* dst, const uint32_t* voff) {
  lds_copy_rows_swizzled<false>(r, dst, voff);
}

}  // namespace

template <typename Fmt>
__global__ __launch_bounds__(kW * 64) void prefill_mfma32_kernel(const DecodeArgs a) {
  __shared__ __align__(16) char lds[kLdsBytes];
  __shared__ uint64_t toff[kWindow];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31;   // row (of the wave's 32) and key row of the K operand
  const int jj = lane >> 5;  // lane half

  // ---- the unit: rows row_base .. + 127 of (sequence, kv head), a partition --
  const int chunks = a.row_chunks;
  const int xi = blockIdx.x, seq = blockIdx.y, part = blockIdx.z;
  const int kvh = xi % a.num_kv_heads;
  const int rc = chunks - 1 - xi / a.num_kv_heads;  // later rows (more keys) start first
  const int G = a.group;
  const int h0 = kvh * G;
  const bool single = a.num_partitions == 1;
  const int q_first = a.query_start[seq];
  const int n_new = a.query_start[seq + 1] - q_first;
  const int row_base = rc * kRows;
  const int nrows = n_new * G;
  if (row_base >= nrows) return;
  const int BS = a.block_size;
  const int tpb_shift = a.block_shift - 4;  // log2(16-row tiles per block)
  const int* table = a.block_tables + (size_t)seq * a.max_blocks_per_seq;
  const int L = min(__builtin_amdgcn_readfirstlane(a.context_lens[seq]), a.max_blocks_per_seq * BS);

  // ---- the query rows to LDS (swizzled like K), then to registers ----------
  for (int idx = threadIdx.x; idx < kRows * 16; idx += kW * 64) {
    const int rr = idx >> 4, piece = idx & 15;
    const int row = row_base + rr;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row < nrows) {
      const int ti = row / G;
      v = reinterpret_cast<const uint4*>(a.q)[((size_t)(q_first + ti) * a.num_heads + h0 + row - ti * G) *
                                                  16 + piece];
    }
    *reinterpret_cast<uint4*>(lds + rr * kRowBytes + ((piece ^ (rr & 15)) << 4)) = v;
  }
  __syncthreads();
  if (L <= 0) {  // no context: zero rows (a single pass writes them)
    if (single) {
      for (int idx = threadIdx.x; idx < kRows * 16; idx += kW * 64) {
        const int row = row_base + (idx >> 4);
        if (row < nrows) {
          const int ti = row / G;
          reinterpret_cast<uint4*>(a.out)[((size_t)(q_first + ti) * a.num_heads + h0 + row - ti * G) * 16 +
                                          (idx & 15)] = make_uint4(0, 0, 0, 0);
        }
      }
    }
    return;
  }
  // the workgroup's rows see keys up to its last new token's position
  const int last_new = min(n_new, (row_base + kRows + G - 1) / G) - 1;
  const int kend = L - n_new + last_new + 1;
  const int tok0 = part * a.partition_blocks * BS;
  if (tok0 >= kend) return;
  const int tok1 = __builtin_amdgcn_readfirstlane(min(kend, tok0 + a.partition_blocks * BS));
  const int nsteps = (tok1 - tok0 + kKeys - 1) / kKeys;
  const int ntiles = (tok1 - tok0 + 15) >> 4;  // 16-row tiles holding the partition's keys
  const int tile0 = tok0 >> 4;

  // this lane's row
  const int wrow0 = row_base + 32 * wave;  // the wave's first row
  const int row = wrow0 + n;
  const bool row_ok = row < nrows;
  const int ti = row / G;
  const int g = row - ti * G;
  const int pos = L - n_new + ti;  // keys 0 .. pos visible (padding rows: past L, never stored)
  const int pos_lo = L - n_new + wrow0 / G;                       // the wave's lowest position
  const int pos_hi = L - n_new + min(wrow0 + 31, nrows - 1) / G;  // and highest
  const bool has_alibi = a.alibi != nullptr;
  const float slope = (has_alibi && row_ok) ? a.alibi[h0 + g] * kLog2e : 0.f;
  uint4 qb[8];
#pragma unroll
  for (int s = 0; s < 8; ++s)
    qb[s] = *reinterpret_cast<const uint4*>(lds + (32 * wave + n) * kRowBytes +
                                            (((2 * s + jj) ^ (n & 15)) << 4));

  // LDS read offsets within a slot: K operand of k-step s; V transpose reads of
  // d-block b (key halves and sub-blocks are immediate offsets)
  uint32_t k_ofs[8], v_ofs[4];
#pragma unroll
  for (int s = 0; s < 8; ++s) k_ofs[s] = n * kRowBytes + (((2 * s + jj) ^ (n & 15)) << 4);
  {
    const int grp = lane >> 4, c = lane & 15, k = c >> 2, q = c & 3;
    const int vrow = 4 * (grp >> 1) + k;
#pragma unroll
    for (int b = 0; b < 4; ++b)
      v_ofs[b] = kKBytes + vrow * kRowBytes + (((4 * b + 2 * (grp & 1) + (q >> 1)) ^ (5 * k)) << 4) +
                 (q & 1) * 8;
  }
  // source offsets of the swizzled copies (transfer c = rows 4 c .. 4 c + 3)
  uint32_t k_src[4], v_src[4];
  {
    const int rr = lane >> 4, piece = lane & 15;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      k_src[c] = rr * kRowBytes + ((piece ^ (4 * c + rr)) << 4);
      v_src[c] = rr * kRowBytes + ((piece ^ (5 * rr)) << 4);
    }
  }

  const size_t head_off = (size_t)kvh * (size_t)a.kv_head_stride;
  const char* kbase = reinterpret_cast<const char*>(a.k_cache) + head_off;
  const char* vbase = reinterpret_cast<const char*>(a.v_cache) + head_off;

  // Source offsets of the partition's 16-row tiles (block-table entry times
  // the block stride, plus the tile's place in its block), kWindow tiles at a
  // time: the lookup and the 64-bit product are done here once per tile, by
  // all lanes, and a step's copy only adds its base.  Entries past the last
  // tile repeat it (their copies read nothing).
  const uint64_t bstride = (uint64_t)a.kv_block_stride;
  const int tpb_mask = (1 << tpb_shift) - 1;
  auto fill_window = [&](int start) {
    for (int i = threadIdx.x; i < kWindow; i += kW * 64) {
      const int ua = tile0 + min(start + i, ntiles - 1);
      toff[i] = (uint64_t)(uint32_t)table[ua >> tpb_shift] * bstride + (uint32_t)((ua & tpb_mask) << 12);
    }
  };
  // the window starts at tile win0; the first step whose second tile lies
  // past it refills it (never, once the window reaches the last tile)
  int win0 = 0;
  auto refill_step = [&](int w0) { return ntiles - 1 - w0 < kWindow ? 0x7fffffff : (w0 + kWindow) / 2; };
  int refill_at = refill_step(0);
  __syncthreads();  // every wave has its query rows: the LDS becomes the ring
  fill_window(0);
  __syncthreads();

  // Every wave copies a quarter of each step: wave w the K (w even) or V (w
  // odd) rows of the step's tile w / 2 -- four 1 KB transfers -- so the copy
  // work and its scalar address arithmetic are shared evenly.  Tiles past the
  // partition read nothing (zeros).
  const int my_kt = wave >> 1;
  const bool my_v = (wave & 1) != 0;
  const char* my_base = my_v ? vbase : kbase;
  // (tiles at or after win0: the index is never negative)
  auto window_off = [&](int j) { return toff[min(min(2 * j + my_kt, ntiles - 1) - win0, kWindow - 1)]; };
  auto copy = [&](int j, int slot, uint64_t off) {
    const int u = 2 * j + my_kt;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)off);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(off >> 32));
    const uint32_t bytes = u < ntiles ? (uint32_t)min(tok1 - (tile0 + u) * 16, 16) * kRowBytes : 0u;
    char* dst = lds + slot * kSlotBytes + (my_v ? kKBytes : 0) + my_kt * 16 * kRowBytes;
    copy_tile(make_rsrc(my_base + (((uint64_t)hi << 32) | lo), bytes), dst, my_v ? v_src : k_src);
  };

  float m = kNegBig, lsum = 0.f;
  f32x16_t acc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[b][r] = 0.f;

  // scores S^T of a step: 16 keys of row n per lane
  auto scores = [&](const char* slot) {
    f32x16_t sc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      sc = Mfma32<Fmt>::mma(*reinterpret_cast<const uint4*>(slot + k_ofs[s]), qb[s], sc);
    return sc;
  };
  auto process = [&](const char* slot, int kb, f32x16_t sc) {
    // logits in log2 units, in place (or, for a step every row sees in full
    // and no ALiBi, the raw scores with the positive scale applied in the
    // exponent: xs)
    float xs = 1.f;
    const bool full = kb + kKeys <= tok1 && kb + kKeys - 1 <= pos_lo;
    if (full && !has_alibi && a.scale_log2 > 0.f) {
      xs = a.scale_log2;
    } else {
      const float base = slope * (float)(kb + 4 * jj - pos);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r >> 2) + (r & 3);  // + 4 jj
        sc[r] = fmaf(sc[r], a.scale_log2, fmaf((float)key, slope, base));
      }
      if (!full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int t = kb + 8 * (r >> 2) + (r & 3) + 4 * jj;
          sc[r] = (t < tok1 && t <= pos) ? sc[r] : kNegBig;
        }
      }
    }
    // row max of the lane's 16 keys: a tree of three-input maxima (depth 3)
    const float t0 = score_max3(sc[0], sc[1], sc[2]), t1 = score_max3(sc[3], sc[4], sc[5]);
    const float t2 = score_max3(sc[6], sc[7], sc[8]), t3 = score_max3(sc[9], sc[10], sc[11]);
    const float t4 = score_max3(sc[12], sc[13], sc[14]);
    // (this lane's half of the row: the other half, lane n + 32, is consulted
    // only by a step that moves m, so both halves move it alike)
    const float local = xs * score_max(score_max3(t0, t1, t2), score_max3(t3, t4, sc[15]));
    if (wave_any(local > m + kRescaleSlack)) {
      const float mn = score_max(m, xor32_pair_max(local));
      const float alpha = fast_exp2(m - mn);
      m = mn;
      lsum *= alpha;
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[b] *= alpha;
    }
    const float nm = -m;
    uint32_t pw[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      pw[q] = Fmt::pack(fast_exp2(fmaf(sc[2 * q], xs, nm)), fast_exp2(fmaf(sc[2 * q + 1], xs, nm)));
      lsum = Fmt::dot2(pw[q], Fmt::kOnes, lsum);  // l sums the rounded weights P.V uses
    }
    // P.V over the two key halves
    typedef short v4s_t __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4s_t lds_v4s_t;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint4 pb = make_uint4(pw[4 * h], pw[4 * h + 1], pw[4 * h + 2], pw[4 * h + 3]);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const char* p = slot + v_ofs[b] + h * 16 * kRowBytes;
        const v4s_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)(lds_void_t*)p);
        const v4s_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)(lds_void_t*)(p + 8 * kRowBytes));
        const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
        acc[b] = Mfma32<Fmt>::mma(make_uint4(l2.x, l2.y, h2.x, h2.y), pb, acc[b]);
      }
    }
  };

  // ---- the staged loop: slot j % kSlots holds step j ------------------------
#pragma unroll
  for (int k = 0; k + 1 < kSlots; ++k) copy(k, k, window_off(k));
  uint64_t off_next = window_off(kSlots - 1);
  // One step; the ring slot is a compile-time constant (the loop below is
  // unrolled by the ring size), so every LDS operand address is a lane offset
  // plus an immediate.
  auto step = [&](int j, auto slot_tag) {
    constexpr int kSlot = decltype(slot_tag)::value;
    wait_vmcnt<kTransfersPerWave * (kSlots - 2)>();  // this wave's part of step j has landed
    const int jc = j + kSlots - 1;  // the step copied now
    const bool refill = jc >= refill_at;  // same for every wave
    if (refill) {
      lds_barrier();  // every wave is done with the old window
      win0 = 2 * jc;
      refill_at = refill_step(win0);
      fill_window(win0);
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    }
    lds_barrier();  // step j is visible to every wave; slot (j - 1) % kSlots is free
    const int kb = tok0 + j * kKeys;
    // (wave-uniform: a wave whose rows are all padding, or sit before every key
    // of the step, has nothing to add)
    const bool work = wrow0 < nrows && kb <= pos_hi;
    // the scores' matrix products are issued before the copy, whose scalar
    // address arithmetic then overlaps them
    f32x16_t sc;
    if (work) sc = scores(lds + kSlot * kSlotBytes);
    copy(jc, (kSlot + kSlots - 1) % kSlots, refill ? window_off(jc) : off_next);
    off_next = window_off(jc + 1);
    if (work) process(lds + kSlot * kSlotBytes, kb, sc);
  };
  static_assert(kSlots == 3, "the loop is unrolled by the ring size");
  for (int j = 0; j < nsteps; j += kSlots) {
    step(j, std::integral_constant<int, 0>{});
    if (j + 1 < nsteps) step(j + 1, std::integral_constant<int, 1>{});
    if (j + 2 < nsteps) step(j + 2, std::integral_constant<int, 2>{});
  }
  wait_vmcnt<0>();  // copies past the end have landed before the workgroup ends

  // ---- finalise ---------------------------------------------------------------
  // l: this lane's keys plus its partner lane's (n, 1 - jj)
  {
    const auto s2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
    lsum = __uint_as_float(s2[0]) + __uint_as_float(s2[1]);
  }
  if (!row_ok) return;
  const float inv = lsum > 0.f ? a.v_scale / lsum : 0.f;
  const size_t orow_idx = (size_t)(q_first + ti) * a.num_heads + h0 + g;
  if (single || (part == 0 && pos < a.partition_blocks * BS)) {
    uint16_t* orow = reinterpret_cast<uint16_t*>(a.out) + orow_idx * kD;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<uint2*>(orow + 32 * b + 8 * i + 4 * jj) =
            make_uint2(Fmt::pack(acc[b][4 * i] * inv, acc[b][4 * i + 1] * inv),
                       Fmt::pack(acc[b][4 * i + 2] * inv, acc[b][4 * i + 3] * inv));
  } else {
    const size_t slot = orow_idx * a.num_partitions + part;
    float* orow = a.ws_o + slot * kD;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<float4*>(orow + 32 * b + 8 * i + 4 * jj) =
            make_float4(acc[b][4 * i] * inv, acc[b][4 * i + 1] * inv, acc[b][4 * i + 2] * inv,
                        acc[b][4 * i + 3] * inv);
    if (jj == 0) reinterpret_cast<float2*>(a.ws_ml)[slot] = make_float2(m, lsum);
  }
}

bool prefill_mfma32_supported(int head_size, bool kv_fp8, int block_size) {
  return head_size == kD && !kv_fp8 && block_size >= 16;
}

hipError_t launch_prefill_mfma32(const DecodeArgs& a, int dtype, hipStream_t s) {
  const dim3 grid(a.num_kv_heads * a.row_chunks, a.num_seqs, a.num_partitions);
  if (dtype == 0) prefill_mfma32_kernel<F16><<<grid, kW * 64, 0, s>>>(a);
  else prefill_mfma32_kernel<BF16><<<grid, kW * 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace pa
