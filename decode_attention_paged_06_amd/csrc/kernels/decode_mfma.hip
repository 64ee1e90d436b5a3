// Paged decode attention on the gfx950 matrix cores.
//
// Operation: for one new query token per head, softmax(scale * q.K + alibi).V
// over the sequence's cached tokens, reached through its block table ("single
// query cached KV attention", vLLM PR #420; GQA head mapping of vLLM PR #452).
//
// Decomposition.  A workgroup (4 waves) owns the query heads that share one
// kv head (the GQA group, padded to HT tiles of 16 heads), for one sequence
// and one context partition.  A head tile is the N = 16 side of the MFMA
// products and each 16-token cache block is one M = 16 tile:
//
//   S^T[t, g]   = sum_d K[t, d] q[g, d]    v_mfma_f32_16x16x32_{f16,bf16}, D/32 steps
//   O^T[d, g]  += sum_t V[t, d] P[g, t]     v_mfma_f32_16x16x16_{f16,bf16}, D/16 tiles
//
// Wave w walks the partition's blocks w, w+4, w+8, ... with a two-deep
// software pipeline (the next block's K/V loads are in flight while the current
// block is processed); the four waves' softmax states are merged at the end.
// Every K/V byte is loaded once per workgroup and feeds all HT head tiles;
// groups of up to 16 heads (HT = 1) keep their q operands in registers,
// larger groups re-read them from LDS to save registers.
//
// Register layouts (lane = 16 j + r, r = lane % 16, j = lane / 16):
//   K operand, step i : lane holds K[t = r][16-byte chunk 4i + j]; the load for
//                       step i reads 64 contiguous bytes of each of the 16 rows.
//   q operand, step i : lane holds q[g = r][chunk 4i + j]   (same k order as K).
//   scores            : lane holds S^T[t = 4j + v][g = r], v = 0..3.
//   V loads i = 0..3  : lane holds V[t = 4j + i][EPL elements at r * EPL]; each
//                       load reads 4 whole rows, fully coalesced.
//   P operand         : lane holds P[g = r][t = 4j + v]: exactly its scores,
//                       rounded to the storage type -- no data movement.
//   V^T operand, tile m: lane holds V[t = 4j + i][d = EPL r + m] for i = 0..3,
//                       regrouped from the four V loads with two v_perm_b32.
//   output tile m     : lane holds O^T[d = EPL (4j + v) + m][g = r], so lane
//                       (r, j) owns the contiguous output slice
//                       d in [4 EPL j, 4 EPL (j + 1)) of head r.
// The contraction index may be any permutation as long as both operands agree,
// which is what lines these layouts up with coalesced loads and no LDS
// staging of K or V.
//
// Softmax: fp32 online softmax in log2 units; the running max of a head is
// shared by the 4 lane groups j (two swizzles per block), each lane keeps a
// partial sum of its own rounded p values, and the accumulator rescale is
// skipped when no lane's max moved.  P is rounded to the storage type before
// the P.V product (the matrix cores take 16-bit operands); the sum l uses the
// same rounded values so the normalisation matches what was accumulated.
#include "../launch.h"
#include "device_common.h"

namespace pa {

template <typename Fmt>
struct Mfma;

template <>
struct Mfma<F16> {
  static __device__ __forceinline__ f32x4_t qk(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t pv(uint2 a, uint2 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                 __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
  }
};

template <>
struct Mfma<BF16> {
  static __device__ __forceinline__ f32x4_t qk(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t pv(uint2 a, uint2 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a),
                                                     __builtin_bit_cast(i16x4_t, b), c, 0, 0, 0);
  }
};

// EPL 16-bit elements per lane per V row load: 8 (uint4) for D = 128, 4 (uint2) for D = 64.
template <int EPL>
struct VRow;
template <>
struct VRow<8> {
  using T = uint4;
  static __device__ __forceinline__ uint32_t word(const T& v, int w) {
    return w == 0 ? v.x : w == 1 ? v.y : w == 2 ? v.z : v.w;
  }
  static __device__ __forceinline__ T zero() { return make_uint4(0, 0, 0, 0); }
};
template <>
struct VRow<4> {
  using T = uint2;
  static __device__ __forceinline__ uint32_t word(const T& v, int w) { return w == 0 ? v.x : v.y; }
  static __device__ __forceinline__ T zero() { return make_uint2(0, 0); }
};

template <typename Fmt, int D, int HT>
__global__ __launch_bounds__(kWaves * 64) void decode_mfma_kernel(const DecodeArgs a) {
  constexpr int BS = kBlockSize;
  static_assert(BS == 16, "one cache block is one M = 16 MFMA tile");
  constexpr int CH = D / 8;     // 16-byte chunks per row
  constexpr int NK = D / 32;    // q.K MFMA steps
  constexpr int EPL = D / 16;   // V elements per lane per row load = number of P.V tiles
  using VR = VRow<EPL>;
  using VT = typename VR::T;
  constexpr float kLog2e = 1.4426950408889634f;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int r = lane & 15;
  const int j = lane >> 4;

  const int kvh = blockIdx.x;
  const int seq = blockIdx.y;
  const int part = blockIdx.z;
  const int G = a.group;
  const int h0 = kvh * G;
  const bool single = a.num_partitions == 1;

  const int L = min(a.context_lens[seq], a.max_blocks_per_seq * BS);
  const int tok0 = part * a.partition_blocks * BS;
  if (L <= 0) {
    if (single) {
      uint4* o = reinterpret_cast<uint4*>(a.out) + ((size_t)seq * a.num_heads + h0) * CH;
      for (int i = threadIdx.x; i < G * CH; i += kWaves * 64) o[i] = make_uint4(0, 0, 0, 0);
    }
    return;
  }
  if (tok0 >= L) return;  // partition past this sequence's end: nothing to do
  const int tok1 = min(L, tok0 + a.partition_blocks * BS);
  const int blk0 = tok0 / BS;
  const int nblk = (tok1 - tok0 + BS - 1) / BS;

  // ---- shared query load: the group's G rows, zero-padded to HT * 16 ------
  __shared__ uint4 q_lds[HT * 16 * CH];
  {
    const uint4* qg = reinterpret_cast<const uint4*>(a.q) + ((size_t)seq * a.num_heads + h0) * CH;
    for (int i = threadIdx.x; i < HT * 16 * CH; i += kWaves * 64)
      q_lds[i] = (i < G * CH) ? qg[i] : make_uint4(0, 0, 0, 0);
  }
  __syncthreads();
  constexpr bool kQInRegs = HT == 1;
  uint4 qb[kQInRegs ? NK : 1];
  if constexpr (kQInRegs) {
#pragma unroll
    for (int i = 0; i < NK; ++i) qb[i] = q_lds[r * CH + 4 * i + j];
  }
  float slope[HT];
#pragma unroll
  for (int n = 0; n < HT; ++n) {
    const int g = n * 16 + r;
    slope[n] = (a.alibi != nullptr && g < G) ? a.alibi[h0 + g] * kLog2e : 0.f;
  }

  float m[HT], lsum[HT];
  f32x4_t acc[HT][EPL];
#pragma unroll
  for (int n = 0; n < HT; ++n) {
    m[n] = kNegBig;
    lsum[n] = 0.f;
#pragma unroll
    for (int t = 0; t < EPL; ++t) acc[n][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  const int* table = a.block_tables + (size_t)seq * a.max_blocks_per_seq + blk0;
  // Byte addressing: a wave-uniform block base (SGPRs) plus a small unsigned
  // per-lane offset, so every K/V load is one buffer load with a VGPR offset.
  const size_t bstride = (size_t)a.num_kv_heads * BS * D * 2;  // bytes per physical block
  const size_t head_off = (size_t)kvh * BS * D * 2;
  const char* kbase = reinterpret_cast<const char*>(a.k_cache) + head_off;
  const char* vbase = reinterpret_cast<const char*>(a.v_cache) + head_off;
  const uint32_t k_lane = (uint32_t)(r * D + j * 8) * 2u;          // step-0 K chunk
  const uint32_t v_lane = (uint32_t)((4 * j) * D + r * EPL) * 2u;  // load-0 V slice
  const int qpos = L - 1;

  // One cache block's K and V in registers.
  struct Tile {
    uint4 k[NK];
    VT v[4];
  };
  auto load = [&](Tile& T, int b) {
    const size_t boff = (size_t)table[b] * bstride;
    const rsrc_t rk = make_rsrc(kbase + boff, BS * D * 2);
    const rsrc_t rv = make_rsrc(vbase + boff, BS * D * 2);
#pragma unroll
    for (int i = 0; i < NK; ++i) T.k[i] = buffer_load(rk, k_lane + 64u * i, (uint4*)nullptr);
#pragma unroll
    for (int i = 0; i < 4; ++i) T.v[i] = buffer_load(rv, v_lane + 2u * D * i, (VT*)nullptr);
  };

  auto process = [&](Tile& T, int b) {
    const int tb = (blk0 + b) * BS;
    const int valid = tok1 - tb;
    uint2 pk[HT];
    float alpha[HT];
    bool rescale = false;

#pragma unroll
    for (int n = 0; n < HT; ++n) {
      f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        uint4 qv;
        if constexpr (kQInRegs) qv = qb[i];
        else qv = q_lds[(n * 16 + r) * CH + 4 * i + j];
        s = Mfma<Fmt>::qk(T.k[i], qv, s);
      }
      float x[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = 4 * j + v;
        const float z = fmaf(s[v], a.scale_log2, slope[n] * (float)(tb + t - qpos));
        x[v] = t < valid ? z : kNegBig;
      }
      float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      mx = fmaxf(mx, shfl_xor(mx, 16));
      mx = fmaxf(mx, shfl_xor(mx, 32));
      const float mn = fmaxf(m[n], mx);
      alpha[n] = fast_exp2(m[n] - mn);
      rescale |= alpha[n] != 1.f;
      m[n] = mn;
      const uint32_t p01 = Fmt::pack(fast_exp2(x[0] - mn), fast_exp2(x[1] - mn));
      const uint32_t p23 = Fmt::pack(fast_exp2(x[2] - mn), fast_exp2(x[3] - mn));
      pk[n] = make_uint2(p01, p23);
      lsum[n] = fmaf(lsum[n], alpha[n],
                     (Fmt::lo(p01) + Fmt::hi(p01)) + (Fmt::lo(p23) + Fmt::hi(p23)));
    }
    if (wave_any(rescale)) {
#pragma unroll
      for (int n = 0; n < HT; ++n) {
#pragma unroll
        for (int t = 0; t < EPL; ++t) acc[n][t] *= alpha[n];
      }
    }

    if (valid < BS) {  // last block of a sequence: slots past L may hold NaN
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * j + i >= valid) T.v[i] = VR::zero();
    }

#pragma unroll
    for (int t = 0; t < EPL; ++t) {
      const int w = t >> 1;
      const uint32_t a0 = VR::word(T.v[0], w), a1 = VR::word(T.v[1], w);
      const uint32_t a2 = VR::word(T.v[2], w), a3 = VR::word(T.v[3], w);
      const uint2 vt = (t & 1) ? make_uint2(pack_hi_hi(a0, a1), pack_hi_hi(a2, a3))
                               : make_uint2(pack_lo_lo(a0, a1), pack_lo_lo(a2, a3));
#pragma unroll
      for (int n = 0; n < HT; ++n) acc[n][t] = Mfma<Fmt>::pv(vt, pk[n], acc[n][t]);
    }
  };

  // Software pipeline: the loads of the wave's next block are in flight while
  // the current block is processed (two register tiles, used alternately).
  Tile ta, tb2;
  int b = wave;
  if (b < nblk) load(ta, b);
  while (b < nblk) {
    const int b1 = b + kWaves;
    if (b1 < nblk) load(tb2, b1);
    process(ta, b);
    if (b1 >= nblk) break;
    const int b2 = b1 + kWaves;
    if (b2 < nblk) load(ta, b2);
    process(tb2, b1);
    b = b2;
  }

  // ---- complete the per-lane sums over the 4 lane groups -------------------
#pragma unroll
  for (int n = 0; n < HT; ++n) {
    lsum[n] += shfl_xor(lsum[n], 16);
    lsum[n] += shfl_xor(lsum[n], 32);
  }

  // ---- merge the waves into wave 0 (fixed order: deterministic) ------------
  __shared__ f32x4_t mrg_acc[HT][EPL][64];
  __shared__ float mrg_m[HT][64];
  __shared__ float mrg_l[HT][64];
  for (int w = 1; w < kWaves; ++w) {
    __syncthreads();
    if (wave == w) {
#pragma unroll
      for (int n = 0; n < HT; ++n) {
        mrg_m[n][lane] = m[n];
        mrg_l[n][lane] = lsum[n];
#pragma unroll
        for (int t = 0; t < EPL; ++t) mrg_acc[n][t][lane] = acc[n][t];
      }
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int n = 0; n < HT; ++n) {
        const float mo = mrg_m[n][lane];
        const float mn = fmaxf(m[n], mo);
        const float f = fast_exp2(m[n] - mn);
        const float fo = fast_exp2(mo - mn);
        lsum[n] = lsum[n] * f + mrg_l[n][lane] * fo;
#pragma unroll
        for (int t = 0; t < EPL; ++t) acc[n][t] = acc[n][t] * f + mrg_acc[n][t][lane] * fo;
        m[n] = mn;
      }
    }
  }

  // ---- finalise ---------------------------------------------------------------
  if (wave != 0) return;
#pragma unroll
  for (int n = 0; n < HT; ++n) {
    const int g = n * 16 + r;
    if (g >= G) continue;
    const float inv = lsum[n] > 0.f ? 1.f / lsum[n] : 0.f;
    const size_t row = (size_t)seq * a.num_heads + h0 + g;
    if (single) {
      uint16_t* orow = reinterpret_cast<uint16_t*>(a.out) + row * D;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        uint32_t wv[EPL / 2];
#pragma unroll
        for (int t = 0; t < EPL; t += 2)
          wv[t / 2] = Fmt::pack(acc[n][t][v] * inv, acc[n][t + 1][v] * inv);
        VT o;
        if constexpr (EPL == 8) o = make_uint4(wv[0], wv[1], wv[2], wv[3]);
        else o = make_uint2(wv[0], wv[1]);
        *reinterpret_cast<VT*>(orow + EPL * (4 * j + v)) = o;
      }
    } else {
      const size_t slot = row * a.num_partitions + part;
      float* orow = a.ws_o + slot * D;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
#pragma unroll
        for (int t = 0; t < EPL; t += 4)
          *reinterpret_cast<float4*>(orow + EPL * (4 * j + v) + t) =
              make_float4(acc[n][t][v] * inv, acc[n][t + 1][v] * inv, acc[n][t + 2][v] * inv,
                          acc[n][t + 3][v] * inv);
      }
      if (j == 0) reinterpret_cast<float2*>(a.ws_ml)[slot] = make_float2(m[n], lsum[n]);
    }
  }
}

namespace {

template <typename Fmt, int D, int HT>
hipError_t launch_t(const DecodeArgs& a, hipStream_t s) {
  dim3 grid(a.num_kv_heads, a.num_seqs, a.num_partitions);
  decode_mfma_kernel<Fmt, D, HT><<<grid, kWaves * 64, 0, s>>>(a);
  return hipGetLastError();
}

template <typename Fmt, int D>
hipError_t launch_g(const DecodeArgs& a, hipStream_t s) {
  switch ((a.group + 15) / 16) {
    case 1: return launch_t<Fmt, D, 1>(a, s);
    case 2: return launch_t<Fmt, D, 2>(a, s);
    case 3: return launch_t<Fmt, D, 3>(a, s);
    default: return launch_t<Fmt, D, 4>(a, s);
  }
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeArgs& a, int dtype, int head_size, hipStream_t s) {
  if (dtype == 0) return head_size == 64 ? launch_g<F16, 64>(a, s) : launch_g<F16, 128>(a, s);
  return head_size == 64 ? launch_g<BF16, 64>(a, s) : launch_g<BF16, 128>(a, s);
}

}  // namespace pa
