// Paged decode attention on the vector ALUs of gfx950.
//
// Operation: for one new query token per head, softmax(scale * q.K + alibi).V
// over the sequence's cached tokens, reached through its block table ("single
// query cached KV attention", vLLM PR #420; GQA head mapping of vLLM PR #452).
//
// Work decomposition
//   workgroup = (kv head, query-head chunk of GT heads, sequence, partition),
//   4 waves.  Wave w takes the partition's 16-row tiles w, w+4, w+8, ...
//   The GT query heads that share the kv head are loaded once into LDS by the
//   whole workgroup and every lane keeps its 16-byte slice in registers (the
//   shared query load of vLLM PR #420, done per kv head so each K/V row read
//   serves all GT heads).
//
// Lane layout inside a wave (D = head size)
//   TPT = D/8 lanes cover one token row (16 bytes each), TPL = 64/TPT token
//   rows per wave-wide 16-byte load, 16/TPL loads per 16-row tile of a cache
//   block.  One load of K (or V) is fully coalesced: TPL consecutive rows of
//   the contiguous [block_size, D] block tile.
//   q.k: each lane takes 4 packed dot2 products over its 8 elements, then a
//   DPP row reduction (mirror / half-mirror / quad swaps) gives every lane of
//   the row the full dot product -- no LDS, no wave-wide barrier.
//   Every lane row keeps its own online-softmax state (running max m, sum l,
//   fp32 accumulator of its 8 output elements per head), so no cross-row
//   traffic happens inside the block loop.  Rows, then waves, are merged once
//   at the end with the exact rescaling identity of the split softmax.
#include "../launch.h"
#include "device_common.h"

namespace pa {

template <typename Fmt, int D, int GT, bool KV8>
__global__ __launch_bounds__(kWaves * 64) void decode_valu_kernel(const DecodeArgs a) {
  // Cache blocks are walked as tiles of TT = min(16, BS) rows (see decode_mfma.hip).
  const int BS = a.block_size;
  const int TT = BS < 16 ? BS : 16;
  const int tpb_shift = a.block_shift > 4 ? a.block_shift - 4 : 0;
  constexpr int CH = D / 8;        // 16-byte chunks per token row
  constexpr int TPT = CH;          // lanes per token row
  constexpr int TPL = 64 / TPT;    // token rows per wave-wide load
  constexpr int NLOAD = 16 / TPL;  // loads per 16-row tile for K, and for V
  static_assert(64 % TPT == 0, "rows must tile the wave");
  constexpr float kLog2e = 1.4426950408889634f;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int rho = lane / TPT;   // token row of this lane within a load
  const int c = lane % TPT;     // 16-byte chunk of the row

  const int nhc = (a.group + GT - 1) / GT;
  const int kvh = blockIdx.x / nhc;
  const int hc = blockIdx.x - kvh * nhc;
  const int seq = blockIdx.y;
  const int part = blockIdx.z;
  const int h0 = kvh * a.group + hc * GT;
  const int nh = min(GT, a.group - hc * GT);
  const bool single = a.num_partitions == 1;

  const int tok0 = part * a.partition_blocks * BS;
  const int tile0 = tok0 / TT;  // first tile of the partition
  const int* table = a.block_tables + (size_t)seq * a.max_blocks_per_seq;

  // The context length, the block ids of this wave's first two tiles (their
  // table positions do not depend on the context length; clamped to the
  // table row) and the query are requested together, so their latencies
  // overlap instead of adding up.
  const int ctx_len = a.context_lens[seq];
  const int blk_first = table[min((tile0 + wave) >> tpb_shift, a.max_blocks_per_seq - 1)];
  const int blk_second = table[min((tile0 + wave + kWaves) >> tpb_shift, a.max_blocks_per_seq - 1)];

  // ---- shared query load --------------------------------------------------
  __shared__ uint4 q_lds[GT * CH];
  {
    const uint4* qg = reinterpret_cast<const uint4*>(a.q) + ((size_t)seq * a.num_heads + h0) * CH;
    for (int i = threadIdx.x; i < GT * CH; i += kWaves * 64)
      q_lds[i] = (i < nh * CH) ? qg[i] : make_uint4(0, 0, 0, 0);
  }
  __syncthreads();

  const int L = min(ctx_len, a.max_blocks_per_seq * BS);
  if (L <= 0) {
    if (single) {
      uint4* o = reinterpret_cast<uint4*>(a.out) + ((size_t)seq * a.num_heads + h0) * CH;
      for (int i = threadIdx.x; i < nh * CH; i += kWaves * 64) o[i] = make_uint4(0, 0, 0, 0);
    }
    return;
  }
  if (tok0 >= L) return;  // partition past this sequence's end: nothing to do
  const int tok1 = min(L, tok0 + a.partition_blocks * BS);
  const int ntiles = (tok1 - tok0 + TT - 1) / TT;
  uint32_t qv[GT][4];
  float slope[GT];
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    const uint4 t = q_lds[g * CH + c];
    qv[g][0] = t.x; qv[g][1] = t.y; qv[g][2] = t.z; qv[g][3] = t.w;
    slope[g] = (a.alibi != nullptr && g < nh) ? a.alibi[h0 + g] * kLog2e : 0.f;
  }

  float m[GT], l[GT], acc[GT][8];
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    m[g] = kNegBig;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
  }

  // ---- block walk -----------------------------------------------------------
  using KS = KVStore<Fmt, KV8>;  // cache storage: 16-bit, or FP8 converted at use
  constexpr int ES = KS::kBytes;
  const size_t bstride = (size_t)a.kv_block_stride;  // bytes per physical block
  const size_t head_off = (size_t)kvh * (size_t)a.kv_head_stride;
  const char* kbase = reinterpret_cast<const char*>(a.k_cache) + head_off;
  const char* vbase = reinterpret_cast<const char*>(a.v_cache) + head_off;
  const uint32_t lane_off = (uint32_t)(rho * D + c * 8) * ES;
  const int qpos = L - 1;  // position of the query token

  // One 16-row tile's K and V as stored.  The buffer bound is the tile's valid
  // rows: rows past the context end (which may hold anything, NaN included)
  // read back as zeros, and a tile past the partition end reads nothing, so
  // every pipeline step issues the same loads and the wait counts stay exact.
  struct VTile {
    typename KS::Raw8 k[NLOAD], v[NLOAD];
  };
  auto block_of = [&](int u) {  // table entry of tile u (clamped to the partition)
    return table[(tile0 + min(u, ntiles - 1)) >> tpb_shift];
  };
  auto load = [&](VTile& T, int u, int blk) {
    const int ua = tile0 + u;
    const size_t off = (size_t)blk * bstride + (size_t)(ua & ((1 << tpb_shift) - 1)) * (16 * D * ES);
    const uint32_t bytes = u < ntiles ? (uint32_t)min(tok1 - ua * TT, TT) * (D * ES) : 0u;
    const rsrc_t rk = make_rsrc(kbase + off, bytes);
    const rsrc_t rv = make_rsrc(vbase + off, bytes);
#pragma unroll
    for (int i = 0; i < NLOAD; ++i)
      T.k[i] = KS::template load8<true>(rk, lane_off + (uint32_t)ES * TPL * D * i);
#pragma unroll
    for (int i = 0; i < NLOAD; ++i)
      T.v[i] = KS::template load8<true>(rv, lane_off + (uint32_t)ES * TPL * D * i);
  };

  auto process = [&](const VTile& T, int u) {
    uint4 kr[NLOAD], vr[NLOAD];
#pragma unroll
    for (int i = 0; i < NLOAD; ++i) {
      kr[i] = KS::to16(T.k[i]);
      vr[i] = KS::to16(T.v[i]);
    }
    const int tb = (tile0 + u) * TT;       // absolute position of the tile's row 0
    const int valid = min(tok1 - tb, TT);  // rows [0, valid) are context tokens

    float x[GT][NLOAD];
#pragma unroll
    for (int i = 0; i < NLOAD; ++i) {
      const int row = i * TPL + rho;
      const float rel = (float)(tb + row - qpos);
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        float s = Fmt::dot2(kr[i].x, qv[g][0], 0.f);
        s = Fmt::dot2(kr[i].y, qv[g][1], s);
        s = Fmt::dot2(kr[i].z, qv[g][2], s);
        s = Fmt::dot2(kr[i].w, qv[g][3], s);
        s = group_sum<TPT>(s);
        const float z = fmaf(s, a.scale_log2, slope[g] * rel);
        x[g][i] = row < valid ? z : kNegBig;
      }
    }

#pragma unroll
    for (int g = 0; g < GT; ++g) {
      float mx = x[g][0];
#pragma unroll
      for (int i = 1; i < NLOAD; ++i) mx = score_max(mx, x[g][i]);
      const float mn = score_max(m[g], mx);
      const float alpha = fast_exp2(m[g] - mn);
      m[g] = mn;
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < NLOAD; ++i) {
        x[g][i] = fast_exp2(x[g][i] - mn);
        ps += x[g][i];
      }
      l[g] = fmaf(l[g], alpha, ps);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] *= alpha;
    }

#pragma unroll
    for (int i = 0; i < NLOAD; ++i) {
      const uint4 w = vr[i];  // zeros past the context end (buffer bound)
      const float v[8] = {Fmt::lo(w.x), Fmt::hi(w.x), Fmt::lo(w.y), Fmt::hi(w.y),
                          Fmt::lo(w.z), Fmt::hi(w.z), Fmt::lo(w.w), Fmt::hi(w.w)};
#pragma unroll
      for (int g = 0; g < GT; ++g) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = fmaf(x[g][i], v[e], acc[g][e]);
      }
    }
  };

  // Two register tiles in a software pipeline: wave w takes tiles w, w + 4,
  // ...; the loads of its next tile are in flight while the current one is
  // processed, and the next table entry is read one load ahead.
  int u = wave;
  if (u < ntiles) {
    VTile ta, tb2;
    // the first two block ids were fetched with the query (a second tile
    // past the partition reads nothing; its id is then the first one's)
    load(ta, u, blk_first);
    int blk_next = u + kWaves < ntiles ? blk_second : blk_first;
    while (true) {
      const int u1 = u + kWaves;
      load(tb2, u1, blk_next);
      blk_next = block_of(u1 + kWaves);
      process(ta, u);
      if (u1 >= ntiles) break;
      const int u2 = u1 + kWaves;
      load(ta, u2, blk_next);
      blk_next = block_of(u2 + kWaves);
      process(tb2, u1);
      if (u2 >= ntiles) break;
      u = u2;
    }
  }

  // ---- merge the lane rows of this wave ------------------------------------
#pragma unroll
  for (int g = 0; g < GT; ++g) {
#pragma unroll
    for (int off = TPT; off < 64; off <<= 1) {
      const float mo = shfl_xor(m[g], off);
      const float lo = shfl_xor(l[g], off);
      const float mn = score_max(m[g], mo);
      const float f = fast_exp2(m[g] - mn);
      const float fo = fast_exp2(mo - mn);
      l[g] = l[g] * f + lo * fo;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] = acc[g][e] * f + shfl_xor(acc[g][e], off) * fo;
      m[g] = mn;
    }
  }

  // ---- merge the waves into wave 0 (fixed order: deterministic) ------------
  __shared__ float mrg_acc[GT][D];
  __shared__ float mrg_ml[GT][2];
  for (int w = 1; w < kWaves; ++w) {
    __syncthreads();
    if (wave == w && rho == 0) {
#pragma unroll
      for (int g = 0; g < GT; ++g) {
#pragma unroll
        for (int e = 0; e < 8; ++e) mrg_acc[g][c * 8 + e] = acc[g][e];
        if (c == 0) {
          mrg_ml[g][0] = m[g];
          mrg_ml[g][1] = l[g];
        }
      }
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        const float mo = mrg_ml[g][0];
        const float lo = mrg_ml[g][1];
        const float mn = score_max(m[g], mo);
        const float f = fast_exp2(m[g] - mn);
        const float fo = fast_exp2(mo - mn);
        l[g] = l[g] * f + lo * fo;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = acc[g][e] * f + mrg_acc[g][c * 8 + e] * fo;
        m[g] = mn;
      }
    }
  }

  // ---- finalise -------------------------------------------------------------
  // A sequence whose keys all lie in partition 0 is finished here; the reduce
  // skips it.
  const bool direct = single || (part == 0 && L <= a.partition_blocks * BS);
  if (wave != 0 || rho != 0) return;
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    if (g >= nh) break;
    const float inv = l[g] > 0.f ? a.v_scale / l[g] : 0.f;
    const size_t row = (size_t)seq * a.num_heads + h0 + g;
    if (direct) {
      uint4 o;
      o.x = Fmt::pack(acc[g][0] * inv, acc[g][1] * inv);
      o.y = Fmt::pack(acc[g][2] * inv, acc[g][3] * inv);
      o.z = Fmt::pack(acc[g][4] * inv, acc[g][5] * inv);
      o.w = Fmt::pack(acc[g][6] * inv, acc[g][7] * inv);
      reinterpret_cast<uint4*>(a.out)[row * CH + c] = o;
    } else {
      const size_t slot = row * a.num_partitions + part;
      float4* o = reinterpret_cast<float4*>(a.ws_o + slot * D + c * 8);
      o[0] = make_float4(acc[g][0] * inv, acc[g][1] * inv, acc[g][2] * inv, acc[g][3] * inv);
      o[1] = make_float4(acc[g][4] * inv, acc[g][5] * inv, acc[g][6] * inv, acc[g][7] * inv);
      if (c == 0) reinterpret_cast<float2*>(a.ws_ml)[slot] = make_float2(m[g], l[g]);
    }
  }
}

namespace {

template <typename Fmt, int D, int GT, bool KV8>
hipError_t launch_t(const DecodeArgs& a, hipStream_t s) {
  const int nhc = (a.group + GT - 1) / GT;
  dim3 grid(a.num_kv_heads * nhc, a.num_seqs, a.num_partitions);
  decode_valu_kernel<Fmt, D, GT, KV8><<<grid, kWaves * 64, 0, s>>>(a);
  return hipGetLastError();
}

template <typename Fmt, int D, bool KV8>
hipError_t launch_g(const DecodeArgs& a, hipStream_t s) {
  switch (valu_heads_per_workgroup(a.group)) {
    case 1: return launch_t<Fmt, D, 1, KV8>(a, s);
    case 2: return launch_t<Fmt, D, 2, KV8>(a, s);
    case 4: return launch_t<Fmt, D, 4, KV8>(a, s);
    default: return launch_t<Fmt, D, 8, KV8>(a, s);
  }
}

}  // namespace

template <typename Fmt, bool KV8>
hipError_t launch_d(const DecodeArgs& a, int head_size, hipStream_t s) {
  return head_size == 64 ? launch_g<Fmt, 64, KV8>(a, s) : launch_g<Fmt, 128, KV8>(a, s);
}

hipError_t launch_decode_valu(const DecodeArgs& a, int dtype, int head_size, bool kv_fp8,
                              hipStream_t s) {
  if (dtype == 0)
    return kv_fp8 ? launch_d<F16, true>(a, head_size, s) : launch_d<F16, false>(a, head_size, s);
  return kv_fp8 ? launch_d<BF16, true>(a, head_size, s) : launch_d<BF16, false>(a, head_size, s);
}

}  // namespace pa
