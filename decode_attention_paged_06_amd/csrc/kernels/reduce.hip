// Combine the split-context partials of paged decode attention.
//
// The pages time a second paged-attention variant ("Paged attention V2",
// kernel-latency tables of vLLM PR #2744) that wins at small batch and long
// context; it splits each sequence's context into partitions.  Each partition
// p of (sequence s, head h) left
//   m_p  running max of its logits (log2 units),
//   l_p  sum of exp2(logit - m_p) over its tokens,
//   o_p  its softmax-normalised output (fp32).
// The full result is the exact merge
//   M = max_p m_p,  w_p = l_p * exp2(m_p - M),  out = sum_p w_p o_p / sum_p w_p
// over the partitions that hold keys the row sees (p < ceil(visible /
// partition_size), visible = L_s for decode, position + 1 for a new token of a
// multi-query call).  A row with a single such partition was written by the
// decode kernel itself and is skipped here.  Under the equal-share schedule
// the pieces of an item (kv head, sequence) that several decode workgroups
// walked take the place of the partitions.  One wave per (head, sequence, new
// token).  The (m_p,
// l_p) pairs are read one partition per lane (64 at a time) and reduced across
// the wave; the partial outputs are read in batches whose loads are all in
// flight together, so a row costs a few memory round trips however many
// partitions it has.
#include <type_traits>

#include "../launch.h"
#include "device_common.h"

namespace pa {

// Maximum (of running maxima: finite) / sum over the 64 lanes of a wave;
// every lane receives the result.
__device__ __forceinline__ float wave_max(float x) {
  x = score_max(x, dpp<kDppQuadXor1>(x));
  x = score_max(x, dpp<kDppQuadXor2>(x));
  x = score_max(x, dpp<kDppRowHalfMirror>(x));
  x = score_max(x, dpp<kDppRowMirror>(x));
  return column_max4(x);
}
__device__ __forceinline__ float wave_sum(float x) { return column_sum4(group_sum<16>(x)); }

// Weighted sum of a row's active partitions.  Lane k holds D/64 elements of
// every partial output; NB partial-output loads per lane are in flight at a
// time (NB chosen from the partition count, up to 32, so that no load is
// wasted on a short row and up to 32 partitions cost one round trip: GQA
// 64/8 batch 1, graph replay, 16 -> 32: context 4096 10.6 -> 10.3 us, 1024
// 8.5 -> 8.3 us).  The first batch is requested before the weights are known, so
// its loads overlap the (m, l) round trip.
template <int NB, typename Part>
__device__ __forceinline__ void weighted_sum(const float2* ml, const Part* o, int nact, int stride,
                                             int lane, float& wsum, float& acc0, float& acc1) {
  Part v[NB];
  auto fetch = [&](int first) {
#pragma unroll
    for (int k = 0; k < NB; ++k) v[k] = o[(size_t)min(first + k, nact - 1) * stride];
  };
  // lane k holds (m, l) of partition k of the first 64; M = max_p m_p
  const float2 s0 = ml[min(lane, nact - 1)];
  fetch(0);
  const float m0 = lane < nact ? s0.x : kNegBig;
  const float l0 = lane < nact ? s0.y : 0.f;
  float M = m0;
  for (int c = 64; c < nact; c += 64) M = score_max(M, c + lane < nact ? ml[c + lane].x : kNegBig);
  M = wave_max(M);

  for (int c = 0; c < nact; c += 64) {
    // lane k holds the weight of partition c + k (0 past the last one)
    float w = 0.f;
    if (c == 0) {
      w = lane < nact ? l0 * fast_exp2(m0 - M) : 0.f;
    } else if (c + lane < nact) {
      const float2 s = ml[c + lane];
      w = s.y * fast_exp2(s.x - M);
    }
    wsum += w;
    const int n = min(64, nact - c);
    for (int b = 0; b < n; b += NB) {
      // every load is issued (indices past the last partition re-read it and
      // get weight 0), so all NB loads are in flight together
      if (c + b > 0) fetch(c + b);
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), b + k));
        if constexpr (sizeof(Part) == 8) {
          acc0 = fmaf(wk, v[k].x, acc0);
          acc1 = fmaf(wk, v[k].y, acc1);
        } else {
          acc0 = fmaf(wk, v[k], acc0);
        }
      }
    }
  }
}

// The merged row: the weighted sum over the lanes' partial weight sums.
template <typename Fmt, int PER>
__device__ __forceinline__ void store_row(uint16_t* orow, float wsum, float acc0, float acc1) {
  wsum = wave_sum(wsum);
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  if constexpr (PER == 2) {
    *reinterpret_cast<uint32_t*>(orow) = Fmt::pack(acc0 * inv, acc1 * inv);
  } else {
    *orow = (uint16_t)(Fmt::pack(acc0 * inv, 0.f) & 0xffffu);
  }
}

template <typename Fmt, int D>
__global__ __launch_bounds__(64) void partition_reduce_kernel(const DecodeArgs a) {
  constexpr int PER = D / 64;
  static_assert(PER == 1 || PER == 2, "head size 64 or 128");
  using Part = typename std::conditional<PER == 2, float2, float>::type;
  const int h = blockIdx.x;
  const int seq = blockIdx.y;
  const int i = blockIdx.z;  // new token of the sequence (0 for decode)
  const int lane = threadIdx.x;
  int q_first = seq, n_new = 1;
  if (a.query_start != nullptr) {
    q_first = a.query_start[seq];
    n_new = a.query_start[seq + 1] - q_first;
  }
  if (i >= n_new) return;
  const size_t row = (size_t)(q_first + i) * a.num_heads + h;
  uint16_t* orow = reinterpret_cast<uint16_t*>(a.out) + row * D + lane * PER;

  if (a.stream_wgs > 0) {
    // Equal shares: item kvh * S + seq has its tiles at stream positions
    // [x0, x0 + n) (after its piece_cost positions); the workgroups whose
    // shares meet them left their partials in consecutive slots item + b,
    // b = owner(x0) .. owner(x0 + n - 1).
    const int S = a.num_seqs;
    const int kvh = h / a.group;
    const int g = h - kvh * a.group;
    const int64_t cost = a.piece_cost;
    const int p0 = a.ws_pfx[seq], n = a.ws_pfx[seq + 1] - p0;
    const int64_t T1 = a.ws_pfx[S] + cost * S;
    if (n <= 0) {  // no context: zero output row
      if constexpr (PER == 2) *reinterpret_cast<uint32_t*>(orow) = 0u;
      else *orow = 0;
      return;
    }
    const int64_t T = T1 * a.num_kv_heads;
    const int64_t nwg = T < a.stream_wgs ? T : a.stream_wgs;  // workgroups with a share
    const int64_t x0 = kvh * T1 + p0 + cost * (seq + 1);
    const int bf = (int)stream_owner(x0, T, nwg);
    const int nact = (int)stream_owner(x0 + n - 1, T, nwg) - bf + 1;
    if (nact == 1) return;  // one workgroup held the whole item and wrote this row
    const size_t first = (size_t)g * a.num_slots + (size_t)kvh * S + seq + bf;
    const float2* ml = reinterpret_cast<const float2*>(a.ws_ml) + first;
    const Part* o = reinterpret_cast<const Part*>(a.ws_o + first * D) + lane;
    float wsum = 0.f, acc0 = 0.f, acc1 = 0.f;
    if (nact <= 4) weighted_sum<4>(ml, o, nact, D / PER, lane, wsum, acc0, acc1);
    else if (nact <= 8) weighted_sum<8>(ml, o, nact, D / PER, lane, wsum, acc0, acc1);
    else if (nact <= 16) weighted_sum<16>(ml, o, nact, D / PER, lane, wsum, acc0, acc1);
    else weighted_sum<32>(ml, o, nact, D / PER, lane, wsum, acc0, acc1);
    store_row<Fmt, PER>(orow, wsum, acc0, acc1);
    return;
  }

  const int L = min(a.context_lens[seq], a.max_blocks_per_seq * a.block_size);
  if (L <= 0) {
    if constexpr (PER == 2) *reinterpret_cast<uint32_t*>(orow) = 0u;
    else *orow = 0;
    return;
  }
  // partitions holding the keys this row sees (0 .. its position)
  const int ptok = a.partition_blocks * a.block_size;
  const int visible = L - n_new + i + 1;
  const int nact = min(a.num_partitions, (visible + ptok - 1) / ptok);
  if (nact == 1) return;  // the decode kernel wrote this row (all its keys in partition 0)
  const float2* ml = reinterpret_cast<const float2*>(a.ws_ml) + row * a.num_partitions;
  const Part* o = reinterpret_cast<const Part*>(a.ws_o + row * a.num_partitions * D) + lane;

  float wsum = 0.f, acc0 = 0.f, acc1 = 0.f;
  if (nact <= 4) weighted_sum<4>(ml, o, nact, D / PER, lane, wsum, acc0, acc1);
  else if (nact <= 8) weighted_sum<8>(ml, o, nact, D / PER, lane, wsum, acc0, acc1);
  else if (nact <= 16) weighted_sum<16>(ml, o, nact, D / PER, lane, wsum, acc0, acc1);
  else weighted_sum<32>(ml, o, nact, D / PER, lane, wsum, acc0, acc1);  // (batch 1: 32 partitions in one round trip)
  store_row<Fmt, PER>(orow, wsum, acc0, acc1);
}

hipError_t launch_partition_reduce(const DecodeArgs& a, int dtype, int head_size, hipStream_t s) {
  dim3 grid(a.num_heads, a.num_seqs, a.max_new_tokens);
  if (dtype == 0) {
    if (head_size == 64) partition_reduce_kernel<F16, 64><<<grid, 64, 0, s>>>(a);
    else partition_reduce_kernel<F16, 128><<<grid, 64, 0, s>>>(a);
  } else {
    if (head_size == 64) partition_reduce_kernel<BF16, 64><<<grid, 64, 0, s>>>(a);
    else partition_reduce_kernel<BF16, 128><<<grid, 64, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace pa
