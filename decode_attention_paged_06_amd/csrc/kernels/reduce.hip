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
// multi-query call).  One wave per (head, sequence, new token); lane k owns
// D/64 output elements.
#include "../launch.h"
#include "device_common.h"

namespace pa {

template <typename Fmt, int D>
__global__ __launch_bounds__(64) void partition_reduce_kernel(const DecodeArgs a) {
  constexpr int PER = D / 64;
  static_assert(PER == 1 || PER == 2, "head size 64 or 128");
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
  const float2* ml = reinterpret_cast<const float2*>(a.ws_ml) + row * a.num_partitions;
  const float* o = a.ws_o + row * a.num_partitions * D + lane * PER;

  float M = kNegBig;
  for (int p = 0; p < nact; ++p) M = fmaxf(M, ml[p].x);
  float wsum = 0.f, acc0 = 0.f, acc1 = 0.f;
  for (int p = 0; p < nact; ++p) {
    const float2 s = ml[p];
    const float w = s.y * fast_exp2(s.x - M);
    wsum += w;
    if constexpr (PER == 2) {
      const float2 v = *reinterpret_cast<const float2*>(o + (size_t)p * D);
      acc0 = fmaf(w, v.x, acc0);
      acc1 = fmaf(w, v.y, acc1);
    } else {
      acc0 = fmaf(w, o[(size_t)p * D], acc0);
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  if constexpr (PER == 2) {
    *reinterpret_cast<uint32_t*>(orow) = Fmt::pack(acc0 * inv, acc1 * inv);
  } else {
    *orow = (uint16_t)(Fmt::pack(acc0 * inv, 0.f) & 0xffffu);
  }
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
