// Longest-first order of the split-decode work units.
//
// With ragged context lengths the partitions of a split plan hold very
// different token counts (a sequence's last partition is partial, short
// sequences leave later partitions empty).  Workgroups are dispatched in grid
// order as earlier ones retire, so starting the longest units first keeps the
// tail of the launch short: the classic longest-processing-time-first list
// schedule.  One workgroup buckets the units by token count (a counting sort
// in LDS) and writes the order the decode kernel then follows, and zeroes the
// counter from which the decode's later workgroups take their places.
#include "../launch.h"
#include "device_common.h"

namespace pa {

namespace {

constexpr int kOrderThreads = 1024;
constexpr int kBuckets = 64;  // bucket 0: full partitions ... 62: shortest, 63: empty
constexpr int kKeep = 4;      // units per thread whose bucket the second pass reuses

__global__ __launch_bounds__(kOrderThreads) void unit_order_kernel(const DecodeArgs a, int32_t* order) {
  __shared__ int count[kBuckets];
  __shared__ int cursor[kBuckets];
  const int S = a.num_seqs;
  const int n_units = S * a.num_partitions;
  const int ptok = a.partition_blocks * a.block_size;
  const int max_len = a.max_blocks_per_seq * a.block_size;
  auto bucket_of = [&](int u) {
    const int seq = u % S;
    const int part = u / S;
    const int L = min(a.context_lens[seq], max_len);
    const int w = min(max(L - part * ptok, 0), ptok);
    return w == 0 ? kBuckets - 1 : (int)((long long)(ptok - w) * (kBuckets - 2) / ptok);
  };
  for (int b = threadIdx.x; b < kBuckets; b += kOrderThreads) count[b] = 0;
  if (threadIdx.x == 0 && a.ticket != nullptr) *a.ticket = 0;
  __syncthreads();
  // the buckets of this thread's first kKeep units stay in registers for the
  // second pass (one round trip to the lengths fewer)
  int kept[kKeep];
#pragma unroll
  for (int k = 0; k < kKeep; ++k) {
    const int u = threadIdx.x + k * kOrderThreads;
    kept[k] = u < n_units ? bucket_of(u) : -1;
  }
#pragma unroll
  for (int k = 0; k < kKeep; ++k)
    if (kept[k] >= 0) atomicAdd(&count[kept[k]], 1);
  for (int u = threadIdx.x + kKeep * kOrderThreads; u < n_units; u += kOrderThreads)
    atomicAdd(&count[bucket_of(u)], 1);
  __syncthreads();
  if (threadIdx.x == 0) {
    int sum = 0;
    for (int b = 0; b < kBuckets; ++b) {
      cursor[b] = sum;
      sum += count[b];
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kKeep; ++k)
    if (kept[k] >= 0) order[atomicAdd(&cursor[kept[k]], 1)] = threadIdx.x + k * kOrderThreads;
  for (int u = threadIdx.x + kKeep * kOrderThreads; u < n_units; u += kOrderThreads)
    order[atomicAdd(&cursor[bucket_of(u)], 1)] = u;
}

}  // namespace

hipError_t launch_unit_order(const DecodeArgs& a, int32_t* order, hipStream_t s) {
  unit_order_kernel<<<1, kOrderThreads, 0, s>>>(a, order);
  return hipGetLastError();
}

}  // namespace pa
