// Streaming-read probe: reads a buffer once with the 16-byte non-temporal
// loads the decode kernels use.  Its time over a buffer much larger than the
// last-level cache is what plain streaming reaches on the device: the
// measured ceiling that the decode kernels' HBM figures are read against.
//
// Two orders:
//  * contiguous (run_bytes = 0): workgroup b owns one contiguous slice of the
//    buffer; its four waves take interleaved runs of eight consecutive 1 KB
//    wave-wide loads, all in flight at once.  (Measured on MI355X over 4 GiB:
//    88-89% of the 8 TB/s peak with 1024..8192 workgroups; a grid-stride order,
//    where each lane's consecutive loads lie a whole grid apart, reached 78%.)
//  * scattered runs (run_bytes = R): the buffer is read as runs of R bytes at
//    scattered positions -- logical run r sits at physical run (r * kSpread +
//    kShift) mod n_runs, a bijection for a power-of-two run count -- each run
//    read by one wave as R / 1 KB consecutive wave-wide loads.  With R the size
//    of a cache tile (one block's K and V of one kv head) this is the access
//    pattern of the paged decode without its table reads and arithmetic.
//
// The loaded words are folded into one XOR per lane; a lane stores it only if
// every bit is set (practically never for any real data), which keeps the
// loads live without adding write traffic.
#include "../launch.h"
#include "device_common.h"

namespace pa {

namespace {

constexpr int kRuns = 8;                    // 1 KB wave-wide loads in flight per wave
constexpr uint64_t kSpread = 0x9E3779B1u;   // odd: multiplication permutes runs mod 2^k
constexpr uint64_t kShift = 12345;

__device__ __forceinline__ void fold(uint4& acc, const uint4& v) {
  acc.x ^= v.x;
  acc.y ^= v.y;
  acc.z ^= v.z;
  acc.w ^= v.w;
}

__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ src,
                                                           size_t n16, size_t per,
                                                           uint4* __restrict__ sink) {
  const size_t lo = (size_t)blockIdx.x * per;
  const size_t hi = lo + per < n16 ? lo + per : n16;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  uint4 acc = make_uint4(0, 0, 0, 0);
  for (size_t base = lo + (size_t)wave * 64 * kRuns; base < hi; base += 4 * 64 * kRuns) {
    uint4 v[kRuns];
#pragma unroll
    for (int u = 0; u < kRuns; ++u) {
      const size_t idx = base + (size_t)u * 64 + lane;
      v[u] = idx < hi ? load_nt(src + idx) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kRuns; ++u) fold(acc, v[u]);
  }
  if ((acc.x & acc.y & acc.z & acc.w) == 0xffffffffu) sink[blockIdx.x] = acc;
}

// Runs of `run16` 16-byte chunks (a multiple of 64: whole 1 KB wave loads);
// n_runs a power of two.  Workgroup b takes logical runs b * per_runs ...,
// wave w every fourth of them, kRuns 1 KB loads in flight at a time.
__global__ __launch_bounds__(256) void scattered_read_kernel(const uint4* __restrict__ src,
                                                              size_t n_runs, size_t run16,
                                                              size_t per_runs,
                                                              uint4* __restrict__ sink) {
  const size_t lo = (size_t)blockIdx.x * per_runs;
  const size_t hi = lo + per_runs < n_runs ? lo + per_runs : n_runs;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  uint4 acc = make_uint4(0, 0, 0, 0);
  for (size_t r = lo + wave; r < hi; r += 4) {
    const size_t phys = (r * kSpread + kShift) & (n_runs - 1);
    const uint4* run = src + phys * run16 + lane;
    for (size_t c = 0; c < run16; c += 64 * kRuns) {
      uint4 v[kRuns];
#pragma unroll
      for (int u = 0; u < kRuns; ++u) {
        const size_t idx = c + (size_t)u * 64;
        v[u] = idx < run16 ? load_nt(run + idx) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < kRuns; ++u) fold(acc, v[u]);
    }
  }
  if ((acc.x & acc.y & acc.z & acc.w) == 0xffffffffu) sink[blockIdx.x] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, size_t run_bytes, void* sink,
                              hipStream_t s) {
  const int grid = stream_read_grid(bytes);
  if (grid == 0) return hipSuccess;
  const size_t n16 = bytes / 16;
  if (run_bytes == 0) {
    const size_t per = (n16 + grid - 1) / grid;
    stream_read_kernel<<<grid, 256, 0, s>>>(static_cast<const uint4*>(src), n16, per,
                                            static_cast<uint4*>(sink));
  } else {
    const size_t n_runs = bytes / run_bytes;
    const size_t per_runs = (n_runs + grid - 1) / grid;
    scattered_read_kernel<<<grid, 256, 0, s>>>(static_cast<const uint4*>(src), n_runs, run_bytes / 16,
                                               per_runs, static_cast<uint4*>(sink));
  }
  return hipGetLastError();
}

}  // namespace pa
