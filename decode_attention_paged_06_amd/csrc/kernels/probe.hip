// Streaming-read probe: reads a buffer once with the 16-byte non-temporal
// loads the decode kernels use.  Workgroup b owns one contiguous slice of the
// buffer; its four waves take interleaved runs of eight consecutive 1 KB
// wave-wide loads, all in flight at once.  Its time over a buffer much larger
// than the last-level cache is what plain streaming reaches on the device:
// the measured ceiling that the decode kernels' HBM figures are read against.
// (Measured on MI355X over 4 GiB: 88-89% of the 8 TB/s peak with contiguous
// slices of 1024..8192 workgroups; a grid-stride order, where each lane's
// consecutive loads lie a whole grid apart, reached 78%.)
//
// The loaded words are folded into one XOR per lane; a lane stores it only if
// every bit is set (practically never for any real data), which keeps the
// loads live without adding write traffic.
#include "../launch.h"
#include "device_common.h"

namespace pa {

namespace {

constexpr int kRuns = 8;  // 1 KB wave-wide loads in flight per wave

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
    for (int u = 0; u < kRuns; ++u) {
      acc.x ^= v[u].x;
      acc.y ^= v[u].y;
      acc.z ^= v[u].z;
      acc.w ^= v[u].w;
    }
  }
  if ((acc.x & acc.y & acc.z & acc.w) == 0xffffffffu) sink[blockIdx.x] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, void* sink, hipStream_t s) {
  const int grid = stream_read_grid(bytes);
  if (grid == 0) return hipSuccess;
  const size_t n16 = bytes / 16;
  const size_t per = (n16 + grid - 1) / grid;
  stream_read_kernel<<<grid, 256, 0, s>>>(static_cast<const uint4*>(src), n16, per,
                                          static_cast<uint4*>(sink));
  return hipGetLastError();
}

}  // namespace pa
