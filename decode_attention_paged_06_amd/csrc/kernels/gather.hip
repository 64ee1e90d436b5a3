// The two row copies between contiguous [num_tokens, num_kv_heads, head_size]
// tensors and the paged cache, bit for bit:
//   gather_cached_kv     cache rows of a list of slots -> contiguous tensors (the
//                        "Memcpy kernel for flash attention" of vLLM PR #29);
//   paged_kv_cache_write contiguous new-token rows -> their cache slots (the cache
//                        operation that precedes attention in vLLM PR #2744).
//
// One thread moves one 16-byte chunk of K and the same chunk of V.  A
// (token, head) row is head_size * element-size contiguous bytes at both ends
// (in either cache layout: separate K and V tensors, or K and V tiles of each
// (block, kv head) side by side), so
// consecutive threads read and write consecutive 16-byte chunks; a row is
// never split across a wave boundary for head sizes that divide 64 chunks.
// Only integer moves: NaN payloads and signed zeros pass through unchanged.
#include "../launch.h"
#include "device_common.h"

namespace pa {

__global__ __launch_bounds__(256) void gather_kv_kernel(uint4* __restrict__ k_out,
                                                         uint4* __restrict__ v_out,
                                                         const uint4* __restrict__ k_cache,
                                                         const uint4* __restrict__ v_cache,
                                                         const int32_t* __restrict__ slots,
                                                         uint32_t total, uint32_t ch,
                                                         uint32_t hkv, uint32_t bs,
                                                         uint64_t bstride, uint64_t hstride) {
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const uint32_t row = i / ch;          // token * hkv + head
    const uint32_t c = i - row * ch;
    const uint32_t tok = row / hkv;
    const uint32_t head = row - tok * hkv;
    const int32_t slot = slots[tok];
    uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
    if (slot >= 0) {
      const uint32_t blk = (uint32_t)slot / bs;
      const uint32_t off = (uint32_t)slot - blk * bs;
      const size_t src = blk * bstride + head * hstride + (size_t)off * ch + c;
      kv = load_nt(k_cache + src);
      vv = load_nt(v_cache + src);
    }
    k_out[i] = kv;
    v_out[i] = vv;
  }
}

__global__ __launch_bounds__(256) void cache_write_kernel(uint4* __restrict__ k_cache,
                                                           uint4* __restrict__ v_cache,
                                                           const uint4* __restrict__ k_new,
                                                           const uint4* __restrict__ v_new,
                                                           const int32_t* __restrict__ slots,
                                                           uint32_t total, uint32_t ch,
                                                           uint32_t hkv, uint32_t bs,
                                                           uint64_t bstride, uint64_t hstride) {
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const uint32_t row = i / ch;          // token * hkv + head
    const uint32_t c = i - row * ch;
    const uint32_t tok = row / hkv;
    const uint32_t head = row - tok * hkv;
    const int32_t slot = slots[tok];
    if (slot < 0) continue;               // padding token: nothing to store
    const uint32_t blk = (uint32_t)slot / bs;
    const uint32_t off = (uint32_t)slot - blk * bs;
    const size_t dst = blk * bstride + head * hstride + (size_t)off * ch + c;
    k_cache[dst] = load_nt(k_new + i);
    v_cache[dst] = load_nt(v_new + i);
  }
}

hipError_t launch_cache_write(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                              const int32_t* slots, int32_t num_tokens, int32_t num_kv_heads,
                              int32_t row_bytes, int32_t block_size, int64_t block_stride,
                              int64_t head_stride, hipStream_t s) {
  const uint32_t ch = (uint32_t)row_bytes / 16;
  const uint32_t total = (uint32_t)num_tokens * (uint32_t)num_kv_heads * ch;
  uint32_t blocks = (total + 255) / 256;
  if (blocks > 65536u) blocks = 65536u;
  cache_write_kernel<<<blocks, 256, 0, s>>>(
      static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), static_cast<const uint4*>(k_new),
      static_cast<const uint4*>(v_new), slots, total, ch, (uint32_t)num_kv_heads,
      (uint32_t)block_size, (uint64_t)block_stride / 16, (uint64_t)head_stride / 16);
  return hipGetLastError();
}

hipError_t launch_gather(void* k_out, void* v_out, const void* k_cache, const void* v_cache,
                         const int32_t* slots, int32_t num_tokens, int32_t num_kv_heads,
                         int32_t row_bytes, int32_t block_size, int64_t block_stride,
                         int64_t head_stride, hipStream_t s) {
  const uint32_t ch = (uint32_t)row_bytes / 16;
  const uint32_t total = (uint32_t)num_tokens * (uint32_t)num_kv_heads * ch;
  const uint32_t threads = 256;
  uint32_t blocks = (total + threads - 1) / threads;
  if (blocks > 65536u) blocks = 65536u;
  gather_kv_kernel<<<blocks, threads, 0, s>>>(
      static_cast<uint4*>(k_out), static_cast<uint4*>(v_out), static_cast<const uint4*>(k_cache),
      static_cast<const uint4*>(v_cache), slots, total, ch, (uint32_t)num_kv_heads,
      (uint32_t)block_size, (uint64_t)block_stride / 16, (uint64_t)head_stride / 16);
  return hipGetLastError();
}

}  // namespace pa
