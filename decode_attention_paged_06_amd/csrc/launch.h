// Internal interface between the C-ABI host layer (host/api.cpp) and the
// HIP kernels (kernels/*.hip).  Not installed; the public contract is
// include/paged_attention.h.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace pa {

constexpr int kMinBlockSize = 8;    // decode block sizes: powers of two in [8, 256]
constexpr int kMaxBlockSize = 256;
constexpr int kWaves = 4;        // waves per decode workgroup
constexpr int kMaxGroup = 64;    // largest num_heads / num_kv_heads supported

// Everything a decode launch needs.  Pointers are device memory.
struct DecodeArgs {
  void* out;                    // [S, Hq, D] storage type
  const void* q;                // [S, Hq, D]
  const void* k_cache;          // first K tile; (block, kv head) tiles of [BS, D] at the strides below
  const void* v_cache;          // first V tile; same strides
  const int32_t* block_tables;  // [S, MAXB]
  const int32_t* context_lens;  // [S]
  const float* alibi;           // [Hq] or nullptr
  float* ws_o;                  // [S, Hq, P, D] fp32 normalised partial outputs (split only)
  float* ws_ml;                 // [S, Hq, P, 2] fp32 (running max in log2 units, sum)
  float scale_log2;             // scale * log2(e)
  int32_t num_seqs;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t max_blocks_per_seq;
  int32_t group;                // num_heads / num_kv_heads
  int32_t num_partitions;       // 1 = single pass straight to `out`
  int32_t partition_blocks;     // cache blocks per partition
  int32_t block_size;           // tokens per cache block (a power of two, 8..256)
  int32_t block_shift;          // log2(block_size)
  float v_scale;                // multiplies the values (1 for 16-bit caches)
  // Multi-query (prefill) calls: sequence s's new tokens are packed rows
  // query_start[s] .. query_start[s+1]-1 of q/out and are its last
  // query_start[s+1]-query_start[s] context tokens.  nullptr = decode (one new
  // token per sequence, row s).
  const int32_t* query_start;
  int32_t max_new_tokens;       // bound on new tokens per sequence (1 for decode)
  int32_t row_chunks;           // workgroups per (sequence, kv head) over the query rows
  // Longest-first schedule: the decode grid is 1-D, workgroup b takes
  // (sequence, partition) unit_order[b / (num_kv_heads * row_chunks)], encoded
  // partition * num_seqs + sequence.  nullptr = the grid's own order.
  const int32_t* unit_order = nullptr;
  // Cache addressing in bytes: the (block, kv head) tile of both caches starts
  // at block * kv_block_stride + kv_head * kv_head_stride from its base.
  int64_t kv_block_stride = 0;
  int64_t kv_head_stride = 0;
};

// Multi-query workgroups: kPrefillWaves waves, each computing
// kPrefillRowTilesPerWave tiles of 16 query rows against every K/V tile it
// reads (the K/V operands and the V regrouping serve all its row tiles).
constexpr int kPrefillWaves = 4;
constexpr int kPrefillRowTilesPerWave = 2;
constexpr int kPrefillRows = 16 * kPrefillWaves * kPrefillRowTilesPerWave;  // rows per workgroup

// Query heads per VALU workgroup for a group size (heads that share a kv head
// are processed in chunks of this many; larger groups use several chunks).
inline int valu_heads_per_workgroup(int group) {
  return group <= 1 ? 1 : group <= 2 ? 2 : group <= 4 ? 4 : 8;
}

// 16-head MFMA tiles needed for a group of `group` query heads.
inline int mfma_head_tiles(int group) { return (group + 15) / 16; }

// dtype: 0 = fp16, 1 = bf16 (pa_dtype).  head_size: 64 or 128.  kv_fp8: the
// caches hold FP8 E4M3 codes (scale_log2 already carries the key scale).
hipError_t launch_decode_valu(const DecodeArgs& a, int dtype, int head_size, bool kv_fp8,
                              hipStream_t s);
hipError_t launch_decode_mfma(const DecodeArgs& a, int dtype, int head_size, bool kv_fp8,
                              hipStream_t s);
hipError_t launch_partition_reduce(const DecodeArgs& a, int dtype, int head_size, hipStream_t s);

// Multi-query calls on 32 x 32 matrix tiles (same grid, row chunks of
// kPrefillRows, partials and reduce as the general kernel): 16-bit caches,
// head size 128, blocks of at least 16 tokens.
bool prefill_mfma32_supported(int head_size, bool kv_fp8, int block_size);
hipError_t launch_prefill_mfma32(const DecodeArgs& a, int dtype, hipStream_t s);

// Writes the num_seqs * num_partitions decode units (sequence, partition),
// encoded partition * num_seqs + sequence, to `order` sorted by decreasing
// token count (in buckets of partition_size / 62 tokens; order within a
// bucket unspecified), empty units last.
hipError_t launch_unit_order(const DecodeArgs& a, int32_t* order, hipStream_t s);

// Row copies move row_bytes-long rows (a multiple of 16) between the cache and
// contiguous [num_tokens, num_kv_heads] row arrays.  The cache's (block, kv
// head) tile starts block * block_stride + kv_head * head_stride bytes from
// its base (both multiples of 16).
hipError_t launch_gather(void* k_out, void* v_out, const void* k_cache, const void* v_cache,
                         const int32_t* slots, int32_t num_tokens, int32_t num_kv_heads,
                         int32_t row_bytes, int32_t block_size, int64_t block_stride,
                         int64_t head_stride, hipStream_t s);

hipError_t launch_cache_write(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                              const int32_t* slots, int32_t num_tokens, int32_t num_kv_heads,
                              int32_t row_bytes, int32_t block_size, int64_t block_stride,
                              int64_t head_stride, hipStream_t s);

// Device address of the allocation-free entry point's scratch array on
// `device`, which must be the current device (looked up once per device,
// then cached).  The array holds PA_NOALLOC_SCRATCH_BYTES bytes.
hipError_t noalloc_scratch(int device, void** ptr);

// Streaming-read probe: reads `bytes` (a multiple of 16) at `src` once;
// `sink` holds stream_read_grid(bytes) 16-byte slots (practically never
// written).  At most kStreamReadMaxBlocks workgroups of 256 threads.
constexpr int kStreamReadMaxBlocks = 4096;
// One workgroup per 32 KB of the buffer, at most kStreamReadMaxBlocks.
inline int stream_read_grid(size_t bytes) {
  const size_t blocks = (bytes / 16 + 2047) / 2048;
  return (int)(blocks < (size_t)kStreamReadMaxBlocks ? blocks : (size_t)kStreamReadMaxBlocks);
}
// run_bytes: 0 for contiguous slices per workgroup, else runs of run_bytes (a
// power of two >= 1024 dividing bytes, bytes / run_bytes a power of two) at
// scattered positions.
hipError_t launch_stream_read(const void* src, size_t bytes, size_t run_bytes, void* sink,
                              hipStream_t s);

}  // namespace pa
