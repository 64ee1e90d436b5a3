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
  // (longest first, staged kernel) workgroups b >= static_wgs -- those that
  // start as earlier ones retire -- take their place in that order from the
  // counter at *ticket (zeroed by the order kernel) in the order they start,
  // whatever XCD they run on
  int32_t* ticket = nullptr;
  int32_t static_wgs = 0;
  // Equal-share schedule (decode on the LDS-staged kernel): stream_wgs > 0
  // workgroups split the batch's tiles, walked item by item (item = kv head *
  // num_seqs + sequence, a sequence's tiles of min(16, block_size) tokens in
  // order), into equal consecutive shares.  Workgroup b's piece of an item that
  // it does not hold whole leaves its partial in slot item + b of ws_o / ws_ml,
  // laid out [head of the group][num_slots][D] and [head of the group][num_slots];
  // workgroup 0 leaves each sequence's first tile in ws_pfx[0 .. num_seqs]
  // (ws_pfx[num_seqs] = tiles of one kv head).
  int32_t stream_wgs = 0;
  int32_t num_slots = 0;
  int32_t* ws_pfx = nullptr;
  // Stream positions each item takes before its tiles: a piece's fixed cost
  // (start-up and finish) in units of one tile's walk, so that shares come
  // out equal in time rather than in tiles (>= 1).
  int32_t piece_cost = 1;
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

// Equal shares of T stream positions among G <= T workgroups (a call with
// fewer positions than workgroups uses G = T): workgroup b takes
// [stream_share_start(b), stream_share_start(b + 1)), at least one position,
// and position x (0 <= x < T) lies in the share of workgroup stream_owner(x),
// so the workgroups holding pieces of an item are consecutive.
__host__ __device__ inline int64_t stream_share_start(int64_t b, int64_t T, int64_t G) {
  return b * T / G;
}
__host__ __device__ inline int64_t stream_owner(int64_t x, int64_t T, int64_t G) {
  return ((x + 1) * G - 1) / T;
}
// Largest batch an equal-share call takes (the tile prefix of num_seqs + 1
// ints is built in the kernel's LDS work area).
constexpr int kStreamMaxSeqs = 2048;

// The kernel's LDS arrays per configuration (also what sizes the equal-share
// grid on the host): a work area -- the query rows before the tile loop, the
// staged ring during it, the token-group merge after it -- and, staged, a
// window of kTableWindow 64-bit tile source offsets.
template <int D, int NT, int TG, int RT, int KT, bool KV8>
struct DecodeLds {
  static constexpr int kES = KV8 ? 1 : 2;
  static constexpr bool kStage = NT > 1;
  static constexpr int kRing = KT == 2 ? 3 : 4;
  static constexpr int kStageBytes = 32 * D * kES;  // K then V of one 16-row tile
  static constexpr int kRingBytes = kStage ? TG * kRing * KT * kStageBytes : 0;
  static constexpr int kMergeSlotBytes = NT * RT * ((D / 16) * 64 * 16 + 2 * 64 * 4);
  static constexpr int kMergeBytes = TG > 1 ? (TG - 1) * kMergeSlotBytes : 0;
  static constexpr int kQueryBytes = NT * RT * 16 * D * 2;
  static constexpr int kWorkBytes = kRingBytes > kMergeBytes
                                        ? (kRingBytes > kQueryBytes ? kRingBytes : kQueryBytes)
                                        : (kMergeBytes > kQueryBytes ? kMergeBytes : kQueryBytes);
  static constexpr int kTableWindow = 512;
  static constexpr int kBytes = kWorkBytes + 8 * (kStage ? kTableWindow : 1);
};

// Token groups (sets of NT waves walking every TG-th tile) of the staged
// decode kernel for NT head tiles, as launch_decode_mfma picks them.
constexpr int staged_token_groups(int nt) { return nt == 2 ? 2 : nt == 3 ? 4 : 1; }
template <int D, bool KV8>
constexpr int staged_lds_bytes(int nt) {
  return nt == 2   ? DecodeLds<D, 2, staged_token_groups(2), 1, KV8 ? 2 : 1, KV8>::kBytes
         : nt == 3 ? DecodeLds<D, 3, staged_token_groups(3), 1, KV8 ? 2 : 1, KV8>::kBytes
                   : DecodeLds<D, 4, staged_token_groups(4), 1, KV8 ? 2 : 1, KV8>::kBytes;
}
constexpr int kLdsPerCu = 160 * 1024;  // gfx950
constexpr int kWavesPerCu = 32;        // 8 per SIMD
// A piece's fixed cost in tiles of its workgroup's walk: ~7 us of start-up
// and finish per piece against ~0.29 us per 16-bit tile for a 12-wave
// workgroup alone on its CU (MQA 48/1 at batch 256: workgroups with 1 / 2 / 3
// / 4 pieces of equal tile shares took 85 / 92 / 99 / 106 us); a workgroup
// sharing its CU with others walks each tile proportionally slower, and FP8
// tiles take about half the time.
inline int staged_piece_cost(int wgs_per_cu, bool kv_fp8) {
  const int c = (kv_fp8 ? 48 : 24) / (wgs_per_cu > 0 ? wgs_per_cu : 1);
  return c > 1 ? c : 1;
}
// Workgroups of the LDS-staged decode kernel (groups of more than 16 heads)
// that one CU holds at once by LDS and wave slots: what an equal-share plan
// sizes its workspace for (the launch takes the device's occupancy, at most this).
inline int staged_decode_wgs_per_cu(int head_size, int group, bool kv_fp8) {
  const int nt = mfma_head_tiles(group);
  const int lds = head_size == 64 ? (kv_fp8 ? staged_lds_bytes<64, true>(nt) : staged_lds_bytes<64, false>(nt))
                                  : (kv_fp8 ? staged_lds_bytes<128, true>(nt) : staged_lds_bytes<128, false>(nt));
  const int by_lds = kLdsPerCu / lds, by_waves = kWavesPerCu / (nt * staged_token_groups(nt));
  return by_lds < by_waves ? by_lds : by_waves;
}
// The same as the runtime's occupancy calculator reports for the kernel (for
// tests of the table above); needs a device.
hipError_t staged_decode_occupancy(int dtype, int head_size, int group, bool kv_fp8, int* wgs);

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
