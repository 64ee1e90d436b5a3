// C-ABI host layer: argument validation, the launch planner, workspace sizing,
// dispatch and error reporting.  See include/paged_attention.h for the
// contract.  Nothing here reads device memory or synchronises a stream.
#include "paged_attention.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "launch.h"
#include "measure.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_last_error[0] = '\0';
  return PA_OK;
}

constexpr size_t kWsAlign = 256;
constexpr int kMaxDevices = 64;
// Workgroups per CU the auto plan aims for before it splits contexts.  Decode
// with one head tile (4-wave workgroups): one per CU, in partitions of at
// least 64 tokens -- fewer, longer partitions measured faster than two per CU
// (GQA 64/8 context 4096 batch 4: 18.6 -> 17.8 us; context 1024 batch 16:
// 19.1 -> 18.4 us, batch 1: 8.7 -> 8.3 us).  Several head tiles and
// multi-query calls: two per CU (48-head MQA with ragged lengths, 12-wave
// workgroups: two partitions of 4096 tokens measured best, 121 us against 134
// with four).  The VALU engine: one (its split costs more than the grid fill
// gains on the 40-head MHA batch: 320 workgroups run best as one pass).
// One-head-tile decode over an FP8 cache: two per CU, in partitions of at
// least 128 tokens -- its register tiles are half the bytes, so a workgroup
// keeps fewer bytes in flight (GQA 64/8 context 4096, graph replay: batch 16
// 41.2 -> 30.8 us, batch 4 15.2 -> 14.6 us; context 1024 batch 16 16.1 ->
// 15.3 us; batch 1 at context 1024 8.4 -> 8.8 us).
constexpr int kTargetGroupsPerCu = 2;
constexpr int kTargetGroupsPerCuOneTile = 1;
constexpr int kTargetGroupsPerCuOneTileFp8 = 2;
constexpr int kTargetGroupsPerCuValu = 1;
// Smallest partition the auto plan makes: 128 tokens (two 16-row tiles per
// wave), 64 for one-head-tile decode over a 16-bit cache.
constexpr int kMinPartitionTokens = 128;
constexpr int kMinPartitionTokensOneTile = 64;

std::atomic<int> g_num_cus[kMaxDevices];

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_dims(const pa_dims* d) {
  if (d == nullptr) return fail(PA_ERR_INVALID_ARG, "dims is NULL");
  if (d->num_seqs < 0 || d->num_seqs > 65535)
    return fail(PA_ERR_INVALID_ARG, "num_seqs = %d (must be in [0, 65535])", d->num_seqs);
  if (d->num_heads <= 0 || d->num_kv_heads <= 0)
    return fail(PA_ERR_INVALID_ARG, "num_heads = %d, num_kv_heads = %d (must be positive)",
                d->num_heads, d->num_kv_heads);
  if (d->num_heads % d->num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, "num_heads (%d) is not a multiple of num_kv_heads (%d)",
                d->num_heads, d->num_kv_heads);
  if (d->num_heads / d->num_kv_heads > pa::kMaxGroup)
    return fail(PA_ERR_UNSUPPORTED, "num_heads / num_kv_heads = %d exceeds %d",
                d->num_heads / d->num_kv_heads, pa::kMaxGroup);
  if (d->dtype != PA_F16 && d->dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "dtype %d (expected PA_F16 or PA_BF16)", d->dtype);
  if (d->head_size != 64 && d->head_size != 128)
    return fail(PA_ERR_UNSUPPORTED, "head_size %d (built for 64 and 128)", d->head_size);
  if (d->block_size < pa::kMinBlockSize || d->block_size > pa::kMaxBlockSize ||
      (d->block_size & (d->block_size - 1)) != 0)
    return fail(PA_ERR_UNSUPPORTED, "block_size %d (a power of two in [%d, %d])", d->block_size,
                pa::kMinBlockSize, pa::kMaxBlockSize);
  if (d->num_blocks <= 0) return fail(PA_ERR_INVALID_ARG, "num_blocks = %d", d->num_blocks);
  if (d->max_blocks_per_seq <= 0)
    return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq = %d", d->max_blocks_per_seq);
  if ((long long)d->max_blocks_per_seq * d->block_size > (1LL << 30))
    return fail(PA_ERR_INVALID_ARG, "context bound max_blocks_per_seq * block_size too large");
  if (d->kv_format != PA_KV_NATIVE && d->kv_format != PA_KV_FP8_E4M3)
    return fail(PA_ERR_UNSUPPORTED, "kv_format %d", d->kv_format);
  if (d->kv_layout != PA_KV_SEPARATE && d->kv_layout != PA_KV_JOINT)
    return fail(PA_ERR_INVALID_ARG, "kv_layout %d", d->kv_layout);
  if (d->kv_format == PA_KV_FP8_E4M3) {
    const float inf = __builtin_inff();
    if (!(d->k_scale > 0.f) || !(d->v_scale > 0.f) || d->k_scale == inf || d->v_scale == inf)
      return fail(PA_ERR_INVALID_ARG, "fp8 caches need finite positive k_scale and v_scale");
  }
  return PA_OK;
}

size_t elem_bytes(int32_t dtype) { return dtype == PA_FP8_E4M3 ? 1 : 2; }

// Byte strides of the caches' (block, kv head) tiles for a pa_kv_layout, and
// the joint layout's pointer relation (value tiles follow key tiles).
int cache_strides(int32_t layout, int32_t num_kv_heads, int32_t block_size, size_t row_bytes,
                  const void* key_cache, const void* value_cache, int64_t* block_stride,
                  int64_t* head_stride) {
  const int64_t tile = (int64_t)block_size * (int64_t)row_bytes;
  if (layout == PA_KV_SEPARATE) {
    *head_stride = tile;
    *block_stride = tile * num_kv_heads;
    return PA_OK;
  }
  if (layout != PA_KV_JOINT) return fail(PA_ERR_INVALID_ARG, "kv_layout %d", layout);
  if (static_cast<const char*>(value_cache) != static_cast<const char*>(key_cache) + tile)
    return fail(PA_ERR_INVALID_ARG,
                "joint K/V layout: value_cache must be key_cache + block_size * head_size elements");
  *head_stride = 2 * tile;
  *block_stride = 2 * tile * num_kv_heads;
  return PA_OK;
}

int current_num_cus(int* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(PA_ERR_DEVICE, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return fail(PA_ERR_DEVICE, "device index %d", dev);
  int n = g_num_cus[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return fail(PA_ERR_DEVICE, "cannot query the compute-unit count of device %d", dev);
    g_num_cus[dev].store(n, std::memory_order_relaxed);
  }
  *out = n;
  return PA_OK;
}

// What one call computes beyond its pa_dims: decode (one new token per
// sequence) or multi-query (packed new tokens, up to max_new per sequence).
struct CallShape {
  bool multi = false;
  int32_t rows = 0;     // rows of query / out: num_seqs for decode
  int32_t max_new = 1;  // bound on new tokens per sequence
};

CallShape decode_shape(const pa_dims* d) {
  CallShape c;
  c.rows = d->num_seqs;
  return c;
}

// Workspace of a split plan: fp32 partial outputs, then (m, l) pairs, then
// (longest-first schedule only) the order of the num_seqs * P work units and
// one int32 counter.
struct SplitLayout {
  size_t ml_offset = 0, order_offset = 0, bytes = 0;
};
SplitLayout split_layout(const pa_dims* d, const CallShape& c, int P, bool longest_first) {
  SplitLayout w;
  if (P <= 1) return w;
  const size_t rows = (size_t)c.rows * d->num_heads * P;
  w.ml_offset = align_up(rows * d->head_size * sizeof(float), kWsAlign);
  w.order_offset = align_up(w.ml_offset + rows * 2 * sizeof(float), kWsAlign);
  // (longest first) the order, then the start counter of the later workgroups
  w.bytes = longest_first ? w.order_offset + ((size_t)d->num_seqs * P + 1) * sizeof(int32_t)
                          : w.ml_offset + rows * 2 * sizeof(float);
  return w;
}
size_t split_workspace(const pa_dims* d, const CallShape& c, int P, bool longest_first) {
  return split_layout(d, c, P, longest_first).bytes;
}

// Workspace of an equal-share decode plan with `wgs` workgroups: fp32 partial
// outputs [group head][slots][D], then (m, l) pairs [group head][slots], then
// the tile prefix over sequences (num_seqs + 1 ints).  A piece of item i
// (kv head * num_seqs + sequence) walked by workgroup b sits in slot i + b.
struct SharesLayout {
  size_t ml_offset = 0, pfx_offset = 0, bytes = 0;
  int64_t slots = 0;
};
SharesLayout shares_layout(const pa_dims* d, int wgs) {
  SharesLayout w;
  const size_t group = (size_t)(d->num_heads / d->num_kv_heads);
  w.slots = (int64_t)d->num_seqs * d->num_kv_heads + wgs;
  w.ml_offset = align_up((size_t)w.slots * group * d->head_size * sizeof(float), kWsAlign);
  w.pfx_offset = align_up(w.ml_offset + (size_t)w.slots * group * 2 * sizeof(float), kWsAlign);
  w.bytes = w.pfx_offset + ((size_t)d->num_seqs + 1) * sizeof(int32_t);
  return w;
}

// Equal shares apply to decode on the staged kernel (groups of more than 16
// heads) for batches whose tile prefix fits the kernel's LDS and int32.
bool shares_fit(const pa_dims* d, const CallShape& c, int engine) {
  const int group = d->num_heads / d->num_kv_heads;
  const int64_t tiles = ((int64_t)d->max_blocks_per_seq * d->block_size + 15) / (d->block_size < 16 ? d->block_size : 16);
  return engine == PA_ENGINE_MFMA && !c.multi && pa::mfma_head_tiles(group) > 1 &&
         d->num_seqs <= pa::kStreamMaxSeqs && (int64_t)d->num_seqs * tiles < ((int64_t)1 << 31);
}

// Workgroups of the equal-share kernel one CU holds on the current device
// (the runtime's occupancy of the compiled kernel; looked up once per device
// and configuration), at most what its LDS allows.
std::atomic<int> g_share_occ[kMaxDevices][2][2][3][2];
int share_occupancy(const pa_dims* d, int* out) {
  const int group = d->num_heads / d->num_kv_heads;
  const bool fp8 = d->kv_format == PA_KV_FP8_E4M3;
  const int bound = pa::staged_decode_wgs_per_cu(d->head_size, group, fp8);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(PA_ERR_DEVICE, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return fail(PA_ERR_DEVICE, "device index %d", dev);
  std::atomic<int>& slot = g_share_occ[dev][d->dtype == PA_BF16][d->head_size == 128]
                                      [pa::mfma_head_tiles(group) - 2][fp8];
  int n = slot.load(std::memory_order_relaxed);
  if (n <= 0) {
    if (pa::staged_decode_occupancy(d->dtype == PA_BF16 ? 1 : 0, d->head_size, group, fp8, &n) != hipSuccess || n <= 0)
      return fail(PA_ERR_DEVICE, "cannot query the occupancy of the decode kernel on device %d", dev);
    slot.store(n, std::memory_order_relaxed);
  }
  *out = n < bound ? n : bound;
  return PA_OK;
}

int resolve_engine(const pa_dims* d, const CallShape& c, const pa_opts* o, int* engine) {
  int e = o ? o->engine : PA_ENGINE_AUTO;
  if (e != PA_ENGINE_AUTO && e != PA_ENGINE_VALU && e != PA_ENGINE_MFMA)
    return fail(PA_ERR_INVALID_ARG, "engine %d", e);
  if (c.multi) {  // many query rows per key: always the matrix cores
    if (e == PA_ENGINE_VALU)
      return fail(PA_ERR_UNSUPPORTED, "multi-query attention runs on the MFMA engine only");
    *engine = PA_ENGINE_MFMA;
    return PA_OK;
  }
  if (e == PA_ENGINE_AUTO) {
    const int group = d->num_heads / d->num_kv_heads;
    e = group >= 4 ? PA_ENGINE_MFMA : PA_ENGINE_VALU;
  }
  *engine = e;
  return PA_OK;
}

// Workgroups per (sequence, kv head): query-head chunks on the VALU path, one
// on the MFMA decode path, query-row chunks of 64 rows for multi-query calls.
long long row_chunks(const pa_dims* d, const CallShape& c, int engine) {
  const int group = d->num_heads / d->num_kv_heads;
  if (c.multi)
    return ((long long)c.max_new * group + pa::kPrefillRows - 1) / pa::kPrefillRows;
  if (engine == PA_ENGINE_VALU)
    return (group + pa::valu_heads_per_workgroup(group) - 1) / pa::valu_heads_per_workgroup(group);
  return 1;
}

// The planner.  `unlimited` ignores ws_bytes (used for sizing).
int make_plan(const pa_dims* d, const CallShape& c, size_t ws_bytes, const pa_opts* o,
              bool unlimited, pa_plan* p) {
  int st = check_dims(d);
  if (st) return st;
  int engine = 0;
  if ((st = resolve_engine(d, c, o, &engine))) return st;
  const int maxb = d->max_blocks_per_seq;
  const int forced = o ? o->partition_size : 0;
  const int group = d->num_heads / d->num_kv_heads;
  const int schedule = o ? o->schedule : PA_SCHEDULE_AUTO;
  if (schedule != PA_SCHEDULE_AUTO && schedule != PA_SCHEDULE_GRID &&
      schedule != PA_SCHEDULE_LONGEST_FIRST && schedule != PA_SCHEDULE_EQUAL_SHARES)
    return fail(PA_ERR_INVALID_ARG, "schedule %d", schedule);
  // Longest-first ordering applies to split decode plans on the MFMA engine;
  // automatic for groups of more than 16 heads that do not take equal shares,
  // on request otherwise.
  const bool longest_first =
      engine == PA_ENGINE_MFMA && !c.multi &&
      (schedule == PA_SCHEDULE_LONGEST_FIRST ||
       ((schedule == PA_SCHEDULE_AUTO || schedule == PA_SCHEDULE_EQUAL_SHARES) &&
        pa::mfma_head_tiles(group) > 1));
  int P = 1, PB = maxb;

  if (forced == -1) {
    P = 1;
  } else if (forced > 0) {
    if (forced % d->block_size != 0)
      return fail(PA_ERR_INVALID_ARG, "partition_size %d is not a multiple of block_size %d",
                  forced, d->block_size);
    PB = forced / d->block_size;
    P = (maxb + PB - 1) / PB;
    if (P > 65535) return fail(PA_ERR_INVALID_ARG, "partition_size %d gives %d partitions", forced, P);
    if (P > 1 && !unlimited && split_workspace(d, c, P, longest_first) > ws_bytes)
      return fail(PA_ERR_WORKSPACE, "forced partition_size %d needs %zu workspace bytes, got %zu",
                  forced, split_workspace(d, c, P, longest_first), ws_bytes);
  } else if (forced == 0) {
    int cus = o ? o->num_cus : 0;
    if (cus < 0) return fail(PA_ERR_INVALID_ARG, "num_cus = %d", cus);
    if (cus == 0 && (st = current_num_cus(&cus))) return st;
    const long long units = (long long)d->num_seqs * d->num_kv_heads * row_chunks(d, c, engine);
    const bool one_tile = engine == PA_ENGINE_MFMA && !c.multi && pa::mfma_head_tiles(group) == 1;
    const bool fp8 = d->kv_format == PA_KV_FP8_E4M3;
    const long long target = (long long)(engine == PA_ENGINE_VALU ? kTargetGroupsPerCuValu
                                         : one_tile && fp8         ? kTargetGroupsPerCuOneTileFp8
                                         : one_tile                ? kTargetGroupsPerCuOneTile
                                                                   : kTargetGroupsPerCu) * cus;
    const int min_tokens = one_tile && !fp8 ? kMinPartitionTokensOneTile : kMinPartitionTokens;
    const int min_pb = min_tokens / d->block_size > 1 ? min_tokens / d->block_size : 1;
    const bool split = units > 0 && units < target && maxb > min_pb;
    // Equal shares (groups of more than 16 heads, on request, or where the
    // auto plan would split a batch of fewer (kv head, sequence) items than
    // the CUs hold workgroups): as many workgroups as the CUs hold at once,
    // each walking an equal share of the batch's tiles.  With at least as
    // many items as workgroup slots every slot starts on a whole item and
    // longest-first partitions balance the rest without cutting items at
    // arbitrary tiles.  Measured, ragged 64..8192 ALiBi batches, graph
    // replay, longest first -> equal shares: 48-head groups batch 32 35.7 ->
    // 28.7 us; 32-head groups batch 64 41.2 -> 38.9 us, batch 256 112.8 ->
    // 109.4 us; 64-head groups batch 256 140.5 -> 125.7 us (FP8 138.3 ->
    // 107.7); but 48-head groups at batch 256 (256 items, one workgroup per
    // CU) 104 -> 109.5 us, so these keep partitions.
    const int wgs_per_cu = pa::staged_decode_wgs_per_cu(d->head_size, group, fp8);
    if (shares_fit(d, c, engine) &&
        (schedule == PA_SCHEDULE_EQUAL_SHARES ||
         (schedule == PA_SCHEDULE_AUTO && split && units < (long long)cus * wgs_per_cu))) {
      const int wgs = cus * wgs_per_cu;
      const size_t need = shares_layout(d, wgs).bytes;
      if (unlimited || need <= ws_bytes) {
        p->num_partitions = wgs;
        p->partition_size = 0;
        p->engine = engine;
        p->schedule = PA_SCHEDULE_EQUAL_SHARES;
        p->workspace_bytes = need;
        return PA_OK;
      }
    }
    if (split) {
      long long want = (target + units - 1) / units;
      PB = (int)((maxb + want - 1) / want);
      if (PB < min_pb) PB = min_pb;
      P = (maxb + PB - 1) / PB;
      // shrink to what the workspace holds
      while (P > 1 && !unlimited && split_workspace(d, c, P, longest_first) > ws_bytes) {
        PB *= 2;
        P = (maxb + PB - 1) / PB;
      }
    }
  } else {
    return fail(PA_ERR_INVALID_ARG, "partition_size %d (use 0, -1 or a positive multiple of %d)",
                forced, d->block_size);
  }
  if (P <= 1) {
    P = 1;
    PB = maxb;
  }
  p->num_partitions = P;
  p->partition_size = PB * d->block_size;
  p->engine = engine;
  p->schedule = P > 1 && longest_first ? PA_SCHEDULE_LONGEST_FIRST : PA_SCHEDULE_GRID;
  p->workspace_bytes = split_workspace(d, c, P, longest_first);
  return PA_OK;
}

// Validation, planning and launch shared by the decode and multi-query calls.
int run_attention(void* out, const void* query, const void* key_cache, const void* value_cache,
                  const int32_t* block_tables, const int32_t* context_lens,
                  const int32_t* query_start, const CallShape& c, float scale, int32_t block_size,
                  const float* alibi_slopes, pa_stream_t stream, const pa_dims* dims,
                  void* workspace, size_t workspace_bytes, const pa_opts* opts) {
  int st = check_dims(dims);
  if (st) return st;
  if (block_size != dims->block_size)
    return fail(PA_ERR_INVALID_ARG, "block_size argument %d differs from dims->block_size %d",
                block_size, dims->block_size);
  if (!(scale == scale) || scale == __builtin_inff() || scale == -__builtin_inff())
    return fail(PA_ERR_INVALID_ARG, "scale is not finite");
  if (c.multi) {
    if (c.rows < 0 || c.max_new < 0)
      return fail(PA_ERR_INVALID_ARG, "num_query_tokens %d, max_query_len %d", c.rows, c.max_new);
    if (c.max_new > 65535)
      return fail(PA_ERR_INVALID_ARG, "max_query_len %d exceeds 65535", c.max_new);
  }
  if (dims->num_seqs == 0 || c.rows == 0 || c.max_new == 0) return ok();
  if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens ||
      (c.multi && !query_start))
    return fail(PA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned(out, 16) || !aligned(query, 16) || !aligned(key_cache, 16) ||
      !aligned(value_cache, 16))
    return fail(PA_ERR_ALIGNMENT, "out, query and caches must be 16-byte aligned");
  if (!aligned(block_tables, 4) || !aligned(context_lens, 4) ||
      (alibi_slopes && !aligned(alibi_slopes, 4)) || (query_start && !aligned(query_start, 4)))
    return fail(PA_ERR_ALIGNMENT,
                "block_tables, context_lens, query_start_loc and alibi_slopes must be 4-byte aligned");

  const bool kv_fp8 = dims->kv_format == PA_KV_FP8_E4M3;
  int64_t kv_block_stride = 0, kv_head_stride = 0;
  if ((st = cache_strides(dims->kv_layout, dims->num_kv_heads, dims->block_size,
                          (size_t)dims->head_size * (kv_fp8 ? 1 : 2), key_cache, value_cache,
                          &kv_block_stride, &kv_head_stride)))
    return st;

  pa_plan plan;
  if ((st = make_plan(dims, c, workspace ? workspace_bytes : 0, opts, false, &plan))) return st;
  const bool shares = plan.schedule == PA_SCHEDULE_EQUAL_SHARES;
  if (plan.num_partitions > 1 || shares) {
    if (!workspace) return fail(PA_ERR_WORKSPACE, "split plan needs a workspace");
    if (!aligned(workspace, kWsAlign))
      return fail(PA_ERR_ALIGNMENT, "workspace must be %zu-byte aligned", kWsAlign);
  }

  pa::DecodeArgs a;
  a.out = out;
  a.q = query;
  a.k_cache = key_cache;
  a.v_cache = value_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.alibi = alibi_slopes;
  a.kv_block_stride = kv_block_stride;
  a.kv_head_stride = kv_head_stride;
  // the key scale folds into the logit scale, the value scale into the output
  a.scale_log2 = scale * 1.4426950408889634f * (kv_fp8 ? dims->k_scale : 1.f);
  a.v_scale = kv_fp8 ? dims->v_scale : 1.f;
  a.num_seqs = dims->num_seqs;
  a.num_heads = dims->num_heads;
  a.num_kv_heads = dims->num_kv_heads;
  a.max_blocks_per_seq = dims->max_blocks_per_seq;
  a.group = dims->num_heads / dims->num_kv_heads;
  a.num_partitions = plan.num_partitions;
  a.partition_blocks = plan.partition_size / dims->block_size;
  a.block_size = dims->block_size;
  a.block_shift = __builtin_ctz((unsigned)dims->block_size);
  a.query_start = c.multi ? query_start : nullptr;
  a.max_new_tokens = c.max_new;
  a.row_chunks = (int32_t)(plan.engine == PA_ENGINE_MFMA ? row_chunks(dims, c, plan.engine) : 1);
  a.ws_o = nullptr;
  a.ws_ml = nullptr;
  a.unit_order = nullptr;
  const bool longest_first = plan.schedule == PA_SCHEDULE_LONGEST_FIRST;
  int32_t* order = nullptr;
  if (shares) {
    // launched: the CUs the plan counted times what one CU holds of this kernel
    int occ = 0;
    if ((st = share_occupancy(dims, &occ))) return st;
    const SharesLayout w = shares_layout(dims, plan.num_partitions);
    a.ws_o = static_cast<float*>(workspace);
    a.ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + w.ml_offset);
    a.ws_pfx = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + w.pfx_offset);
    a.num_slots = (int32_t)w.slots;
    const int group = dims->num_heads / dims->num_kv_heads;
    a.stream_wgs = plan.num_partitions / pa::staged_decode_wgs_per_cu(dims->head_size, group, kv_fp8) * occ;
    a.piece_cost = pa::staged_piece_cost(occ, kv_fp8);
    a.num_partitions = 1;
  } else if (plan.num_partitions > 1) {
    const SplitLayout w = split_layout(dims, c, plan.num_partitions, longest_first);
    a.ws_o = static_cast<float*>(workspace);
    a.ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + w.ml_offset);
    if (longest_first) order = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + w.order_offset);
  }
  if ((long long)dims->num_kv_heads * a.row_chunks > 0x7fffffffLL)
    return fail(PA_ERR_INVALID_ARG, "too many query rows per sequence");

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (order != nullptr) {
    if ((long long)dims->num_kv_heads * a.row_chunks * dims->num_seqs * plan.num_partitions > 0x7fffffffLL)
      return fail(PA_ERR_INVALID_ARG, "too many work units for a longest-first schedule");
    // staged decode with one workgroup per CU: the workgroups after the first
    // round take their places in the order by start (a counter after the
    // order); with several per CU it measured no faster (32-head groups) or
    // 1% slower (64-head groups)
    const int group = dims->num_heads / dims->num_kv_heads;
    if (plan.engine == PA_ENGINE_MFMA && !c.multi && pa::mfma_head_tiles(group) > 1) {
      int occ = 0, cus = 0;
      if ((st = share_occupancy(dims, &occ)) || (st = current_num_cus(&cus))) return st;
      if (occ == 1) {
        a.ticket = order + (size_t)dims->num_seqs * plan.num_partitions;
        a.static_wgs = cus;
      }
    }
    hipError_t e = pa::launch_unit_order(a, order, s);
    if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "schedule launch: %s", hipGetErrorString(e));
    a.unit_order = order;
  }
  hipError_t e =
      plan.engine != PA_ENGINE_MFMA ? pa::launch_decode_valu(a, dims->dtype, dims->head_size, kv_fp8, s)
      : c.multi && pa::prefill_mfma32_supported(dims->head_size, kv_fp8, dims->block_size)
          ? pa::launch_prefill_mfma32(a, dims->dtype, s)
          : pa::launch_decode_mfma(a, dims->dtype, dims->head_size, kv_fp8, s);
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "attention launch: %s", hipGetErrorString(e));
  if (plan.num_partitions > 1 || shares) {
    e = pa::launch_partition_reduce(a, dims->dtype, dims->head_size, s);
    if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "reduce launch: %s", hipGetErrorString(e));
  }
  return ok();
}

}  // namespace

extern "C" {

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_ALIGNMENT: return "misaligned pointer";
    case PA_ERR_WORKSPACE: return "workspace too small";
    case PA_ERR_LAUNCH: return "kernel launch failed";
    case PA_ERR_DEVICE: return "device query failed";
    default: return "unknown status";
  }
}

const char* pa_last_error(void) { return g_last_error; }

int paged_attention_plan(const pa_dims* dims, size_t workspace_bytes, const pa_opts* opts,
                         pa_plan* plan) {
  if (plan == nullptr) return fail(PA_ERR_INVALID_ARG, "plan is NULL");
  pa_plan p;
  const int st = make_plan(dims, decode_shape(dims), workspace_bytes, opts, false, &p);
  if (st) return st;
  *plan = p;
  return ok();
}

size_t paged_attention_workspace_bytes(const pa_dims* dims, const pa_opts* opts) {
  pa_plan p;
  if (!dims || make_plan(dims, decode_shape(dims), 0, opts, true, &p)) return 0;
  return p.workspace_bytes;
}

int paged_attention_decode(void* out, const void* query, const void* key_cache,
                           const void* value_cache, const int32_t* block_tables,
                           const int32_t* context_lens, float scale, int32_t block_size,
                           const float* alibi_slopes, pa_stream_t stream, const pa_dims* dims,
                           void* workspace, size_t workspace_bytes, const pa_opts* opts) {
  if (dims == nullptr) return fail(PA_ERR_INVALID_ARG, "dims is NULL");
  return run_attention(out, query, key_cache, value_cache, block_tables, context_lens, nullptr,
                       decode_shape(dims), scale, block_size, alibi_slopes, stream, dims,
                       workspace, workspace_bytes, opts);
}

int paged_attention_decode_noalloc(void* out, const void* query, const void* key_cache,
                                   const void* value_cache, const int32_t* block_tables,
                                   const int32_t* context_lens, float scale, int32_t block_size,
                                   const float* alibi_slopes, pa_stream_t stream,
                                   const pa_dims* dims, const pa_opts* opts) {
  if (dims == nullptr) return fail(PA_ERR_INVALID_ARG, "dims is NULL");
  int st = check_dims(dims);
  if (st) return st;
  if (dims->num_seqs == 0) return ok();
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(PA_ERR_DEVICE, "hipGetDevice failed");
  void* scratch = nullptr;
  const hipError_t e = pa::noalloc_scratch(dev, &scratch);
  if (e != hipSuccess)
    return fail(PA_ERR_DEVICE, "scratch address on device %d: %s", dev, hipGetErrorString(e));
  st = run_attention(out, query, key_cache, value_cache, block_tables, context_lens, nullptr,
                     decode_shape(dims), scale, block_size, alibi_slopes, stream, dims, scratch,
                     PA_NOALLOC_SCRATCH_BYTES, opts);
  if (st == PA_ERR_WORKSPACE) {
    char detail[sizeof(g_last_error)];
    std::memcpy(detail, g_last_error, sizeof(detail));
    return fail(PA_ERR_WORKSPACE,
                "the forced partition_size needs more than the %zu-byte scratch of the "
                "allocation-free entry point (%s)",
                (size_t)PA_NOALLOC_SCRATCH_BYTES, detail);
  }
  return st;
}

static CallShape prefill_shape(int32_t num_query_tokens, int32_t max_query_len) {
  CallShape c;
  c.multi = true;
  c.rows = num_query_tokens;
  c.max_new = max_query_len;
  return c;
}

int paged_attention_prefill_plan(const pa_dims* dims, int32_t num_query_tokens,
                                 int32_t max_query_len, size_t workspace_bytes,
                                 const pa_opts* opts, pa_plan* plan) {
  if (plan == nullptr) return fail(PA_ERR_INVALID_ARG, "plan is NULL");
  if (num_query_tokens < 0 || max_query_len < 0)
    return fail(PA_ERR_INVALID_ARG, "num_query_tokens %d, max_query_len %d", num_query_tokens,
                max_query_len);
  pa_plan p;
  const int st = make_plan(dims, prefill_shape(num_query_tokens, max_query_len), workspace_bytes,
                           opts, false, &p);
  if (st) return st;
  *plan = p;
  return ok();
}

size_t paged_attention_prefill_workspace_bytes(const pa_dims* dims, int32_t num_query_tokens,
                                               int32_t max_query_len, const pa_opts* opts) {
  pa_plan p;
  if (!dims || num_query_tokens < 0 || max_query_len < 0 ||
      make_plan(dims, prefill_shape(num_query_tokens, max_query_len), 0, opts, true, &p))
    return 0;
  return p.workspace_bytes;
}

int paged_attention_prefill(void* out, const void* query, const void* key_cache,
                            const void* value_cache, const int32_t* block_tables,
                            const int32_t* context_lens, const int32_t* query_start_loc,
                            int32_t num_query_tokens, int32_t max_query_len, float scale,
                            int32_t block_size, const float* alibi_slopes, pa_stream_t stream,
                            const pa_dims* dims, void* workspace, size_t workspace_bytes,
                            const pa_opts* opts) {
  if (dims == nullptr) return fail(PA_ERR_INVALID_ARG, "dims is NULL");
  return run_attention(out, query, key_cache, value_cache, block_tables, context_lens,
                       query_start_loc, prefill_shape(num_query_tokens, max_query_len), scale,
                       block_size, alibi_slopes, stream, dims, workspace, workspace_bytes, opts);
}

// Shared checks of the two row-copy entry points.
static int check_copy_args(int32_t num_tokens, int32_t num_kv_heads, int32_t head_size,
                    int32_t block_size, int32_t num_blocks, int32_t dtype) {
  if (dtype != PA_F16 && dtype != PA_BF16 && dtype != PA_FP8_E4M3)
    return fail(PA_ERR_UNSUPPORTED, "dtype %d", dtype);
  if (num_tokens < 0 || num_kv_heads <= 0 || block_size <= 0 || num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARG, "num_tokens %d, num_kv_heads %d, block_size %d, num_blocks %d",
                num_tokens, num_kv_heads, block_size, num_blocks);
  const long long row_bytes = (long long)head_size * elem_bytes(dtype);
  if (head_size <= 0 || row_bytes % 16 != 0)
    return fail(PA_ERR_UNSUPPORTED, "head_size %d (a row must be a multiple of 16 bytes)", head_size);
  // the kernels index 16-byte pieces with 32-bit counters that step by up to
  // 2^24 (their grid): below 2^31 pieces no step can wrap around
  if ((unsigned long long)num_tokens * num_kv_heads * (row_bytes / 16) >= (1ULL << 31))
    return fail(PA_ERR_INVALID_ARG, "num_tokens * num_kv_heads * head_size too large (2^31 16-byte pieces or more)");
  if ((unsigned long long)num_blocks * block_size > 0x7fffffffULL)
    return fail(PA_ERR_INVALID_ARG, "num_blocks * block_size exceeds the int32 slot range");
  return PA_OK;
}

int paged_kv_cache_write(void* key_cache, void* value_cache, const void* key, const void* value,
                         const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                         int32_t head_size, int32_t block_size, int32_t num_blocks, int32_t dtype,
                         int32_t kv_layout, pa_stream_t stream) {
  int st = check_copy_args(num_tokens, num_kv_heads, head_size, block_size, num_blocks, dtype);
  if (st) return st;
  if (kv_layout != PA_KV_SEPARATE && kv_layout != PA_KV_JOINT)
    return fail(PA_ERR_INVALID_ARG, "kv_layout %d", kv_layout);
  if (num_tokens == 0) return ok();
  if (!key_cache || !value_cache || !key || !value || !slot_mapping)
    return fail(PA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned(key_cache, 16) || !aligned(value_cache, 16) || !aligned(key, 16) ||
      !aligned(value, 16) || !aligned(slot_mapping, 4))
    return fail(PA_ERR_ALIGNMENT, "16-bit tensors must be 16-byte aligned, slot_mapping 4-byte");
  const size_t row_bytes = (size_t)head_size * elem_bytes(dtype);
  int64_t bstride = 0, hstride = 0;
  if ((st = cache_strides(kv_layout, num_kv_heads, block_size, row_bytes, key_cache, value_cache,
                          &bstride, &hstride)))
    return st;
  const hipError_t e = pa::launch_cache_write(key_cache, value_cache, key, value, slot_mapping,
                                              num_tokens, num_kv_heads, (int32_t)row_bytes,
                                              block_size, bstride, hstride,
                                              reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "cache write launch: %s", hipGetErrorString(e));
  return ok();
}

int gather_cached_kv(void* key_out, void* value_out, const void* key_cache,
                     const void* value_cache, const int32_t* slot_mapping, int32_t num_tokens,
                     int32_t num_kv_heads, int32_t head_size, int32_t block_size,
                     int32_t num_blocks, int32_t dtype, int32_t kv_layout, pa_stream_t stream) {
  int st = check_copy_args(num_tokens, num_kv_heads, head_size, block_size, num_blocks, dtype);
  if (st) return st;
  if (kv_layout != PA_KV_SEPARATE && kv_layout != PA_KV_JOINT)
    return fail(PA_ERR_INVALID_ARG, "kv_layout %d", kv_layout);
  if (num_tokens == 0) return ok();
  if (!key_out || !value_out || !key_cache || !value_cache || !slot_mapping)
    return fail(PA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned(key_out, 16) || !aligned(value_out, 16) || !aligned(key_cache, 16) ||
      !aligned(value_cache, 16) || !aligned(slot_mapping, 4))
    return fail(PA_ERR_ALIGNMENT, "16-bit tensors must be 16-byte aligned, slot_mapping 4-byte");
  const size_t row_bytes = (size_t)head_size * elem_bytes(dtype);
  int64_t bstride = 0, hstride = 0;
  if ((st = cache_strides(kv_layout, num_kv_heads, block_size, row_bytes, key_cache, value_cache,
                          &bstride, &hstride)))
    return st;
  const hipError_t e = pa::launch_gather(key_out, value_out, key_cache, value_cache, slot_mapping,
                                         num_tokens, num_kv_heads, (int32_t)row_bytes, block_size,
                                         bstride, hstride, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "gather launch: %s", hipGetErrorString(e));
  return ok();
}

size_t pa_stream_read_sink_bytes(size_t bytes) { return (size_t)pa::stream_read_grid(bytes) * 16; }

int pa_share_occupancy(const pa_dims* dims, int32_t* table_wgs, int32_t* device_wgs,
                       int32_t* piece_cost) {
  int st = check_dims(dims);
  if (st) return st;
  if (!table_wgs || !device_wgs || !piece_cost) return fail(PA_ERR_INVALID_ARG, "a required pointer is NULL");
  CallShape c = decode_shape(dims);
  if (!shares_fit(dims, c, PA_ENGINE_MFMA))
    return fail(PA_ERR_INVALID_ARG, "these dims do not take equal shares");
  const int group = dims->num_heads / dims->num_kv_heads;
  const bool fp8 = dims->kv_format == PA_KV_FP8_E4M3;
  int n = 0;
  if (pa::staged_decode_occupancy(dims->dtype == PA_BF16 ? 1 : 0, dims->head_size, group, fp8, &n) !=
      hipSuccess)
    return fail(PA_ERR_DEVICE, "occupancy query failed");
  *table_wgs = pa::staged_decode_wgs_per_cu(dims->head_size, group, fp8);
  *device_wgs = n;
  *piece_cost = pa::staged_piece_cost(n < *table_wgs ? n : *table_wgs, fp8);
  return ok();
}

int pa_stream_read_probe(const void* src, size_t bytes, size_t run_bytes, void* sink,
                         size_t sink_bytes, pa_stream_t stream) {
  auto pow2 = [](size_t x) { return x != 0 && (x & (x - 1)) == 0; };
  if (bytes % 16 != 0) return fail(PA_ERR_INVALID_ARG, "bytes %zu is not a multiple of 16", bytes);
  if (run_bytes != 0 && (!pow2(run_bytes) || run_bytes < 1024 || bytes % run_bytes != 0 ||
                         !pow2(bytes / run_bytes)))
    return fail(PA_ERR_INVALID_ARG,
                "run_bytes %zu: a power of two >= 1024 with bytes / run_bytes a power of two", run_bytes);
  if (bytes == 0) return ok();
  if (!src || !sink) return fail(PA_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!aligned(src, 16) || !aligned(sink, 16))
    return fail(PA_ERR_ALIGNMENT, "src and sink must be 16-byte aligned");
  if (sink_bytes < pa_stream_read_sink_bytes(bytes))
    return fail(PA_ERR_INVALID_ARG, "sink needs %zu bytes, got %zu", pa_stream_read_sink_bytes(bytes),
                sink_bytes);
  const hipError_t e =
      pa::launch_stream_read(src, bytes, run_bytes, sink, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "probe launch: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
