// Host-layer checks of the C ABI built with the stubs of hip_stubs.cpp (no
// GPU): validation, the planner and the launch arguments each call sets up,
// run under AddressSanitizer and UndefinedBehaviorSanitizer.  Device pointers
// are fake addresses that the host layer never dereferences.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>

#include "hip_stubs.h"
#include "paged_attention.h"
#include "measure.h"

static int g_fail = 0;
#define CHECK(c)                                                                 \
  do {                                                                           \
    if (!(c)) {                                                                  \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
      ++g_fail;                                                                  \
    }                                                                            \
  } while (0)

static char* const FAKE = reinterpret_cast<char*>(0x10000000);

static pa_dims dims(int S, int Hq, int Hkv, int D = 128, int BS = 16, int NB = 65536, int MAXB = 256,
                    int dtype = PA_BF16) {
  pa_dims d;
  std::memset(&d, 0, sizeof(d));
  d.num_seqs = S;
  d.num_heads = Hq;
  d.num_kv_heads = Hkv;
  d.head_size = D;
  d.block_size = BS;
  d.num_blocks = NB;
  d.max_blocks_per_seq = MAXB;
  d.dtype = dtype;
  return d;
}

static int decode(const pa_dims& d, const void* k, const void* v, void* ws = nullptr,
                  size_t ws_bytes = 0, const pa_opts* o = nullptr) {
  return paged_attention_decode(FAKE, FAKE, k, v, reinterpret_cast<const int32_t*>(FAKE),
                                reinterpret_cast<const int32_t*>(FAKE), 0.088f, d.block_size, nullptr,
                                nullptr, &d, ws, ws_bytes, o);
}

static bool near(float a, float b) { return std::fabs(a - b) <= 1e-6f * std::fabs(b); }

static void headline_single_pass() {
  g_launches.clear();
  pa_dims d = dims(256, 64, 8);
  CHECK(decode(d, FAKE, FAKE + (1 << 30)) == PA_OK);
  CHECK(g_launches.size() == 1);
  const Launch& l = g_launches[0];
  CHECK(std::strcmp(l.kind, "mfma") == 0);
  CHECK(l.a.num_partitions == 1 && l.a.group == 8 && l.a.row_chunks == 1);
  CHECK(l.a.kv_block_stride == 8 * 16 * 128 * 2 && l.a.kv_head_stride == 16 * 128 * 2);
  CHECK(near(l.a.scale_log2, 0.088f * 1.4426950408889634f));
  CHECK(l.a.query_start == nullptr && l.a.unit_order == nullptr && l.a.ws_o == nullptr);
}

static void joint_layout() {
  g_launches.clear();
  pa_dims d = dims(256, 64, 8);
  d.kv_layout = PA_KV_JOINT;
  const int tile = 16 * 128 * 2;
  CHECK(decode(d, FAKE, FAKE + tile) == PA_OK);
  CHECK(g_launches.size() == 1);
  CHECK(g_launches[0].a.kv_block_stride == 2 * 8 * tile && g_launches[0].a.kv_head_stride == 2 * tile);
  CHECK(decode(d, FAKE, FAKE + 2 * tile) == PA_ERR_INVALID_ARG);
  CHECK(std::string(pa_last_error()).find("joint") != std::string::npos);
  CHECK(g_launches.size() == 1);  // nothing launched by the failed call
  d.kv_layout = 5;
  CHECK(decode(d, FAKE, FAKE + tile) == PA_ERR_INVALID_ARG);
}

static void split_small_batch() {
  g_launches.clear();
  pa_dims d = dims(1, 64, 8);
  const size_t ws = paged_attention_workspace_bytes(&d, nullptr);
  CHECK(ws > 0);
  char* w = FAKE + (1 << 20);
  CHECK(decode(d, FAKE, FAKE + (1 << 28), w, ws) == PA_OK);
  CHECK(g_launches.size() == 2);
  CHECK(std::strcmp(g_launches[0].kind, "mfma") == 0 && std::strcmp(g_launches[1].kind, "reduce") == 0);
  const pa::DecodeArgs& a = g_launches[0].a;
  CHECK(a.num_partitions == 32 && a.partition_blocks == 8);
  CHECK(reinterpret_cast<char*>(a.ws_o) == w);
  const char* ml = reinterpret_cast<const char*>(a.ws_ml);
  CHECK(ml > w && ml + 64 * 32 * 8 <= w + ws);
  // an undersized workspace gives fewer partitions, never an error
  g_launches.clear();
  CHECK(decode(d, FAKE, FAKE + (1 << 28), w, ws / 3) == PA_OK);
  CHECK(!g_launches.empty() && g_launches[0].a.num_partitions < 32);
  // a forced split without a workspace fails before launching anything
  g_launches.clear();
  pa_opts o = {128, PA_ENGINE_AUTO, 0, PA_SCHEDULE_AUTO};
  CHECK(decode(d, FAKE, FAKE + (1 << 28), nullptr, 0, &o) == PA_ERR_WORKSPACE);
  CHECK(g_launches.empty());
}

static void mqa_longest_first() {
  g_launches.clear();
  pa_dims d = dims(256, 48, 1, 128, 16, 70000, 512, PA_F16);
  const pa_opts o = {0, PA_ENGINE_AUTO, 0, PA_SCHEDULE_LONGEST_FIRST};
  const size_t ws = paged_attention_workspace_bytes(&d, &o);
  char* w = FAKE + (1 << 20);
  const float slopes = 0.f;
  CHECK(paged_attention_decode(FAKE, FAKE, FAKE, FAKE + (1 << 28), reinterpret_cast<const int32_t*>(FAKE),
                               reinterpret_cast<const int32_t*>(FAKE), 0.088f, 16,
                               reinterpret_cast<const float*>(FAKE + 64), nullptr, &d, w, ws,
                               &o) == PA_OK);
  (void)slopes;
  CHECK(g_launches.size() == 3);
  CHECK(std::strcmp(g_launches[0].kind, "order") == 0);
  CHECK(std::strcmp(g_launches[1].kind, "mfma") == 0);
  CHECK(std::strcmp(g_launches[2].kind, "reduce") == 0);
  const pa::DecodeArgs& a = g_launches[1].a;
  CHECK(a.num_partitions == 2 && a.group == 48);
  CHECK(a.unit_order == g_launches[0].ptr);
  const char* order = reinterpret_cast<const char*>(a.unit_order);
  CHECK(order >= w && order + 256 * 2 * 4 <= w + ws);
  // one 12-wave workgroup per CU: the workgroups after the first round take
  // their places from the counter right after the order, in the workspace
  CHECK(a.ticket == a.unit_order + 256 * 2 && reinterpret_cast<const char*>(a.ticket + 1) <= w + ws);
  CHECK(a.static_wgs == kStubCus);
  CHECK(a.alibi == reinterpret_cast<const float*>(FAKE + 64));
}

static void mqa_equal_shares() {
  g_launches.clear();
  pa_dims d = dims(64, 48, 1, 128, 16, 70000, 512, PA_F16);  // fewer items than CUs: equal shares
  const size_t ws = paged_attention_workspace_bytes(&d, nullptr);
  char* w = FAKE + (1 << 20);
  CHECK(paged_attention_decode(FAKE, FAKE, FAKE, FAKE + (1 << 28), reinterpret_cast<const int32_t*>(FAKE),
                               reinterpret_cast<const int32_t*>(FAKE), 0.088f, 16, nullptr, nullptr, &d, w,
                               ws, nullptr) == PA_OK);
  CHECK(g_launches.size() == 2);
  CHECK(std::strcmp(g_launches[0].kind, "mfma") == 0);
  CHECK(std::strcmp(g_launches[1].kind, "reduce") == 0);
  const pa::DecodeArgs& a = g_launches[0].a;
  // one workgroup per CU; slots for 64 items and 256 workgroups
  CHECK(a.stream_wgs == kStubCus && a.num_slots == 64 + kStubCus && a.unit_order == nullptr);
  CHECK(a.piece_cost == 24);
  CHECK(g_launches[1].a.stream_wgs == a.stream_wgs && g_launches[1].a.ws_pfx == a.ws_pfx);
  const char* o = reinterpret_cast<const char*>(a.ws_o);
  const char* ml = reinterpret_cast<const char*>(a.ws_ml);
  const char* pfx = reinterpret_cast<const char*>(a.ws_pfx);
  CHECK(o == w && ml >= o + (size_t)a.num_slots * 48 * 128 * 4 && pfx >= ml + (size_t)a.num_slots * 48 * 8);
  CHECK(pfx + 65 * 4 <= w + ws);
  // too little workspace for the shares: a partitioned plan that fits
  g_launches.clear();
  CHECK(paged_attention_decode(FAKE, FAKE, FAKE, FAKE + (1 << 28), reinterpret_cast<const int32_t*>(FAKE),
                               reinterpret_cast<const int32_t*>(FAKE), 0.088f, 16, nullptr, nullptr, &d, w,
                               ws - 1, nullptr) == PA_OK);
  for (const Launch& l : g_launches) CHECK(l.a.stream_wgs == 0);
}

static void fp8_cache() {
  g_launches.clear();
  pa_dims d = dims(256, 64, 8);
  d.kv_format = PA_KV_FP8_E4M3;
  d.k_scale = 0.5f;
  d.v_scale = 0.25f;
  CHECK(decode(d, FAKE, FAKE + (1 << 28)) == PA_OK);
  CHECK(g_launches.size() == 1 && g_launches[0].kv_fp8);
  const pa::DecodeArgs& a = g_launches[0].a;
  CHECK(near(a.scale_log2, 0.088f * 1.4426950408889634f * 0.5f) && a.v_scale == 0.25f);
  CHECK(a.kv_block_stride == 8 * 16 * 128 && a.kv_head_stride == 16 * 128);
  d.k_scale = 0.f;
  CHECK(decode(d, FAKE, FAKE + (1 << 28)) == PA_ERR_INVALID_ARG);
}

static void mha_valu_and_forced_engines() {
  g_launches.clear();
  pa_dims d = dims(8, 40, 40, 128, 16, 4096, 16, PA_F16);
  CHECK(decode(d, FAKE, FAKE + (1 << 28)) == PA_OK);
  CHECK(g_launches.size() == 1 && std::strcmp(g_launches[0].kind, "valu") == 0);
  pa_opts o = {-1, PA_ENGINE_MFMA, 0, PA_SCHEDULE_AUTO};
  CHECK(decode(d, FAKE, FAKE + (1 << 28), nullptr, 0, &o) == PA_OK);
  CHECK(g_launches.size() == 2 && std::strcmp(g_launches[1].kind, "mfma") == 0);
  o.engine = 7;
  CHECK(decode(d, FAKE, FAKE + (1 << 28), nullptr, 0, &o) == PA_ERR_INVALID_ARG);
}

static void prefill() {
  g_launches.clear();
  pa_dims d = dims(4, 64, 8);
  const int T = 2048, maxq = 512;
  const size_t ws = paged_attention_prefill_workspace_bytes(&d, T, maxq, nullptr);
  char* w = FAKE + (1 << 20);
  CHECK(paged_attention_prefill(FAKE, FAKE, FAKE, FAKE + (1 << 28), reinterpret_cast<const int32_t*>(FAKE),
                                reinterpret_cast<const int32_t*>(FAKE),
                                reinterpret_cast<const int32_t*>(FAKE + 128), T, maxq, 0.088f, 16,
                                nullptr, nullptr, &d, w, ws, nullptr) == PA_OK);
  // bf16, head size 128, 16-token blocks: the 32 x 32 tile kernel
  CHECK(!g_launches.empty() && std::strcmp(g_launches[0].kind, "prefill32") == 0);
  const pa::DecodeArgs& a = g_launches[0].a;
  CHECK(a.query_start == reinterpret_cast<const int32_t*>(FAKE + 128));
  CHECK(a.max_new_tokens == maxq && a.row_chunks == (maxq * 8 + 127) / 128);
  // 8-token blocks and head size 64 stay on the general kernel
  for (int variant = 0; variant < 2; ++variant) {
    g_launches.clear();
    pa_dims e = variant == 0 ? dims(4, 64, 8, 128, 8, 65536, 512) : dims(4, 64, 8, 64);
    const size_t wse = paged_attention_prefill_workspace_bytes(&e, T, maxq, nullptr);
    CHECK(paged_attention_prefill(FAKE, FAKE, FAKE, FAKE + (1 << 28), reinterpret_cast<const int32_t*>(FAKE),
                                  reinterpret_cast<const int32_t*>(FAKE),
                                  reinterpret_cast<const int32_t*>(FAKE + 128), T, maxq, 0.088f,
                                  e.block_size, nullptr, nullptr, &e, w, wse, nullptr) == PA_OK);
    CHECK(!g_launches.empty() && std::strcmp(g_launches[0].kind, "mfma") == 0);
  }
  pa_opts o = {0, PA_ENGINE_VALU, 0, PA_SCHEDULE_AUTO};
  CHECK(paged_attention_prefill(FAKE, FAKE, FAKE, FAKE + (1 << 28), reinterpret_cast<const int32_t*>(FAKE),
                                reinterpret_cast<const int32_t*>(FAKE),
                                reinterpret_cast<const int32_t*>(FAKE + 128), T, maxq, 0.088f, 16,
                                nullptr, nullptr, &d, w, ws, &o) == PA_ERR_UNSUPPORTED);
}

static void row_copies() {
  g_launches.clear();
  const int tile = 8 * 128 * 2;  // block 8, head size 128, fp16
  CHECK(gather_cached_kv(FAKE, FAKE, FAKE, FAKE + (1 << 28), reinterpret_cast<const int32_t*>(FAKE), 2048,
                         40, 128, 8, 1024, PA_F16, PA_KV_SEPARATE, nullptr) == PA_OK);
  CHECK(gather_cached_kv(FAKE, FAKE, FAKE, FAKE + tile, reinterpret_cast<const int32_t*>(FAKE), 2048, 40,
                         128, 8, 1024, PA_F16, PA_KV_JOINT, nullptr) == PA_OK);
  CHECK(paged_kv_cache_write(FAKE, FAKE + tile, FAKE, FAKE, reinterpret_cast<const int32_t*>(FAKE), 7, 40,
                             128, 8, 1024, PA_F16, PA_KV_JOINT, nullptr) == PA_OK);
  CHECK(paged_kv_cache_write(FAKE, FAKE + 2 * tile, FAKE, FAKE, reinterpret_cast<const int32_t*>(FAKE), 7,
                             40, 128, 8, 1024, PA_F16, PA_KV_JOINT, nullptr) == PA_ERR_INVALID_ARG);
  CHECK(g_launches.size() == 3);
  CHECK(g_launches[0].block_stride == 40 * tile && g_launches[0].head_stride == tile);
  CHECK(g_launches[1].block_stride == 2 * 40 * tile && g_launches[1].head_stride == 2 * tile);
  CHECK(std::strcmp(g_launches[2].kind, "write") == 0 && g_launches[2].num_tokens == 7);
  CHECK(g_launches[0].row_bytes == 256 && g_launches[0].num_kv_heads == 40 && g_launches[0].block_size == 8);
}

static void probe() {
  g_launches.clear();
  const size_t n = size_t(4) << 30;
  CHECK(pa_stream_read_sink_bytes(n) == 16 * 4096);
  CHECK(pa_stream_read_probe(FAKE, n, 0, FAKE, 16 * 4096, nullptr) == PA_OK);
  CHECK(pa_stream_read_probe(FAKE, n, 8192, FAKE, 16 * 4096, nullptr) == PA_OK);
  CHECK(g_launches.size() == 2 && g_launches[0].bytes == n && g_launches[1].run_bytes == 8192);
  CHECK(pa_stream_read_probe(FAKE, n, 0, FAKE, 16, nullptr) == PA_ERR_INVALID_ARG);
  CHECK(pa_stream_read_probe(FAKE, n, 512, FAKE, 16 * 4096, nullptr) == PA_ERR_INVALID_ARG);   // below 1 KB
  CHECK(pa_stream_read_probe(FAKE, n, 3072, FAKE, 16 * 4096, nullptr) == PA_ERR_INVALID_ARG);  // not 2^k
  CHECK(pa_stream_read_probe(FAKE, 3 * 8192, 8192, FAKE, 16 * 4096, nullptr) == PA_ERR_INVALID_ARG);
}

// The allocation-free entry point: split partials in the library's scratch,
// the same launches as a call given that much workspace; a forced partition
// size too large for the scratch is rejected before anything is launched.
static void decode_noalloc() {
  const auto tab = reinterpret_cast<const int32_t*>(FAKE);
  pa_dims d = dims(1, 64, 8);  // batch 1: a split plan
  g_launches.clear();
  CHECK(paged_attention_decode_noalloc(FAKE, FAKE, FAKE, FAKE + (1 << 30), tab, tab, 0.088f, 16,
                                       nullptr, nullptr, &d, nullptr) == PA_OK);
  CHECK(g_launches.size() == 2 && std::strcmp(g_launches[1].kind, "reduce") == 0);
  const Launch split = g_launches[0];
  CHECK(split.a.num_partitions > 1);
  CHECK(split.a.ws_o == reinterpret_cast<float*>(0x7f0000000000ull));
  g_launches.clear();
  char* ws = reinterpret_cast<char*>(0x7f0000000000ull);
  CHECK(decode(d, FAKE, FAKE + (1 << 30), ws, PA_NOALLOC_SCRATCH_BYTES) == PA_OK);
  CHECK(g_launches.size() == 2 && g_launches[0].a.num_partitions == split.a.num_partitions &&
        g_launches[0].a.partition_blocks == split.a.partition_blocks);
  // planned for 1024 CUs the auto split would exceed the scratch: fewer
  // partitions, still OK (for 256 CUs every auto plan fits: at most
  // 512 units x 64 heads x 128 x 4 bytes of partials)
  pa_dims big = dims(4, 64, 1, 128, 16, 1 << 20, 1 << 16);
  pa_opts o = {0, 0, 1024, 0};
  pa_plan unlimited, fits;
  CHECK(paged_attention_plan(&big, (size_t)1 << 40, &o, &unlimited) == PA_OK);
  CHECK(unlimited.workspace_bytes > PA_NOALLOC_SCRATCH_BYTES);
  CHECK(paged_attention_plan(&big, PA_NOALLOC_SCRATCH_BYTES, &o, &fits) == PA_OK);
  CHECK(fits.workspace_bytes <= PA_NOALLOC_SCRATCH_BYTES && fits.num_partitions < unlimited.num_partitions);
  g_launches.clear();
  CHECK(paged_attention_decode_noalloc(FAKE, FAKE, FAKE, FAKE + (1 << 30), tab, tab, 0.088f, 16,
                                       nullptr, nullptr, &big, &o) == PA_OK);
  CHECK(!g_launches.empty() && g_launches[0].a.num_partitions == fits.num_partitions);
  // forced: 256-token partitions of a 2^20-token bound need 4 * 64 * 4096 * 128 * 4 bytes
  pa_opts forced = {256, 0, 256, 0};
  g_launches.clear();
  CHECK(paged_attention_decode_noalloc(FAKE, FAKE, FAKE, FAKE + (1 << 30), tab, tab, 0.088f, 16,
                                       nullptr, nullptr, &big, &forced) == PA_ERR_WORKSPACE);
  CHECK(g_launches.empty());
  CHECK(std::string(pa_last_error()).find("scratch") != std::string::npos);
  CHECK(paged_attention_decode_noalloc(FAKE, FAKE, FAKE, FAKE + (1 << 30), tab, tab, 0.088f, 16,
                                       nullptr, nullptr, nullptr, nullptr) == PA_ERR_INVALID_ARG);
}

static void last_error_is_per_thread() {
  pa_dims bad = dims(1, 60, 8);
  CHECK(decode(bad, FAKE, FAKE) == PA_ERR_INVALID_ARG);
  std::string other;
  std::thread t([&] {
    pa_dims good = dims(256, 64, 8);
    other = decode(good, FAKE, FAKE + (1 << 28)) == PA_OK ? pa_last_error() : "failed";
  });
  t.join();
  CHECK(other.empty());
  CHECK(std::string(pa_last_error()).find("multiple") != std::string::npos);
  CHECK(std::string(pa_status_string(PA_ERR_ALIGNMENT)).size() > 0);
}

int main() {
  headline_single_pass();
  joint_layout();
  split_small_batch();
  mqa_longest_first();
  mqa_equal_shares();
  fp8_cache();
  mha_valu_and_forced_engines();
  prefill();
  row_copies();
  probe();
  decode_noalloc();
  last_error_is_per_thread();
  if (g_fail) {
    std::fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  std::printf("host layer: all checks passed\n");
  return 0;
}
