// Host-only stand-ins for the three HIP runtime calls the C-ABI host layer
// makes and for the kernel launchers it calls, so that layer (validation,
// planning, launch arguments) builds with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer and runs without a GPU.  Every launcher records
// what it was asked to launch; nothing is executed.
#include "hip_stubs.h"

#include <cstring>

std::vector<Launch> g_launches;

extern "C" {
hipError_t hipGetDevice(int* device) {
  *device = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t, int) {
  *value = kStubCus;
  return hipSuccess;
}
const char* hipGetErrorString(hipError_t) { return "stub launch error"; }
}

namespace {
void record(const char* kind, const pa::DecodeArgs* a, int dtype, int head_size, bool kv_fp8) {
  Launch l{};
  std::strncpy(l.kind, kind, sizeof(l.kind) - 1);
  if (a) l.a = *a;
  l.dtype = dtype;
  l.head_size = head_size;
  l.kv_fp8 = kv_fp8;
  g_launches.push_back(l);
}
}  // namespace

namespace pa {
hipError_t launch_decode_valu(const DecodeArgs& a, int dtype, int head_size, bool kv_fp8, hipStream_t) {
  record("valu", &a, dtype, head_size, kv_fp8);
  return hipSuccess;
}
hipError_t launch_decode_mfma(const DecodeArgs& a, int dtype, int head_size, bool kv_fp8, hipStream_t) {
  record("mfma", &a, dtype, head_size, kv_fp8);
  return hipSuccess;
}
bool prefill_mfma32_supported(int head_size, bool kv_fp8, int block_size) {
  return head_size == 128 && !kv_fp8 && block_size >= 16;
}
hipError_t launch_prefill_mfma32(const DecodeArgs& a, int dtype, hipStream_t) {
  record("prefill32", &a, dtype, 128, false);
  return hipSuccess;
}
hipError_t launch_partition_reduce(const DecodeArgs& a, int dtype, int head_size, hipStream_t) {
  record("reduce", &a, dtype, head_size, false);
  return hipSuccess;
}
hipError_t staged_decode_occupancy(int, int head_size, int group, bool kv_fp8, int* wgs) {
  *wgs = staged_decode_wgs_per_cu(head_size, group, kv_fp8);
  return hipSuccess;
}
hipError_t launch_unit_order(const DecodeArgs& a, int32_t* order, hipStream_t) {
  record("order", &a, 0, 0, false);
  g_launches.back().ptr = order;
  return hipSuccess;
}
hipError_t launch_gather(void*, void*, const void*, const void*, const int32_t*, int32_t num_tokens,
                         int32_t num_kv_heads, int32_t row_bytes, int32_t block_size,
                         int64_t block_stride, int64_t head_stride, hipStream_t) {
  record("gather", nullptr, 0, 0, false);
  Launch& l = g_launches.back();
  l.num_tokens = num_tokens;
  l.num_kv_heads = num_kv_heads;
  l.row_bytes = row_bytes;
  l.block_size = block_size;
  l.block_stride = block_stride;
  l.head_stride = head_stride;
  return hipSuccess;
}
hipError_t launch_cache_write(void*, void*, const void*, const void*, const int32_t*, int32_t num_tokens,
                              int32_t num_kv_heads, int32_t row_bytes, int32_t block_size,
                              int64_t block_stride, int64_t head_stride, hipStream_t) {
  record("write", nullptr, 0, 0, false);
  Launch& l = g_launches.back();
  l.num_tokens = num_tokens;
  l.num_kv_heads = num_kv_heads;
  l.row_bytes = row_bytes;
  l.block_size = block_size;
  l.block_stride = block_stride;
  l.head_stride = head_stride;
  return hipSuccess;
}
// A fake device address for the allocation-free entry point's scratch.
hipError_t noalloc_scratch(int, void** ptr) {
  *ptr = reinterpret_cast<void*>(uintptr_t(0x7f0000000000ull));
  return hipSuccess;
}
hipError_t launch_stream_read(const void*, size_t bytes, size_t run_bytes, void*, hipStream_t) {
  record("probe", nullptr, 0, 0, false);
  g_launches.back().bytes = bytes;
  g_launches.back().run_bytes = run_bytes;
  return hipSuccess;
}
}  // namespace pa
