// Launch records of the host-only build (see hip_stubs.cpp).
#pragma once

#include <hip/hip_runtime.h>

#include <vector>

#include "launch.h"

constexpr int kStubCus = 256;  // compute units the stub device reports

struct Launch {
  char kind[16];
  pa::DecodeArgs a;
  int dtype, head_size;
  bool kv_fp8;
  const void* ptr;
  int32_t num_tokens, num_kv_heads, row_bytes, block_size;
  int64_t block_stride, head_stride;
  size_t bytes, run_bytes;
};

extern std::vector<Launch> g_launches;
