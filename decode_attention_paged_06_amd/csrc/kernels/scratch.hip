// Device-resident scratch of the allocation-free decode entry point.
//
// One statically sized array per GPU, part of the library's code object:
// each device that loads the library holds its own copy until the process
// ends.  Its device address is looked up once per device (with that device
// current) and kept; host code only ever passes that address, never the
// array's name (which on the host is a stand-in, not a device pointer).
#include <mutex>

#include "../launch.h"
#include "paged_attention.h"

namespace pa {

namespace {

static __device__ __align__(256) char scratch[PA_NOALLOC_SCRATCH_BYTES];

constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};

}  // namespace

hipError_t noalloc_scratch(int device, void** ptr) {
  if (device < 0 || device >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[device] = p;
  }
  *ptr = g_scratch_ptr[device];
  return hipSuccess;
}

}  // namespace pa
