// noalloc.hip -- the device-resident scratch of the entry point that
// allocates nothing (pa_decode_step_noalloc).
//
// A multi-partition decode plan needs fp32 partials between the attention
// launch and the merge launch.  The ordinary entry points take them from the
// caller's workspace; for callers that cannot allocate, they live in this
// file-scope device array instead.  Every device that loads the library holds
// its own copy, at its own address, until the process ends.  In host code the
// name `scratch` stands for a host-side shadow, not a device address: the
// address each device holds is looked up once per device with
// hipGetSymbolAddress and only that pointer is handed to kernels.
#include <mutex>

#include "kv_ops.h"
#include "noalloc.h"

namespace pa {

static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // with `dev` current
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return hipSuccess;
}

}  // namespace pa
