// The fixed device scratch of octo_decode_attn_static: the split-K partials
// and rotated queries of the decode calls, held in a file-scope device array
// instead of a caller's workspace, for callers that cannot allocate.
#include <mutex>

#include "octo_internal.hpp"

namespace octo {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};
}  // namespace

// The device address of `scratch` on `device`, which must be the current
// device: each GPU holds its own copy of the array at its own address.  The
// host-side name `scratch` is not a device address and is never used as one.
hipError_t static_scratch(int device, void** out) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[device] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[device] = p;
  }
  *out = g_scratch[device];
  return hipSuccess;
}

}  // namespace octo
