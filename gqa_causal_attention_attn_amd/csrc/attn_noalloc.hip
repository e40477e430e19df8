// The library's one device buffer of its own: the scratch that attn_decode_noalloc uses for the
// split partials instead of a caller-provided workspace (for callers that cannot allocate).
//
// `scratch` is a file-scope device array; every GPU the library runs on holds its own copy,
// at its own address, until the process ends.  In host code its name is only a stand-in, so
// the device address is looked up once per device (hipGetSymbolAddress, with that device
// current) and kept; kernels receive that address like any workspace pointer.  Every call on
// one GPU shares that GPU's array: calls that overlap on one GPU (different streams) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "attn_internal.h"

namespace gqa {
namespace {

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device, null until looked up

}  // namespace

hipError_t scratch_of_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

}  // namespace gqa
