// Library-owned device scratch for the entry points that allocate nothing
// (nq_attn_decode_static): one file-scope device array, present once on every
// GPU the library runs on, and the per-device lookup of its address.
//
// In host code the array's name is a host-side stand-in, not a device address,
// so nothing outside this file uses it: the address comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// every kernel argument uses that pointer.
#include <mutex>

#include "common.hpp"

namespace nq {

static __device__ __align__(256) unsigned char scratch[kAttnScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};
}  // namespace

hipError_t static_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // the current device's copy
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace nq
