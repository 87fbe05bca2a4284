// noalloc.hip -- the library's static device scratch, used by
// lkv_mla_decode_noalloc in place of a caller workspace (for callers that
// cannot allocate: code under HIP graph capture, tight serving loops).
//
// `scratch` is a file-scope device array: each GPU the library runs on holds
// its own copy, at its own address, until the process ends.  Host code never
// uses the array's name as an address (on the host it is only a stand-in for
// the symbol): the device address comes from hipGetSymbolAddress, taken once
// per device with that device current, and is kept per device.
#include <hip/hip_runtime.h>

#include <mutex>

#include "lkv.h"
#include "lkv_internal.h"

namespace {

__device__ __align__(256) unsigned char scratch[LKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

}  // namespace

namespace lkv {

hipError_t static_scratch(void **ptr, size_t *bytes) {
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  *bytes = LKV_NOALLOC_SCRATCH_BYTES;
  return hipSuccess;
}

}  // namespace lkv
