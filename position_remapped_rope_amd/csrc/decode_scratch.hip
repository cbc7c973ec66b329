// A fixed device array for the decode entry point that allocates nothing
// (prope_attn_decode_noalloc): the split-K partials of one launch, at most
// kDecodeScratchBytes. The code object holds one copy of the array on every
// device it is loaded on, until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory, so it is
// never passed to a kernel or a copy. Its device address is looked up once per
// device, with that device current, and kept; every later call on the device
// uses that address. Calls on one device share the array, so calls that may
// overlap on a device (other streams, concurrent graph replays) race on it. No
// part of it needs to start at zero: the split kernel writes every partial the
// combine reads.
#include <mutex>

#include "internal.hpp"

namespace prope {
namespace {

__device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];

}  // namespace

hipError_t decode_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p || reinterpret_cast<uintptr_t>(p) % 256) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

}  // namespace prope
