// Fixed device scratch behind kda_chunk_fwd_noalloc, for callers that cannot
// allocate device memory.
//
// `scratch` is a file-scope device array: each GPU the library runs on holds
// its own copy until the process ends.  In host code its name is a host-side
// stand-in, not a device address; the address kernels may use is looked up
// here, once per device with that device current, by hipGetSymbolAddress, and
// kept per device.  Host code uses only that address.
#include <mutex>

#include "../../include/kda.h"
#include "kda_launch.h"

__device__ __attribute__((aligned(256))) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace kda {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, void** out, char* why, size_t why_len) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) {
    snprintf(why, why_len, "device of the stream");
    return e;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    snprintf(why, why_len, "device %d out of range", dev);
    return hipErrorInvalidDevice;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    int cur = -1;
    if ((e = hipGetDevice(&cur)) != hipSuccess) {
      snprintf(why, why_len, "current device");
      return e;
    }
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) {
      snprintf(why, why_len, "making device %d current", dev);
      return e;
    }
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) {
      snprintf(why, why_len, "address on device %d", dev);
      return e;
    }
    if (back != hipSuccess) {
      snprintf(why, why_len, "restoring device %d", cur);
      return back;
    }
    if (!ptr || reinterpret_cast<uintptr_t>(ptr) % 256) {
      snprintf(why, why_len, "address on device %d is not 256-byte aligned", dev);
      return hipErrorInvalidValue;
    }
    g_ptr[dev] = ptr;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace kda
