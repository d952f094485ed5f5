// Library-owned device scratch for the entry points that must not allocate
// (callers that run under HIP graph capture, in serving loops without
// allocations, or in harnesses that forbid hipMalloc).
//
// The array lives in the code object: every device the library runs on holds
// its own copy, at its own address, from module load until the process ends.
// Host code never uses the array's name as a device address (on the host it
// is only a stand-in); the address comes from hipGetSymbolAddress, taken once
// per device with that device current, and is kept per device.
//
// Every call on one device shares that device's copy and leaves the last
// call's contents in it; calls that overlap on one device (for example on two
// streams) race on it.

#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"

namespace fp4w {
namespace {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

void* g_scratch[kMaxDevices];
bool g_scratch_ok[kMaxDevices];

}  // namespace

int static_scratch(void** out) {
  static std::once_flag once[kMaxDevices];
  const int dev = current_device();
  if (dev < 0 || dev >= kMaxDevices) return -1;
  std::call_once(once[dev], [dev] {
    void* p = nullptr;
    g_scratch_ok[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess && p != nullptr;
    g_scratch[dev] = g_scratch_ok[dev] ? p : nullptr;
  });
  if (!g_scratch_ok[dev]) return -1;
  *out = g_scratch[dev];
  return 0;
}

}  // namespace fp4w
