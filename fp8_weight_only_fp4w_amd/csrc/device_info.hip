// Per-device host state of the library: the current device and its compute
// unit count, each queried once per device and thread-safely (the calls of
// the C ABI are re-entrant; calls on different streams and threads may
// overlap).

#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"

namespace fp4w {

int current_device() {
  int dev = 0;
  return hipGetDevice(&dev) == hipSuccess ? dev : 0;
}

int device_cus() {
  static std::once_flag once[kMaxDevices];
  static int cus[kMaxDevices];
  const int dev = current_device();
  auto query = [dev] {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v < 1) v = 256;
    return v;
  };
  if (dev < 0 || dev >= kMaxDevices) return query();
  std::call_once(once[dev], [&] { cus[dev] = query(); });
  return cus[dev];
}

}  // namespace fp4w
