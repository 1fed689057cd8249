// device.cpp -- cached device properties used to size launches.
#include <atomic>

#include "launch.hpp"

namespace fp4 {

// Compute units and LDS bytes per CU of the current device. The attribute
// queries cost several microseconds, comparable to a launch, so the values (a
// fixed property of the device) are kept per device ordinal after the first.
DeviceInfo device_info() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cus_cached[kMaxDevices], lds_cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return {256, 160 * 1024};
  const bool keep = dev >= 0 && dev < kMaxDevices;
  if (keep) {
    const int c = cus_cached[dev].load(std::memory_order_relaxed);
    const int l = lds_cached[dev].load(std::memory_order_relaxed);
    if (c > 0 && l > 0) return {c, l};
  }
  int c = 0, l = 0;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
    c = 256;
  if (hipDeviceGetAttribute(&l, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
          hipSuccess || l <= 0)
    l = 160 * 1024;
  if (keep) {
    cus_cached[dev].store(c, std::memory_order_relaxed);
    lds_cached[dev].store(l, std::memory_order_relaxed);
  }
  return {c, l};
}

}  // namespace fp4
