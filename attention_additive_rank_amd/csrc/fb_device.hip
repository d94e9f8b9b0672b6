// Device properties that the launchers need, looked up once per device.
#include <atomic>

#include "fb_internal.h"

namespace fb {

int device_cu_count() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];   // 0 = not looked up yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 0;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace fb
