// ccv_device_info.hip -- the compute-unit count of the GPU a call runs on, read
// from the runtime once per device and kept for the life of the process.
#include <hip/hip_runtime.h>

#include <atomic>

#include "ccv_launch.hpp"

namespace ccv {
namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];   // 0 until read
std::atomic<int> g_last{0};            // the count of the device of the latest launch

}  // namespace

int device_cu_count(void* stream) {
  int dev = -1;
  const hipError_t e = stream ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) : hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) return -1;
  int n = dev < kMaxDevices ? g_cus[dev].load(std::memory_order_relaxed) : 0;
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return -1;
    if (dev < kMaxDevices) g_cus[dev].store(n, std::memory_order_relaxed);
  }
  g_last.store(n, std::memory_order_relaxed);
  return n;
}

int last_cu_count() { return g_last.load(std::memory_order_relaxed); }

}  // namespace ccv
