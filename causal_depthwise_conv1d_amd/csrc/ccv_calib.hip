// ccv_calib.hip -- a plain streaming copy and an empty kernel, used only to
// measure the GPU next to the conv kernels (see include/ccv_calib.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ccv_calib.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kCopyUnroll = 4;

// Thread i of workgroup g copies 16-byte vectors g*1024*U/... laid out so that
// each load or store instruction of a wave covers 1 KB of consecutive bytes.
__global__ void __launch_bounds__(256) copy_kernel(u32x4* __restrict__ dst,
                                                   const u32x4* __restrict__ src, int64_t n16) {
  const int64_t base = (int64_t)blockIdx.x * 256 * kCopyUnroll + threadIdx.x;
  u32x4 v[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t i = base + u * 256;
    if (i < n16) v[u] = src[i];
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t i = base + u * 256;
    if (i < n16) dst[i] = v[u];
  }
}

__global__ void empty_kernel() {}

}  // namespace

extern "C" int ccv_calib_copy(void* dst, const void* src, int64_t nbytes, void* stream) {
  if (!dst || !src) return -1;
  if (nbytes < 0 || (nbytes & 15) || ((uintptr_t)dst & 15) || ((uintptr_t)src & 15)) return -2;
  const int64_t n16 = nbytes / 16;
  if (n16 == 0) return 0;
  const int64_t grid = (n16 + 256 * kCopyUnroll - 1) / (256 * kCopyUnroll);
  if (grid > INT32_MAX) return -2;
  u32x4* d = static_cast<u32x4*>(dst);
  const u32x4* s = static_cast<const u32x4*>(src);
  void* args[] = {&d, &s, const_cast<int64_t*>(&n16)};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&copy_kernel), dim3((uint32_t)grid),
                                 dim3(256), args, 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? 0 : -8;
}

extern "C" int ccv_calib_empty(void* stream) {
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&empty_kernel), dim3(1), dim3(64),
                                 nullptr, 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? 0 : -8;
}
