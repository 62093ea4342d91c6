// ccv_calib.hip -- streaming copies, a read-only sweep and an empty kernel, used
// only to measure the GPU next to the conv kernels (see include/ccv_calib.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ccv_calib.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kUnroll = 4;                 // 16-byte vectors per lane per chunk
constexpr int kChunk16 = 64 * kUnroll;     // vectors per wave chunk (4 KB)
constexpr int kWavesPerGroup = 4;

// A chunk is 4 KB: lane l moves vectors l, l + 64, l + 128, l + 192 of it, so each
// load or store instruction of the wave covers 1 KB of consecutive bytes (the
// forward kernels' layout).  Wave w takes chunks w, w + W, ... (W waves launched);
// a grid with one wave per chunk is the one-shot form.  The last, partial chunk is
// bounds-checked per vector.
template <bool NT>
__global__ void __launch_bounds__(256) copy_kernel(u32x4* __restrict__ dst, const u32x4* __restrict__ src,
                                                   int64_t n16, int64_t nwaves) {
  const int lane = threadIdx.x & 63;
  const int64_t w0 = (int64_t)blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6);
  const int64_t nchunks = (n16 + kChunk16 - 1) / kChunk16;
  for (int64_t ch = w0; ch < nchunks; ch += nwaves) {
    const int64_t base = ch * kChunk16 + lane;
    u32x4 v[kUnroll];
    if (base + (kUnroll - 1) * 64 < n16) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        v[u] = NT ? __builtin_nontemporal_load(src + base + u * 64) : src[base + u * 64];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (NT) __builtin_nontemporal_store(v[u], dst + base + u * 64);
        else dst[base + u * 64] = v[u];
      }
    } else {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        if (base + u * 64 < n16) dst[base + u * 64] = src[base + u * 64];
    }
  }
}

// Reads every 16-byte vector once with ordinary (cached) loads and folds them with
// xor; a wave stores its fold only when it equals `key`, which the caller picks so
// that practically never happens, so the loads cannot be dropped and nothing is
// written.
__global__ void __launch_bounds__(256) read_kernel(const u32x4* __restrict__ src, int64_t n16, int64_t nwaves,
                                                   unsigned key, unsigned* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t w0 = (int64_t)blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6);
  const int64_t nchunks = (n16 + kChunk16 - 1) / kChunk16;
  unsigned acc = 0;
  for (int64_t ch = w0; ch < nchunks; ch += nwaves) {
    const int64_t base = ch * kChunk16 + lane;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (base + u * 64 < n16) {
        const u32x4 v = src[base + u * 64];
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
      }
    }
  }
  if (acc == key) sink[lane] = acc;
}

__global__ void empty_kernel() {}

int check_buffer(const void* p, int64_t nbytes) {
  if (!p) return -1;
  if (nbytes < 0 || (nbytes & 15) || ((uintptr_t)p & 15)) return -2;
  return 0;
}

// Waves to launch for n16 vectors: one per chunk (waves_per_cu <= 0) or at most
// waves_per_cu * cus, rounded up to whole workgroups.
int64_t waves_for(int64_t n16, int waves_per_cu, int cus) {
  const int64_t nchunks = (n16 + kChunk16 - 1) / kChunk16;
  int64_t w = nchunks;
  if (waves_per_cu > 0 && (int64_t)waves_per_cu * cus < w) w = (int64_t)waves_per_cu * cus;
  return (w + kWavesPerGroup - 1) / kWavesPerGroup * kWavesPerGroup;
}

}  // namespace

extern "C" int ccv_calib_copy_ex(void* dst, const void* src, int64_t nbytes, int32_t waves_per_cu,
                                 int32_t nontemporal, void* stream) {
  int st = check_buffer(dst, nbytes);
  if (st == 0) st = check_buffer(src, nbytes);
  if (st) return st;
  const int64_t n16 = nbytes / 16;
  if (n16 == 0) return 0;
  int64_t nwaves = waves_for(n16, waves_per_cu, 256);
  const int64_t grid = nwaves / kWavesPerGroup;
  if (grid > INT32_MAX) return -2;
  u32x4* d = static_cast<u32x4*>(dst);
  const u32x4* s = static_cast<const u32x4*>(src);
  int64_t n = n16;
  void* args[] = {&d, &s, &n, &nwaves};
  const void* fn = nontemporal ? reinterpret_cast<const void*>(&copy_kernel<true>)
                               : reinterpret_cast<const void*>(&copy_kernel<false>);
  hipError_t e = hipLaunchKernel(fn, dim3((uint32_t)grid), dim3(64 * kWavesPerGroup), args, 0,
                                 static_cast<hipStream_t>(stream));
  return e == hipSuccess ? 0 : -8;
}

extern "C" int ccv_calib_copy(void* dst, const void* src, int64_t nbytes, void* stream) {
  return ccv_calib_copy_ex(dst, src, nbytes, 16, 1, stream);
}

extern "C" int ccv_calib_read(const void* src, int64_t nbytes, uint32_t key, void* sink, void* stream) {
  int st = check_buffer(src, nbytes);
  if (st == 0 && !sink) st = -1;
  if (st) return st;
  const int64_t n16 = nbytes / 16;
  if (n16 == 0) return 0;
  int64_t nwaves = waves_for(n16, 16, 256);
  const int64_t grid = nwaves / kWavesPerGroup;
  const u32x4* s = static_cast<const u32x4*>(src);
  int64_t n = n16;
  unsigned k = key;
  unsigned* out = static_cast<unsigned*>(sink);
  void* args[] = {&s, &n, &nwaves, &k, &out};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&read_kernel), dim3((uint32_t)grid),
                                 dim3(64 * kWavesPerGroup), args, 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? 0 : -8;
}

extern "C" int ccv_calib_empty(void* stream) {
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&empty_kernel), dim3(1), dim3(64),
                                 nullptr, 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? 0 : -8;
}
