// ccv_bwd_static.hip -- ccv_bwd_static: the backward with its fp32 partial sums in
// a fixed device array of this library instead of a caller-provided workspace, for
// callers that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).  Same kernels, same launches,
// same results as ccv_bwd.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "ccv.h"

namespace {

constexpr int64_t kScratchBytes = CCV_BWD_STATIC_SCRATCH_BYTES;

// The partial-sum rows of every ccv_bwd_static call on a device.  Each device the
// library runs on holds its own copy from the first call there until the process
// ends.  Host code never uses this name as an address (on the host it is only a
// handle); it uses the device address that hipGetSymbolAddress returns.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];      // device address of `scratch`, per device, once known

// The device address of `scratch` on `dev`, which must be the current device.
int scratch_on(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return CCV_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CCV_E_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return CCV_OK;
}

}  // namespace

extern "C" int ccv_bwd_static(const ccv_bwd_args_t* args, void* hip_stream) {
  if (!args) return CCV_E_NULL;
  if (args->struct_size != (int64_t)sizeof(ccv_bwd_args_t)) return CCV_E_ABI;
  ccv_bwd_args_t a = *args;
  a.workspace = nullptr;
  a.workspace_bytes = 0;
  const int64_t need = ccv_bwd_workspace_size(&a);
  if (need < 0) return (int)need;                  // an argument error, as ccv_bwd reports it
  if (need > kScratchBytes) return CCV_E_SCRATCH;
  if (need > 0) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return CCV_E_HIP;
    if (hip_stream) {                               // the array of the stream's own device
      int sdev = -1;
      if (hipStreamGetDevice(static_cast<hipStream_t>(hip_stream), &sdev) != hipSuccess) return CCV_E_HIP;
      if (sdev != dev) return CCV_E_UNSUPPORTED;
    }
    const int st = scratch_on(dev, &a.workspace);
    if (st != CCV_OK) return st;
    a.workspace_bytes = kScratchBytes;
  }
  return ccv_bwd(&a, hip_stream);
}
