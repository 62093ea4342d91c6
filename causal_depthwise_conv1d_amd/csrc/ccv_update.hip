// ccv_update.hip -- the update (decode) kernel: a few new steps of every (b, c)
// row against the K-1 step history before them, and the history advanced in
// place (Ch.4 "Dao interface and source map", section "Reading the source along
// the call chain": the update kernel reads the history and moves the state
// forward in place).
//
// Work split.  Decode touches O(B*C*K) bytes and has no reuse between rows, so
// one thread owns one (b, c) row: it loads the row's weights, bias and whole
// history into registers, runs the L new steps through a register window, and
// only then writes the new history.  Because every row is read before it is
// written by the same thread, the state needs no second buffer and threads need
// no ordering.  Threads of a wave take 64 consecutive channels of one batch, so
// with the usual layouts (channel stride 1, or K-1 for a [B, C, K-1] state)
// their accesses fall in a handful of cache lines.
//
// Arithmetic.  The same as the forward kernels' term for term: acc = bias (0
// without one), one fused multiply-add per tap in ascending k over the extended
// input (history, then x), the same SiLU on the fp32 accumulator, the same
// round-to-nearest-even down-convert (Ch.5 "Dao forward CUDA implementation",
// section "How adjacent threads and chunks exchange history", stencil equation
// for z_i).  So decoding one step at a time reproduces the forward's bits, and
// the new history is a bit copy of the last K-1 inputs (Ch.5, section "Three
// kinds of boundary handled separately").
#include "ccv_device.hpp"
#include "ccv_update_launch.hpp"

namespace ccv {
namespace {

template <class S, int K, bool SILU>
__global__ void __launch_bounds__(kUpdateBlock) update_kernel(const UpdArgs a) {
  using raw = typename S::raw;
  constexpr int H = K - 1;
  const int64_t r = (int64_t)blockIdx.x * kUpdateBlock + threadIdx.x;
  if (r >= a.rows) return;
  const int64_t b = r / a.C;
  const int64_t c = r - b * a.C;

  float w[K];
  load_params<K>(a.w, a.w_dtype, c * K, w);
  const float beta = a.bias ? load_param(a.bias, a.w_dtype, c) : 0.0f;

  raw* __restrict__ st = static_cast<raw*>(a.state) + b * a.s_sb + c * a.s_sc;
  raw hist[H];                                   // X~ just left of the next step, oldest first
#pragma unroll
  for (int i = 0; i < H; ++i) hist[i] = st[i * a.s_si];

  const raw* __restrict__ xr = static_cast<const raw*>(a.x) + b * a.x_sb + c * a.x_sc;
  raw* __restrict__ orow = static_cast<raw*>(a.out) + b * a.o_sb + c * a.o_sc;
  for (int64_t t = 0; t < a.L; ++t) {
    const raw xv = xr[t * a.x_sl];
    float acc = beta;
#pragma unroll
    for (int k = 0; k < H; ++k) acc = __builtin_fmaf(w[k], S::to_f(hist[k]), acc);
    acc = __builtin_fmaf(w[H], S::to_f(xv), acc);
    orow[t * a.o_sl] = S::from_f(SILU ? silu(acc) : acc);
#pragma unroll
    for (int i = 0; i + 1 < H; ++i) hist[i] = hist[i + 1];
    hist[H - 1] = xv;
  }

#pragma unroll
  for (int i = 0; i < H; ++i) st[i * a.s_si] = hist[i];
}

template <class S, int K>
int launch_k(const UpdArgs& a, bool silu, uint32_t grid, void* st) {
  const void* fn = silu ? reinterpret_cast<const void*>(&update_kernel<S, K, true>)
                        : reinterpret_cast<const void*>(&update_kernel<S, K, false>);
  void* args[] = {const_cast<UpdArgs*>(&a)};
  return (int)hipLaunchKernel(fn, dim3(grid), dim3(kUpdateBlock), args, 0, static_cast<hipStream_t>(st));
}

template <class S>
int launch_s(const UpdArgs& a, int K, bool silu, uint32_t grid, void* st) {
  switch (K) {
    case 2: return launch_k<S, 2>(a, silu, grid, st);
    case 3: return launch_k<S, 3>(a, silu, grid, st);
    case 4: return launch_k<S, 4>(a, silu, grid, st);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace

int launch_update(const UpdArgs& a, int dtype, int K, bool silu, uint32_t grid, void* stream) {
  switch (dtype) {
    case CCV_DT_F32: return launch_s<F32>(a, K, silu, grid, stream);
    case CCV_DT_F16: return launch_s<F16>(a, K, silu, grid, stream);
    case CCV_DT_BF16: return launch_s<BF16>(a, K, silu, grid, stream);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace ccv
