// ccv_bwd.hip -- the backward of the causal depthwise conv1d: dx, dinitial_states,
// dweight and dbias from dout and dfinal_states (Ch.4 "Dao interface and source
// map", section "How autograd links forward and backward"; the formulas are
// stated in ccv.h beside ccv_bwd).
//
// Gradient kernel.  One lane owns one (b, c) row and one tile of T time steps.
// It walks u = t0 .. t_end + K - 2 once, with three register windows over the
// positions u-K+1 .. u: the extended input X~, the sequence ids, and dz.  At
// each u < L it recomputes the pre-activation z[u] exactly as the forward does
// (bias first, k ascending, fused multiply-adds) and forms dz[u] = dout[u] *
// act'(z[u]); for u inside the tile it adds the tap products dz[u] * X~[u-K+1+k]
// to its fp32 partial dweight and dbias.  Position j = u-K+1 then has every dz it
// reads (dz[j .. j+K-1]), so dX~[j] is finished and stored: to dx when j lies in
// the tile, to dinitial_states when j < 0 in the row's first tile.  Recomputing
// z over the K-1 steps past the tile is the halo; nothing from the forward is
// stored.  The lane's partial sums go to the workspace.  Lanes take consecutive
// channels, so a wave's accesses are coalesced when channels are unit-stride
// and repeat over the same cache lines from step to step otherwise.
//
// Reduction kernel.  One lane per (tap or bias, channel) sums the partials of
// all (b, tile) in a fixed order (chunks of kBwdChunk, then the chunk sums), so
// dweight and dbias repeat bit for bit, and rounds once to the weight dtype
// (the fp32-accumulate-then-convert of the section cited above).
#include "ccv_bwd_launch.hpp"
#include "ccv_device.hpp"

namespace ccv {
namespace {

// d silu(z) / dz = s (1 + z (1 - s)) with s = sigmoid(z), on the hardware exp2 and
// rcp as the forward's SiLU.
__device__ inline float silu_slope(float z) {
  const float s = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.44269504088896341f));
  return s * (1.0f + z * (1.0f - s));
}

template <class S, int K, bool SILU, bool SEQ>
__global__ void __launch_bounds__(kBwdBlock) bwd_kernel(const BwdArgs a) {
  using raw = typename S::raw;
  constexpr int H = K - 1;
  const int64_t id = (int64_t)blockIdx.x * kBwdBlock + threadIdx.x;
  if (id >= a.lanes) return;
  const int64_t bt = id / a.C;
  const int64_t c = id - bt * a.C;
  const int64_t b = bt / a.ntt;
  const int64_t t0 = (bt - b * a.ntt) * a.T;
  const int64_t L = a.L;
  const int64_t t_end = t0 + a.T < L ? t0 + a.T : L;

  float w[K];
  load_params<K>(a.w, a.w_dtype, c * K, w);
  const float beta = a.bias ? load_param(a.bias, a.w_dtype, c) : 0.0f;
  const raw* xr = static_cast<const raw*>(a.x) + b * a.x_sb + c * a.x_sc;
  const raw* gr = static_cast<const raw*>(a.dout) + b * a.d_sb + c * a.d_sc;
  raw* dxr = static_cast<raw*>(a.dx) + b * a.g_sb + c * a.g_sc;
  const int32_t* sr = SEQ ? a.seq + b * L : nullptr;

  // Slots 0 .. H-1 hold positions u-H .. u-1 before step u; slot H takes u.
  float xw[K], dzw[K];
  int idw[K];
#pragma unroll
  for (int i = 0; i < H; ++i) {
    const int64_t j = t0 - H + i;
    if (j >= 0)
      xw[i] = S::to_f(xr[j * a.x_sl]);
    else if (a.init)
      xw[i] = S::to_f(static_cast<const raw*>(a.init)[b * a.is_b + c * a.is_c + (j + H) * a.is_i]);
    else
      xw[i] = 0.0f;
    idw[i] = (SEQ && j >= 0) ? sr[j] : 0;
    dzw[i] = 0.0f;                                 // dz left of the tile is never read
  }
  float pw[K], pb = 0.0f;
#pragma unroll
  for (int k = 0; k < K; ++k) pw[k] = 0.0f;

  for (int64_t u = t0; u < t_end + H; ++u) {
    float xu = 0.0f, dzu = 0.0f;
    int idu = 0;
    if (u < L) {
      xu = S::to_f(xr[u * a.x_sl]);
      if constexpr (SEQ) idu = sr[u];
      bool keep[H];
      float z = beta;
#pragma unroll
      for (int k = 0; k < H; ++k) {
        keep[k] = !SEQ || (u - H + k >= 0 && idw[k] == idu);
        if (keep[k]) z = __builtin_fmaf(w[k], xw[k], z);
      }
      z = __builtin_fmaf(w[H], xu, z);
      const float go = S::to_f(gr[u * a.d_sl]);
      dzu = SILU ? go * silu_slope(z) : go;
      if (u < t_end) {
#pragma unroll
        for (int k = 0; k < H; ++k)
          if (keep[k]) pw[k] = __builtin_fmaf(dzu, xw[k], pw[k]);
        pw[H] = __builtin_fmaf(dzu, xu, pw[H]);
        pb += dzu;
      }
    }
    xw[H] = xu;
    dzw[H] = dzu;
    idw[H] = idu;

    // dX~ at j = u - H reads dz[j .. u] = slots 0 .. H.
    const int64_t j = u - H;
    const bool to_dx = j >= t0;
    const bool to_init = j < 0 && a.dinit != nullptr;
    if (to_dx || to_init) {
      float acc = 0.0f;
#pragma unroll
      for (int k = 0; k < K; ++k) {                // output t = j + H - k uses tap k on X~[j]
        const int64_t t = j + H - k;
        const bool keep = t >= 0 && t < L && (!SEQ || idw[0] == idw[H - k]);
        if (keep) acc = __builtin_fmaf(w[k], dzw[H - k], acc);
      }
      if (a.dfs && j >= L - H)
        acc += S::to_f(static_cast<const raw*>(a.dfs)[b * a.fs_b + c * a.fs_c + (j - (L - H)) * a.fs_i]);
      if (j >= 0)
        dxr[j * a.g_sl] = S::from_f(acc);
      else
        static_cast<raw*>(a.dinit)[b * a.di_b + c * a.di_c + (j + H) * a.di_i] = S::from_f(acc);
    }
#pragma unroll
    for (int i = 0; i < H; ++i) {
      xw[i] = xw[i + 1];
      dzw[i] = dzw[i + 1];
      idw[i] = idw[i + 1];
    }
  }

  float* part = a.part + bt * (K + 1) * a.C + c;
#pragma unroll
  for (int k = 0; k < K; ++k) part[k * a.C] = pw[k];
  part[K * a.C] = pb;
}

__device__ inline void store_param(void* p, int dtype, int64_t i, float v) {
  if (dtype == CCV_DT_F32)
    static_cast<float*>(p)[i] = v;
  else if (dtype == CCV_DT_BF16)
    static_cast<uint16_t*>(p)[i] = BF16::from_f(v);
  else
    static_cast<uint16_t*>(p)[i] = F16::from_f(v);
}

__global__ void __launch_bounds__(kBwdBlock) bwd_reduce_kernel(const BwdReduceArgs r) {
  const int64_t id = (int64_t)blockIdx.x * kBwdBlock + threadIdx.x;
  const int64_t slots = (int64_t)(r.K + 1) * r.C;
  if (id >= slots) return;
  const int64_t slot = id / r.C;
  const int64_t c = id - slot * r.C;
  if (slot == r.K && !r.db) return;
  const float* p = r.part + slot * r.C + c;
  const int64_t stride = (int64_t)(r.K + 1) * r.C;
  float total = 0.0f;
  for (int64_t p0 = 0; p0 < r.nparts; p0 += kBwdChunk) {
    const int64_t p1 = p0 + kBwdChunk < r.nparts ? p0 + kBwdChunk : r.nparts;
    float chunk = 0.0f;
    for (int64_t q = p0; q < p1; ++q) chunk += p[q * stride];
    total += chunk;
  }
  if (slot < r.K)
    store_param(r.dw, r.w_dtype, c * r.K + slot, total);
  else
    store_param(r.db, r.w_dtype, c, total);
}

template <class S, int K, bool SILU, bool SEQ>
int launch_one(const BwdArgs& a, uint32_t grid, void* st) {
  void* args[] = {const_cast<BwdArgs*>(&a)};
  return (int)hipLaunchKernel(reinterpret_cast<const void*>(&bwd_kernel<S, K, SILU, SEQ>), dim3(grid),
                              dim3(kBwdBlock), args, 0, static_cast<hipStream_t>(st));
}

template <class S, int K>
int launch_k(const BwdArgs& a, bool silu, bool seq, uint32_t grid, void* st) {
  if (silu) return seq ? launch_one<S, K, true, true>(a, grid, st) : launch_one<S, K, true, false>(a, grid, st);
  return seq ? launch_one<S, K, false, true>(a, grid, st) : launch_one<S, K, false, false>(a, grid, st);
}

template <class S>
int launch_s(const BwdArgs& a, int K, bool silu, bool seq, uint32_t grid, void* st) {
  switch (K) {
    case 2: return launch_k<S, 2>(a, silu, seq, grid, st);
    case 3: return launch_k<S, 3>(a, silu, seq, grid, st);
    case 4: return launch_k<S, 4>(a, silu, seq, grid, st);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace

int launch_bwd(const BwdArgs& a, int dtype, int K, bool silu, bool seq, uint32_t grid, void* stream) {
  switch (dtype) {
    case CCV_DT_F32: return launch_s<F32>(a, K, silu, seq, grid, stream);
    case CCV_DT_F16: return launch_s<F16>(a, K, silu, seq, grid, stream);
    case CCV_DT_BF16: return launch_s<BF16>(a, K, silu, seq, grid, stream);
  }
  return (int)hipErrorInvalidValue;
}

int launch_bwd_reduce(const BwdReduceArgs& r, uint32_t grid, void* stream) {
  void* args[] = {const_cast<BwdReduceArgs*>(&r)};
  return (int)hipLaunchKernel(reinterpret_cast<const void*>(&bwd_reduce_kernel), dim3(grid), dim3(kBwdBlock),
                              args, 0, static_cast<hipStream_t>(stream));
}

}  // namespace ccv
