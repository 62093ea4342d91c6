// ccv_update.hip -- the update (decode) kernel: a few new steps of every (b, c)
// row against the K-1 step history before them, and the history advanced in
// place (Ch.4 "Dao interface and source map", section "Reading the source along
// the call chain": the update kernel reads the history and moves the state
// forward in place).
//
// Work split.  Decode touches O(B*C*K) bytes and has no reuse between rows, so
// each (b, c) row belongs to one lane: it loads the row's weights, bias and
// whole history into registers, runs the L new steps through a register window,
// and only then writes the new history.  Because every row is read before it is
// written by the same lane, the state needs no second buffer and lanes need no
// ordering.  The call is bound by how many bytes are in flight, so a lane takes
// R rows and issues all their loads before any arithmetic, and the grid is sized
// to be resident at once.  A wave's lanes take consecutive rows (rows are
// numbered b * C + c), so with the usual layouts (channel stride 1, or K-1 for a
// [B, C, K-1] state) each load instruction touches a few cache lines.
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

// Element e of a run of 16-byte vectors holding raw values of S, and the reverse.
template <class S>
__device__ inline typename S::raw get_elem(const u32x4* v, int e) {
  if constexpr (sizeof(typename S::raw) == 4) {
    return dword(v[e / 4], e % 4);
  } else {
    const uint32_t d = dword(v[e / 8], (e % 8) / 2);
    return (uint16_t)((e & 1) ? d >> 16 : d & 0xffffu);
  }
}

template <class S, int N>
__device__ inline void put_elems(const typename S::raw (&r)[N], u32x4* v) {
  if constexpr (sizeof(typename S::raw) == 4) {
#pragma unroll
    for (int e = 0; e < N; ++e) v[e / 4][e % 4] = r[e];
  } else {
#pragma unroll
    for (int e = 0; e < N; e += 2) v[e / 8][(e % 8) / 2] = (uint32_t)r[e] | ((uint32_t)r[e + 1] << 16);
  }
}

// The 16-byte path: a lane owns V = 16 / sizeof(raw) consecutive channels
// c .. c+V-1 of batch row b.  With x and out unit-stride in channels and the state
// stored [B, C, K-1] contiguously, the lane's x and out of one step and its (K-1)*V
// history values are whole aligned vectors, and its K*V weights and V biases (WB
// bytes each, any of the three dtypes) whole 16- or 8-byte blocks: for bf16 with
// bf16 weights, K-1 + K + 2 loads and K stores cover V rows.  x and out are touched
// once and use streaming (non-temporal) accesses; the state, which the next decode
// step reads again, uses ordinary ones.
template <class S, int K, bool SILU, int WB>
__device__ inline void update_rows_vec(const UpdArgs& a, int64_t b, int64_t c) {
  using raw = typename S::raw;
  constexpr int V = S::V;
  constexpr int H = K - 1;
  constexpr int NWB = V * K * WB, NBB = V * WB;    // bytes of the lane's weights, biases
  const uintptr_t zero = reinterpret_cast<uintptr_t>(kZeroSrc);
  // Every load before any arithmetic: weights, bias, history and the first step's
  // x (a call with no new steps launches nothing, so L >= 1), so the lane waits
  // for one memory latency rather than one per kind of operand.
  uint32_t wv[NWB / 4], bv[NBB / 4];
  load_param_block<NWB>(reinterpret_cast<uintptr_t>(a.w) + c * K * WB, wv);
  load_param_block<NBB>(pick(a.bias != nullptr, reinterpret_cast<uintptr_t>(a.bias) + c * WB, zero), bv);
  u32x4 hv[H];
  raw* sp = static_cast<raw*>(a.state) + b * a.s_sb + c * H;
#pragma unroll
  for (int i = 0; i < H; ++i) hv[i] = gload<u32x4>(reinterpret_cast<uintptr_t>(sp + i * V));
  const uintptr_t xr = reinterpret_cast<uintptr_t>(static_cast<const raw*>(a.x) + b * a.x_sb + c);
  const uintptr_t xs = (uintptr_t)a.x_sl * sizeof(raw);
  u32x4 xv = gload16_stream(xr);
  __builtin_amdgcn_sched_barrier(0);               // keep every load above the arithmetic

  float w[V][K], beta[V];
  raw hist[V][H];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    beta[j] = param_f32<WB>(block_param_raw<WB>(bv, j), a.w_dtype);
#pragma unroll
    for (int k = 0; k < K; ++k) w[j][k] = param_f32<WB>(block_param_raw<WB>(wv, j * K + k), a.w_dtype);
#pragma unroll
    for (int i = 0; i < H; ++i) hist[j][i] = get_elem<S>(hv, j * H + i);
  }

  raw* orow = static_cast<raw*>(a.out) + b * a.o_sb + c;
  for (int64_t t = 0;;) {
    // the next step's x in flight during this step's arithmetic; none after the
    // last step (a load from the zero array there cost 6% of a one-step call's
    // kernel time, measured)
    u32x4 xn = {0u, 0u, 0u, 0u};
    if (t + 1 < a.L) xn = gload16_stream(xr + (uintptr_t)(t + 1) * xs);
    const u32x4 xcur[1] = {xv};
    float y[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const raw xe = get_elem<S>(xcur, j);
      float acc = beta[j];
#pragma unroll
      for (int k = 0; k < H; ++k) acc = __builtin_fmaf(w[j][k], S::to_f(hist[j][k]), acc);
      acc = __builtin_fmaf(w[j][H], S::to_f(xe), acc);
      y[j] = SILU ? silu(acc) : acc;
#pragma unroll
      for (int i = 0; i + 1 < H; ++i) hist[j][i] = hist[j][i + 1];
      hist[j][H - 1] = xe;
    }
    store16_stream(orow + t * a.o_sl, S::pack(y));
    if (++t >= a.L) break;
    xv = xn;
  }

  raw flat[V * H];
#pragma unroll
  for (int j = 0; j < V; ++j)
#pragma unroll
    for (int i = 0; i < H; ++i) flat[j * H + i] = hist[j][i];
  put_elems<S, V * H>(flat, hv);
#pragma unroll
  for (int i = 0; i < H; ++i) store16(sp + i * V, hv[i]);
}

template <class S, int K, bool SILU, bool VEC, int WB>
__global__ void __launch_bounds__(kUpdateBlock) update_kernel(const UpdArgs a) {
  if constexpr (VEC) {
    constexpr int V = S::V;
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * (kUpdateBlock / 64) + (threadIdx.x >> 6);
    const int64_t first = wave * (64 * V);         // the wave's 64 * V consecutive rows
    if (first >= a.rows) return;
    const int64_t b0 = first / a.C;                // wave-uniform: one division per wave
    int64_t b = b0, c = first - b0 * a.C + (int64_t)lane * V;
    if (c >= a.C) {                                // crossed into a later batch row
      const int64_t q = c / a.C;
      b += q;
      c -= q * a.C;
    }
    // C is a multiple of V, so a lane has all V of its rows or none.
    if (first + (int64_t)lane * V < a.rows) update_rows_vec<S, K, SILU, WB>(a, b, c);
    return;
  }
  using raw = typename S::raw;
  constexpr int H = K - 1;
  constexpr int R = kUpdateRowsPerLane;
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kUpdateBlock / 64) + (threadIdx.x >> 6);
  const int64_t first = wave * (64 * R);          // the wave's R * 64 consecutive rows
  if (first >= a.rows) return;                     // whole wave leaves together
  const int64_t b0 = first / a.C;                  // wave-uniform: one division per wave
  const int64_t c0 = first - b0 * a.C;

  // Phase 1: every load of the lane's R rows (R groups of 64 consecutive rows, so
  // each load instruction of the wave touches consecutive rows), issued before
  // any arithmetic.  Rows past the end load row rows-1 and store nothing.
  bool ok[R];
  int64_t bb[R], cc[R];
  float w[R][K], beta[R];
  raw hist[R][H];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int64_t r = first + j * 64 + lane;
    ok[j] = r < a.rows;
    int64_t b = b0, c = c0 + j * 64 + lane;
    if (c >= a.C) {                                // crossed into a later batch row
      const int64_t q = c / a.C;
      b += q;
      c -= q * a.C;
    }
    if (!ok[j]) {
      b = (a.rows - 1) / a.C;
      c = (a.rows - 1) - b * a.C;
    }
    bb[j] = b;
    cc[j] = c;
    load_params<K>(a.w, a.w_dtype, c * K, w[j]);
    beta[j] = a.bias ? load_param(a.bias, a.w_dtype, c) : 0.0f;
    const raw* st = static_cast<const raw*>(a.state) + b * a.s_sb + c * a.s_sc;
#pragma unroll
    for (int i = 0; i < H; ++i) hist[j][i] = st[i * a.s_si];
  }

  // Phase 2: the new steps, one at a time (the loads of a step's R rows together).
  for (int64_t t = 0; t < a.L; ++t) {
    raw xv[R];
#pragma unroll
    for (int j = 0; j < R; ++j)
      xv[j] = static_cast<const raw*>(a.x)[bb[j] * a.x_sb + cc[j] * a.x_sc + t * a.x_sl];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      float acc = beta[j];
#pragma unroll
      for (int k = 0; k < H; ++k) acc = __builtin_fmaf(w[j][k], S::to_f(hist[j][k]), acc);
      acc = __builtin_fmaf(w[j][H], S::to_f(xv[j]), acc);
      if (ok[j])
        static_cast<raw*>(a.out)[bb[j] * a.o_sb + cc[j] * a.o_sc + t * a.o_sl] =
            S::from_f(SILU ? silu(acc) : acc);
#pragma unroll
      for (int i = 0; i + 1 < H; ++i) hist[j][i] = hist[j][i + 1];
      hist[j][H - 1] = xv[j];
    }
  }

  // Phase 3: the new history, written only after the row's old one was read.
#pragma unroll
  for (int j = 0; j < R; ++j) {
    if (!ok[j]) continue;
    raw* st = static_cast<raw*>(a.state) + bb[j] * a.s_sb + cc[j] * a.s_sc;
#pragma unroll
    for (int i = 0; i < H; ++i) st[i * a.s_si] = hist[j][i];
  }
}

template <class S, int K>
int launch_k(const UpdArgs& a, bool silu, bool vec, uint32_t grid, void* st) {
  const void* fn;
  const bool w4 = a.w_dtype == CCV_DT_F32;        // the 16-byte path's weight width
  if (vec && w4)
    fn = silu ? reinterpret_cast<const void*>(&update_kernel<S, K, true, true, 4>)
              : reinterpret_cast<const void*>(&update_kernel<S, K, false, true, 4>);
  else if (vec)
    fn = silu ? reinterpret_cast<const void*>(&update_kernel<S, K, true, true, 2>)
              : reinterpret_cast<const void*>(&update_kernel<S, K, false, true, 2>);
  else
    fn = silu ? reinterpret_cast<const void*>(&update_kernel<S, K, true, false, 0>)
              : reinterpret_cast<const void*>(&update_kernel<S, K, false, false, 0>);
  void* args[] = {const_cast<UpdArgs*>(&a)};
  return (int)hipLaunchKernel(fn, dim3(grid), dim3(kUpdateBlock), args, 0, static_cast<hipStream_t>(st));
}

template <class S>
int launch_s(const UpdArgs& a, int K, bool silu, bool vec, uint32_t grid, void* st) {
  switch (K) {
    case 2: return launch_k<S, 2>(a, silu, vec, grid, st);
    case 3: return launch_k<S, 3>(a, silu, vec, grid, st);
    case 4: return launch_k<S, 4>(a, silu, vec, grid, st);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace

int launch_update(const UpdArgs& a, int dtype, int K, bool silu, bool vec, uint32_t grid, void* stream) {
  switch (dtype) {
    case CCV_DT_F32: return launch_s<F32>(a, K, silu, vec, grid, stream);
    case CCV_DT_F16: return launch_s<F16>(a, K, silu, vec, grid, stream);
    case CCV_DT_BF16: return launch_s<BF16>(a, K, silu, vec, grid, stream);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace ccv
