// ccv_bwd_launch.hpp -- launch descriptors of the backward kernels, seen by the
// host validation code and the kernels.  No HIP types.
#pragma once

#include <stdint.h>

namespace ccv {

// Gradient kernel: one lane per (b, c) row and time tile [tt * T, tt * T + T).
// Lanes are numbered ((b * ntt + tt) * C + c), so a wave's lanes take consecutive
// channels.  Strides are in elements.
struct BwdArgs {
  const void* x;
  const void* w;            // [C, K] contiguous, w_dtype
  const void* bias;         // [C] or nullptr, w_dtype
  const int32_t* seq;       // [B, L] contiguous or nullptr
  const void* init;         // [B, C, K-1] or nullptr
  const void* dout;
  const void* dfs;          // [B, C, K-1] or nullptr
  void* dx;
  void* dinit;              // [B, C, K-1] or nullptr
  float* part;              // [B * ntt][K + 1][C] fp32 partial sums (dw taps, then db)
  int64_t B, C, L;
  int64_t x_sb, x_sc, x_sl;
  int64_t d_sb, d_sc, d_sl;     // dout
  int64_t g_sb, g_sc, g_sl;     // dx
  int64_t is_b, is_c, is_i;     // initial_states
  int64_t fs_b, fs_c, fs_i;     // dfinal_states
  int64_t di_b, di_c, di_i;     // dinitial_states
  int64_t T, ntt, lanes;        // tile length, tiles per row, B * ntt * C
  int32_t w_dtype;
};

// Reduction kernel: one lane per (slot, c), slot < K + 1; sums the B * ntt
// partials in a fixed order and writes dweight[c, slot] (slot < K) or dbias[c].
struct BwdReduceArgs {
  const float* part;
  void* dw;                 // [C, K], w_dtype
  void* db;                 // [C] or nullptr, w_dtype
  int64_t C, nparts;
  int32_t K, w_dtype;
};

constexpr int kBwdBlock = 256;
constexpr int kBwdTile = 64;        // T: time steps per lane
constexpr int kBwdChunk = 32;       // partials summed per chunk in the reduction

int launch_bwd(const BwdArgs& a, int dtype, int K, bool silu, bool seq, uint32_t grid, void* stream);
int launch_bwd_reduce(const BwdReduceArgs& r, uint32_t grid, void* stream);

}  // namespace ccv
