// ccv_bwd_launch.hpp -- launch descriptors of the backward kernels, seen by the
// host validation code and the kernels.  No HIP types.
#pragma once

#include <stdint.h>

namespace ccv {

// Gradient kernel: one lane per (b, c) row and group of tpi consecutive time
// tiles [tt * T, tt * T + T); the lane sums the parameter gradients of its whole
// group and writes one partial row.  Lanes are numbered
// ((b * ngr + g) * C + c), so a wave's lanes take consecutive channels.  Strides
// are in elements.
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
  float* part;              // [B * ngr][K + 1][C] fp32 partial sums (dw taps, then db)
  int64_t B, C, L;
  int64_t x_sb, x_sc, x_sl;
  int64_t d_sb, d_sc, d_sl;     // dout
  int64_t g_sb, g_sc, g_sl;     // dx
  int64_t is_b, is_c, is_i;     // initial_states
  int64_t fs_b, fs_c, fs_i;     // dfinal_states
  int64_t di_b, di_c, di_i;     // dinitial_states
  int64_t T, ntt, tpi, ngr, lanes;  // tile length, tiles per row, tiles per group, groups per row, B*ngr*C
  int64_t items;            // work items of the register channel-first kernel (one wave each)
  int32_t w_dtype;
  int32_t off24;            // channel strides of x, dout and dx below 2^24 bytes (24-bit lane offsets)
};

// Reduction over the partial rows, a tree of fixed shape: each level sums groups
// of kBwdFanIn consecutive rows in order, starting from zero, until one row is
// left.  A level kernel: lane (g, s) with s < (K + 1) * C sums
// in[32 g .. 32 g + 31][s] (fewer in the last group) into out[g][s].  The final
// kernel does the last two levels at once for n_in <= kBwdFanIn * kBwdFinalWaves
// rows: a workgroup of ceil(n_in / 32) waves takes 64 columns, wave w sums rows
// 32 w .. 32 w + 31, and one wave sums the wave sums in order, which is exactly
// the arithmetic of the two levels; it rounds the result to the weight dtype and
// writes dweight[c, slot] (slot < K) or dbias[c] (slot = K).
struct BwdReduceArgs {
  const float* in;          // [n_in][(K + 1) * C]
  float* out;               // [ceil(n_in / 32)][(K + 1) * C] (level kernel)
  void* dw;                 // [C, K], w_dtype (final kernel)
  void* db;                 // [C] or nullptr, w_dtype (final kernel)
  int64_t C, n_in;
  int32_t K, w_dtype;
};

constexpr int kBwdBlock = 256;      // element path: lanes per workgroup
// Consecutive tiles summed into one partial row when x is unit-stride in channels
// (a step of 64 channels is whole cache lines).  With unit stride in time a tile's
// row segment is half a cache line, and the neighbouring tile is better run at
// the same time by another wave than after this one: then one tile per row.
constexpr int kBwdTilesPerItem = 4;
constexpr int kBwdFanIn = 32;       // partial sums added per lane and level of the reduction
constexpr int kBwdFinalWaves = 16;  // waves of the final reduction kernel's workgroups, at most

// Gradient kernel variants: the element path (one lane per (b, tile group, c), any
// strides; grid = ceil(lanes / kBwdBlock)) and the LDS-staged paths (one 64-lane
// workgroup per (b, tile group, 64 channels); grid = B * ngr * ceil(C / 64)),
// which need x, dout and dx unit-stride in the same dimension (time for CF,
// channels for CL), 16-byte aligned bases and strides, and L (CF) or C (CL) a
// multiple of 16 / element size.
// kBwdPathRegCfOdd and kBwdPathLdsClOdd are the register channel-first and the
// LDS-staged channel-last paths on rows that are not 16-byte aligned (kernel
// instantiations of their own, so that the aligned kernels' code is unchanged);
// the plan reports them as kBwdPathRegCf and kBwdPathLdsCl.
enum { kBwdPathElement = 0, kBwdPathLdsCf = 1, kBwdPathLdsCl = 2, kBwdPathRegCf = 3, kBwdPathRegCfOdd = 4,
       kBwdPathLdsClOdd = 5 };

// The register-only channel-first path (x, dout and dx unit-stride in time, any
// alignment; with seq_idx, a 16-byte aligned seq_idx): work items are
// segments of bwd_reg_span(dtype) steps of
// one (b, c) row, numbered row-major; a partial row per (b, segment); a grid of
// kBwdBlock-lane workgroups, one wave per item.
int bwd_reg_span(int dtype);

// Time steps per tile T for a dtype (32 for all three; both paths use the same T,
// so their partial sums, and so dweight and dbias, are identical).
int bwd_tile_steps(int dtype);

int launch_bwd(const BwdArgs& a, int dtype, int K, bool silu, bool seq, int path, uint32_t grid,
               void* stream);
int launch_bwd_reduce(const BwdReduceArgs& r, uint32_t grid, void* stream);
int launch_bwd_reduce_final(const BwdReduceArgs& r, uint32_t grid, int waves, void* stream);

// Rows the reduction needs after the B * ngr partial rows: the outputs of the
// level kernels, which run while more rows are left than the final kernel takes.
inline int64_t bwd_reduce_rows(int64_t nparts) {
  int64_t rows = 0;
  for (int64_t n = nparts; n > (int64_t)kBwdFanIn * kBwdFinalWaves;) {
    n = (n + kBwdFanIn - 1) / kBwdFanIn;
    rows += n;
  }
  return rows;
}

}  // namespace ccv
