// ccv_update_launch.hpp -- launch descriptor of the update (decode) kernel, seen
// by the host validation code and the kernel.  No HIP types.
#pragma once

#include <stdint.h>

namespace ccv {

// Rows are numbered r = b * C + c.  Element path: wave w takes rows
// [w * 64 * R, (w + 1) * 64 * R), lane l of it rows w * 64 * R + j * 64 + l, j < R.
// 16-byte path (V = 16 / element size): wave w takes rows [w * 64 * V, (w + 1) * 64 * V),
// lane l of it the V rows from w * 64 * V + l * V.  Strides are in elements.
struct UpdArgs {
  const void* x;        // [B, C, L], x dtype
  void* out;            // [B, C, L], x dtype
  const void* w;        // [C, K] contiguous, w_dtype
  const void* bias;     // [C] or nullptr, w_dtype
  void* state;          // [B, C, K-1], x dtype; read, then overwritten
  int64_t C, L, rows;   // rows = B * C
  int64_t x_sb, x_sc, x_sl;
  int64_t o_sb, o_sc, o_sl;
  int64_t s_sb, s_sc, s_si;
  int32_t w_dtype;
};

constexpr int kUpdateBlock = 256;          // 4 waves
constexpr int kUpdateRowsPerLane = 4;      // R

// Launch one instance; returns a hipError_t value (0 = success).  vec selects the
// 16-byte path, which needs: C a multiple of V; x and out unit-stride in channels;
// the state stored [B, C, K-1] contiguously (s_i = 1, s_c = K-1); every base
// pointer and every used stride 16-byte aligned.  Weight and bias may take any of
// the three dtypes.
int launch_update(const UpdArgs& a, int dtype, int K, bool silu, bool vec, uint32_t grid, void* stream);

}  // namespace ccv
