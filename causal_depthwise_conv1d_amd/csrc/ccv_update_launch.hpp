// ccv_update_launch.hpp -- launch descriptor of the update (decode) kernel, seen
// by the host validation code and the kernel.  No HIP types.
#pragma once

#include <stdint.h>

namespace ccv {

// One thread per (b, c) row, rows numbered r = b * C + c.  Strides are in elements.
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

constexpr int kUpdateBlock = 256;

// Launch one instance; returns a hipError_t value (0 = success).
int launch_update(const UpdArgs& a, int dtype, int K, bool silu, uint32_t grid, void* stream);

}  // namespace ccv
