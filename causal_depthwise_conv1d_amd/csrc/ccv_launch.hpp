// ccv_launch.hpp -- internal launch descriptors passed by value to the kernels,
// and the launch entry of each kernel family.  Host and device code both see
// this header; it holds no HIP types so the validation code compiles anywhere.
#pragma once

#include <stdint.h>

namespace ccv {

enum { CCV_DT_F32 = 0, CCV_DT_F16 = 1, CCV_DT_BF16 = 2 };

// Fields common to both kernels.  Strides are in elements.
struct Common {
  const void* x;
  void* out;
  const void* w;        // [C, K] contiguous, w_dtype
  const void* bias;     // [C] or nullptr, w_dtype
  const int32_t* seq;   // [B, L] contiguous or nullptr
  const void* init;     // [B, C, K-1] or nullptr, x dtype
  void* fin;            // [B, C, K-1] or nullptr, x dtype
  int64_t B, C, L;
  int64_t is_b, is_c, is_i;   // initial_states strides
  int64_t fs_b, fs_c, fs_i;   // final_states strides
  int64_t nwork;              // wave work items
  uint32_t xcd_q, xcd_r;      // workgroups per XCD (quotient / remainder of G / 8); channel-last only
  int32_t w_dtype;
};

// Channel-first (s_L == 1 for x and out): a segment is `span` consecutive steps of
// one (b, c) row; a row has `nseg` segments, of which the first `nfull` lie wholly
// inside the row and take the 16-byte path (0 when the views are not aligned).
// Wave w of the `nwaves` launched takes, in three phases, whole segments
// w, w + nwaves, ... (numbered row by row), then the remaining partial segments,
// then the final states of rows w, w + nwaves, ...
struct CfArgs {
  Common m;
  int64_t x_sb, x_sc, o_sb, o_sc;
  int64_t span;    // 64 lanes * V * U
  int64_t nseg;    // segments per row
  int64_t nfull;   // whole 16-byte segments per row
  int64_t nwaves;  // waves launched
};

// Channel-last (s_C == 1 for x and out): a work item is a tile of `tile` time
// rows of one group of 64 * V channels of one batch; items are numbered with the
// channel group fastest, then the time tile, then the batch.  Wave w of the
// `nwaves` launched takes items w, w + nwaves, ..., then writes the final states
// of (batch, channel group) pairs w, w + nwaves, ...
struct ClArgs {
  Common m;
  int64_t x_sb, x_sl, o_sb, o_sl;
  int64_t tile;      // time rows per work item (a multiple of the row batch)
  int64_t ntt;       // time tiles per (b, channel group)
  int64_t ncg;       // channel groups
  int64_t nwaves;    // waves launched
  int32_t vec_init;  // initial_states rows load as aligned 16-byte channel vectors
  int32_t vec_seq;   // seq_idx rows load as aligned 16-byte vectors of 4 ids
  int32_t vec_par;   // weight and bias blocks of a lane load as aligned 16-byte vectors
  int32_t lds;       // 1: whole tiles staged through LDS (tile == kClLdsRows); 2: the
                     // transposing tile (kClTrChannels channels, one workgroup per item)
};

// Compute units of the GPU that `stream` (a hipStream_t; NULL = the current
// device's null stream) belongs to, read from the runtime once per device; -1 when
// the runtime cannot say.  last_cu_count(): the count of the device of the latest
// such query, 0 before any.
int device_cu_count(void* stream);
int last_cu_count();

// Launch one kernel instance; returns a hipError_t value (0 = success).
// dtype: CCV_DT_*; silu/seq/vec select the template instance.
int launch_cf(const CfArgs& a, int dtype, int K, bool silu, bool seq, bool vec,
              uint32_t grid, void* stream);
int launch_cl(const ClArgs& a, int dtype, int K, bool silu, bool seq, bool vec,
              uint32_t grid, void* stream);

// Compile-time work per lane, shared by the planner and the kernels.
constexpr int kWavesPerGroup = 4;
constexpr int kCfUnroll = 4;     // 16-byte vectors per lane per segment
constexpr int kClUnroll = 4;     // time rows loaded ahead per lane
constexpr int kClLdsRows = 16;   // rows of a tile staged through LDS
constexpr int kClTrChannels = 256;   // channels (threads) of a transposing tile
constexpr int cl_tr_rows(int es) { return es == 2 ? 64 : 32; }   // its time rows (LDS near 34 KB)
static_assert(kClTrChannels == 64 * kWavesPerGroup, "a transposing tile is one workgroup");

}  // namespace ccv
