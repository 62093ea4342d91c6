// ccv_cl.hip -- channel-last forward (x and out have unit stride in channels; the
// time stride s_L may exceed C, e.g. a slice of a wider projection buffer, and is
// used as given: Ch.4 "Dao interface and source map", section "Why one shape
// still has two layouts").
//
// Same arithmetic as the channel-first kernel (Ch.5 "Dao forward CUDA
// implementation", stencil equation for z_i).  Work split: a wave owns 64 * V
// consecutive channels (lane l holds one 16-byte vector of V channels) of one
// batch, over a tile of consecutive time rows.  Each load or store instruction
// of the wave moves one 1 KB channel row, so access is coalesced along channels;
// each lane then walks time with its own K-1 rows of history in registers.  The
// tile's first output reads the K-1 rows above the tile from memory (or from
// initial_states / zeros at t = 0), so tiles are independent (Ch.5, section "Why
// the channel-contiguous path reorganises": time tiles as independent blocks,
// each reading its own left halo).  Since a lane already computes along time for
// fixed channels, no LDS transpose is needed for either the loads or the stores.
//
// Items are numbered with the channel group fastest, so the waves running at
// one time read neighbouring 1 KB pieces of the same rows.  A whole tile of
// whole channel vectors runs on a straight-line path: its parameter, history and
// first row-batch loads are issued before any wait, and each next batch of rows
// is issued before the current batch's arithmetic.  seq_idx ids are shared by all
// channels of a row, so the masks are wave-uniform, and a batch whose window
// holds one sequence skips the masking altogether.
#include <type_traits>

#include "ccv_device.hpp"

namespace ccv {

struct TilePos {
  int64_t b, cg, tt;
};

__device__ inline TilePos tile_pos(const ClArgs& a, int64_t item) {
  const int64_t cg = item % a.ncg;
  const int64_t rest = item / a.ncg;
  return TilePos{rest / a.ntt, cg, rest % a.ntt};
}

// The K-tap stencil (and SiLU) for one time row of this lane's V channels.
// rows[k] is the extended input row t-H+k (k = K-1 is row t itself).  MASKED
// is a template argument so that the unmasked form holds no selects at all.
template <class S, int K, bool SILU, bool MASKED>
__device__ inline void row_stencil(const float (&w)[S::V][K], const float (&beta)[S::V],
                                   const float* const (&rows)[K], const bool (&keep)[K],
                                   float (&y)[S::V]) {
#pragma unroll
  for (int i = 0; i < S::V; ++i) {
    float acc = beta[i];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      if (MASKED) acc = keep[k] ? __builtin_fmaf(w[i][k], rows[k][i], acc) : acc;
      else acc = __builtin_fmaf(w[i][k], rows[k][i], acc);
    }
    y[i] = SILU ? silu(acc) : acc;
  }
}

// ---- whole tiles: straight-line path ---------------------------------------------

// Addresses are a wave-uniform base plus this lane's 32-bit offset, so the loads
// and stores use the scalar-base addressing mode.
//
// Two ways to keep rows in flight.  Registers (LDSM false): each next batch
// of U rows is loaded into registers before the current batch's arithmetic.  LDS
// (LDSM; rows = this wave's region of kClLdsRows x 1 KB, the tile that long): every row
// of the tile goes straight from global memory into LDS with 16-byte
// global-to-LDS loads, one 1 KB row per instruction, before any arithmetic; each
// lane then reads its own 16 bytes of each row back.  The rows then take no
// registers while in flight, so more waves fit on a CU; the arithmetic is the
// same, term for term.
typedef u32x4 __attribute__((address_space(3))) lds_u32x4;

template <class S, int K, bool SILU, bool SEQ, int WB, bool LDSM>
__device__ inline void tile_fast(const ClArgs& a, const TilePos& p, int lane, lds_u32x4* rows) {
  constexpr int V = S::V;
  constexpr int U = kClUnroll;
  constexpr int H = K - 1;
  constexpr int ES = sizeof(typename S::raw);
  constexpr int NWB = V * K * WB;                    // bytes of a lane's weights
  constexpr int NBB = V * WB;                        // bytes of a lane's biases
  static_assert(U == 4 && U >= H, "a row batch is 4 rows and covers the history");
  const Common& m = a.m;
  const uintptr_t zero = reinterpret_cast<uintptr_t>(kZeroSrc);
  const int64_t cbase = p.cg * (64 * V);             // the wave's first channel
  const int64_t t0 = p.tt * a.tile;
  const uint32_t lx = (uint32_t)lane * (V * ES);     // lane offset inside a row
  const uintptr_t xb = reinterpret_cast<uintptr_t>(m.x) + (p.b * a.x_sb + cbase) * ES;
  const uintptr_t ob = reinterpret_cast<uintptr_t>(m.out) + (p.b * a.o_sb + cbase) * ES;
  const uintptr_t xs = a.x_sl * ES, os = a.o_sl * ES;
  const uintptr_t sr = reinterpret_cast<uintptr_t>(m.seq) + p.b * m.L * 4;

  // Parameters and history first: waiting for them later leaves the row batches
  // issued after them in flight.
  uint32_t wv[NWB / 4], bv[NBB / 4];
  const uintptr_t wl = reinterpret_cast<uintptr_t>(m.w) + cbase * K * WB;
  load_param_block<NWB>(wl + (uint32_t)lane * NWB, wv);
  const uintptr_t bl = pick(m.bias != nullptr, reinterpret_cast<uintptr_t>(m.bias) + cbase * WB, zero);
  load_param_block<NBB>(bl + (uint32_t)lane * NBB, bv);
  u32x4 hv[H];
  const uintptr_t il = reinterpret_cast<uintptr_t>(m.init) + (p.b * m.is_b + cbase) * ES;
#pragma unroll
  for (int j = 0; j < H; ++j) {
    const uintptr_t from_x = xb + (t0 - H + j) * xs;
    const uintptr_t from_init = pick(m.init != nullptr, il + j * m.is_i * ES, zero);
    hv[j] = gload<u32x4>(pick(t0 >= H, from_x, from_init) + lx);
  }
  // Ids of the U rows above the tile; at t = 0 the history's id is seq_idx[b, 0].
  u32x4 hid_v = {0u, 0u, 0u, 0u};
  if constexpr (SEQ) hid_v = gload<u32x4>(pick(t0 >= U, sr + (t0 - U) * 4, pick(m.init != nullptr, sr, zero)));

  // Row batches: A holds the current batch, B the next one.
  u32x4 ra[U], rb[U], ia = {0u, 0u, 0u, 0u}, ib = {0u, 0u, 0u, 0u};
  auto issue = [&](int64_t t, u32x4 (&r)[U], u32x4& iv) {
#pragma unroll
    for (int u = 0; u < U; ++u) r[u] = gload16_stream(xb + (t + u) * xs + lx);
    if constexpr (SEQ) iv = gload<u32x4>(sr + t * 4);
  };
  constexpr int NLB = kClLdsRows / U;               // row batches of an LDS tile
  if constexpr (LDSM) {
#pragma unroll
    for (int r = 0; r < kClLdsRows; ++r)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(xb + (t0 + r) * xs + lx),
                                       reinterpret_cast<__attribute__((address_space(3))) void*>(rows + r * 64),
                                       16, 0, 0);
    // The tile's ids after its rows: lane i < kClLdsRows brings the id of row t0 + i.
    if constexpr (SEQ)
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const void*>(pick(lane < kClLdsRows, sr + (t0 + lane) * 4, zero)),
          reinterpret_cast<__attribute__((address_space(3))) void*>(rows + kClLdsRows * 64), 4, 0, 0);
  } else {
    issue(t0, ra, ia);
  }

  // Convert parameters and history (waits for them only).
  float w[V][K], beta[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      w[i][k] = param_f32<WB>(block_param_raw<WB>(wv, i * K + k), m.w_dtype);
    }
    beta[i] = param_f32<WB>(block_param_raw<WB>(bv, i), m.w_dtype);
  }
  // Sliding window of the last K rows as fp32: win[0] is the oldest.
  float win[K][V];
#pragma unroll
  for (int j = 0; j < H; ++j) S::unpack(hv[j], win[j + 1]);
  // Ids of the window rows.  Rows left of t = 0 are the history of the row's first
  // sequence (id seq_idx[b, 0]); without a history they never count.
  int wid[K];
  bool wok[K];
#pragma unroll
  for (int j = 0; j < H; ++j) {
    wid[j + 1] = SEQ ? __builtin_amdgcn_readfirstlane((int)dword(hid_v, t0 >= U ? U - H + j : 0)) : 0;
    wok[j + 1] = t0 - H + j >= 0 || m.init != nullptr;
  }

  auto compute = [&](int64_t t, const u32x4 (&r)[U], const u32x4& iv) {
    int id[U];
    bool masked = false;
    if constexpr (SEQ) {
#pragma unroll
      for (int u = 0; u < U; ++u) id[u] = __builtin_amdgcn_readfirstlane((int)dword(iv, u));
      // One sequence across the whole window (history and batch): no masking.
      bool one = true;
#pragma unroll
      for (int u = 1; u < U; ++u) one = one && id[u] == id[0];
#pragma unroll
      for (int j = 1; j < K; ++j) one = one && wok[j] && wid[j] == id[0];
      masked = !one;
    }
    // The batch's rows, with or without the masks; two copies of the code, chosen
    // per batch on a wave-uniform flag (as one code with the flag folded into
    // every term, each output paid K-1 selects).
    auto batch = [&](auto masked_c) {
      constexpr bool MASKED = decltype(masked_c)::value;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        // Slide: drop the oldest row, append row t + u.
#pragma unroll
        for (int j = 0; j < H; ++j) {
#pragma unroll
          for (int i = 0; i < V; ++i) win[j][i] = win[j + 1][i];
          wid[j] = wid[j + 1];
          wok[j] = wok[j + 1];
        }
        S::unpack(r[u], win[H]);
        wid[H] = SEQ ? id[u] : 0;
        wok[H] = true;
        const float* rows[K];
        bool keep[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
          rows[k] = win[k];
          keep[k] = !SEQ || (wok[k] && wid[k] == wid[H]);
        }
        float y[V];
        row_stencil<S, K, SILU, MASKED>(w, beta, rows, keep, y);
        gstore16_stream(ob + (t + u) * os + lx, S::pack(y));
      }
    };
    if (SEQ && __builtin_expect(masked, 0)) batch(std::true_type{});
    else batch(std::false_type{});
  };

  if constexpr (LDSM) {
    // Wait for every global-to-LDS load of the tile before the first read of it.
    // The compiler's own waits do not cover these loads reliably: it once left the
    // ids' load in flight at the first read of the ids, so a batch could take the
    // previous tile's ids and the wrong masks.
    __builtin_amdgcn_s_waitcnt(0x0F70);            // vmcnt(0); expcnt, lgkmcnt not waited
#pragma unroll 1
    for (int j = 0; j < NLB; ++j) {
#pragma unroll
      for (int u = 0; u < U; ++u) ra[u] = rows[(j * U + u) * 64 + lane];
      if constexpr (SEQ) ia = rows[kClLdsRows * 64 + j];   // 4 ids, the same for every lane
      compute(t0 + j * U, ra, ia);
    }
    return;
  }
  const int64_t nb = a.tile / U;
  int64_t j = 0;
  while (true) {
    if (j + 1 >= nb) {
      compute(t0 + j * U, ra, ia);
      break;
    }
    issue(t0 + (j + 1) * U, rb, ib);
    compute(t0 + j * U, ra, ia);
    ++j;
    if (j + 1 >= nb) {
      compute(t0 + j * U, rb, ib);
      break;
    }
    issue(t0 + (j + 1) * U, ra, ia);
    compute(t0 + j * U, rb, ib);
    ++j;
  }
}

// ---- any tile: element-wise general path ---------------------------------------

template <class S, int K, bool SILU, bool SEQ, bool VEC>
__device__ inline void tile_general(const ClArgs& a, const TilePos& p, int lane) {
  constexpr int V = S::V;
  constexpr int U = kClUnroll;
  constexpr int H = K - 1;
  using raw = typename S::raw;
  const Common& m = a.m;
  const int64_t L = m.L;
  const int64_t c0 = p.cg * (64 * V) + lane * V;
  const int nch = (int)(m.C - c0 < V ? (m.C - c0 > 0 ? m.C - c0 : 0) : V);
  const bool full = VEC && nch == V;
  const int64_t t0 = p.tt * a.tile;
  const int64_t t1 = (t0 + a.tile < L) ? t0 + a.tile : L;
  if (t0 >= t1) return;

  const raw* __restrict__ xb = static_cast<const raw*>(m.x) + p.b * a.x_sb + c0;
  raw* __restrict__ ob = static_cast<raw*>(m.out) + p.b * a.o_sb + c0;
  const raw* __restrict__ ib = static_cast<const raw*>(m.init);
  const int32_t* __restrict__ sr = SEQ ? m.seq + p.b * L : nullptr;

  float w[V][K], beta[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const bool in = i < nch;
#pragma unroll
    for (int k = 0; k < K; ++k) w[i][k] = in ? load_param(m.w, m.w_dtype, (c0 + i) * K + k) : 0.0f;
    beta[i] = (in && m.bias) ? load_param(m.bias, m.w_dtype, c0 + i) : 0.0f;
  }

  // History rows X~[t0-H .. t0-1] for this lane's channels.
  float hist[H][V];
  int hid[H];
  bool hok[H];
#pragma unroll
  for (int j = 0; j < H; ++j) {
    const int64_t src = t0 - H + j;
    if (src >= 0) {
      if (full) {
        S::unpack(load16(xb + src * a.x_sl), hist[j]);
      } else {
#pragma unroll
        for (int i = 0; i < V; ++i) hist[j][i] = i < nch ? S::to_f(xb[src * a.x_sl + i]) : 0.0f;
      }
    } else {
#pragma unroll
      for (int i = 0; i < V; ++i)
        hist[j][i] = (ib && i < nch) ? S::to_f(ib[p.b * m.is_b + (c0 + i) * m.is_c + (src + H) * m.is_i]) : 0.0f;
    }
    hok[j] = src >= 0 || ib != nullptr;              // the history: the first sequence's
    hid[j] = SEQ ? (src >= 0 ? sr[src] : (ib ? sr[0] : 0)) : 0;
  }

  for (int64_t t = t0; t < t1; t += U) {
    float e[U][V];
    int id[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t tr = t + u;
      if (tr < t1) {
        if (full) {
          S::unpack(load16(xb + tr * a.x_sl), e[u]);
        } else {
#pragma unroll
          for (int i = 0; i < V; ++i) e[u][i] = i < nch ? S::to_f(xb[tr * a.x_sl + i]) : 0.0f;
        }
        id[u] = SEQ ? sr[tr] : 0;
      } else {
#pragma unroll
        for (int i = 0; i < V; ++i) e[u][i] = 0.0f;
        id[u] = 0;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t tr = t + u;
      const float* rows[K];
      bool keep[K];
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int rr = u - H + k;
        rows[k] = rr >= 0 ? e[rr] : hist[H + rr];
        keep[k] = !SEQ || (rr >= 0 ? id[rr] == id[u] : (hok[H + rr] && hid[H + rr] == id[u]));
      }
      float y[V];
      row_stencil<S, K, SILU, SEQ>(w, beta, rows, keep, y);
      if (tr < t1) {
        if (full) {
          store16(ob + tr * a.o_sl, S::pack(y));
        } else {
#pragma unroll
          for (int i = 0; i < V; ++i)
            if (i < nch) ob[tr * a.o_sl + i] = S::from_f(y[i]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < H; ++j) {
#pragma unroll
      for (int i = 0; i < V; ++i) hist[j][i] = e[U - H + j][i];
      hid[j] = id[U - H + j];
      hok[j] = true;
    }
  }
}

// final_states of one (batch, channel group): the last K-1 extended inputs of the
// lane's channels, bit for bit (Ch.5, section "Three kinds of boundary handled
// separately"); with seq_idx, those of the row's last sequence only.
template <class S, int K>
__device__ inline void final_states_group(const ClArgs& a, int64_t b, int64_t cg, int lane) {
  constexpr int V = S::V;
  constexpr int H = K - 1;
  using raw = typename S::raw;
  const Common& m = a.m;
  const int64_t L = m.L;
  const int64_t c0 = cg * (64 * V) + lane * V;
  const int nch = (int)(m.C - c0 < V ? (m.C - c0 > 0 ? m.C - c0 : 0) : V);
  const raw* __restrict__ xb = static_cast<const raw*>(m.x) + b * a.x_sb + c0;
  const raw* __restrict__ ib = static_cast<const raw*>(m.init);
  raw* __restrict__ fb = static_cast<raw*>(m.fin) + b * m.fs_b;
  for (int i = 0; i < nch; ++i) {
#pragma unroll
    for (int j = 0; j < H; ++j) {
      const int64_t src = L - H + j;
      raw v;
      if (src >= 0) v = xb[src * a.x_sl + i];
      else if (ib) v = ib[b * m.is_b + (c0 + i) * m.is_c + (src + H) * m.is_i];
      else v = 0;
      if (!final_kept(m.seq ? m.seq + b * L : nullptr, L, src, ib != nullptr)) v = 0;
      fb[(c0 + i) * m.fs_c + j * m.fs_i] = v;
    }
  }
}

// The last channel group when it holds only a few channels (C not a multiple of
// 64 * V, at most kClNarrowVectors * V channels left): lane r takes time row t0 + r
// of the tile and walks the group's channels, so a wave moves up to 64 rows per
// instruction where the general code would keep a lane or two busy.  The
// arithmetic is the general code's, term for term (bias first, then the taps
// oldest first, the history from initial_states or zeros, the same masks).
constexpr int kClNarrowVectors = 4;

template <class S, int K, bool SILU, bool SEQ>
__device__ inline void tile_narrow(const ClArgs& a, const TilePos& p, int lane) {
  constexpr int H = K - 1;
  using raw = typename S::raw;
  const Common& m = a.m;
  const int64_t L = m.L;
  const int64_t c0 = p.cg * (64 * S::V);
  const int nch = (int)(m.C - c0);
  const int64_t t0 = p.tt * a.tile;
  const int64_t t1 = (t0 + a.tile < L) ? t0 + a.tile : L;
  const raw* __restrict__ xb = static_cast<const raw*>(m.x) + p.b * a.x_sb + c0;
  raw* __restrict__ ob = static_cast<raw*>(m.out) + p.b * a.o_sb + c0;
  const raw* __restrict__ ib = static_cast<const raw*>(m.init);
  const int32_t* __restrict__ sr = SEQ ? m.seq + p.b * L : nullptr;
  for (int64_t t = t0 + lane; t < t1; t += 64) {
    const int id = SEQ ? sr[t] : 0;
    bool keep[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int64_t src = t - H + k;               // left of t = 0: the first sequence's history
      keep[k] = !SEQ || (src >= 0 ? sr[src] == id : (ib != nullptr && sr[0] == id));
    }
    for (int i = 0; i < nch; ++i) {
      const int64_t c = c0 + i;
      float acc = m.bias ? load_param(m.bias, m.w_dtype, c) : 0.0f;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int64_t src = t - H + k;
        const float xv = src >= 0 ? S::to_f(xb[src * a.x_sl + i])
                                  : (ib ? S::to_f(ib[p.b * m.is_b + c * m.is_c + (src + H) * m.is_i]) : 0.0f);
        const float f = __builtin_fmaf(load_param(m.w, m.w_dtype, c * K + k), xv, acc);
        acc = SEQ ? (keep[k] ? f : acc) : f;
      }
      ob[t * a.o_sl + i] = S::from_f(SILU ? silu(acc) : acc);
    }
  }
}

template <class S, int K, bool SILU, bool SEQ, bool VEC, int WB, bool LDSM>
__device__ inline void cl_fwd_body(const ClArgs& a, lds_u32x4* rows) {
  constexpr int V = S::V;
  const Common& m = a.m;
  const int lane = threadIdx.x & 63;
  const uint32_t g = xcd_order(blockIdx.x, m.xcd_q, m.xcd_r);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t w0 = (int64_t)g * kWavesPerGroup + wave;
  if (w0 >= a.nwaves) return;                       // whole wave leaves together
  const int64_t W = a.nwaves;

  if (m.L > 0) {
    for (int64_t it = w0; it < m.nwork; it += W) {
      const TilePos p = tile_pos(a, it);
      if constexpr (VEC) {
        const int64_t t0 = p.tt * a.tile;
        const bool fast = a.vec_par && (a.tile % kClUnroll) == 0 && (p.cg + 1) * (64 * V) <= m.C &&
                          t0 + a.tile <= m.L &&
                          (t0 >= K - 1 || m.init == nullptr || a.vec_init) && (!SEQ || a.vec_seq);
        if (fast) {
          tile_fast<S, K, SILU, SEQ, WB, LDSM>(a, p, lane, LDSM ? rows + wave * (kClLdsRows * 64 + 16) : rows);
          continue;
        }
        if (m.C - p.cg * (64 * V) <= kClNarrowVectors * V) {
          tile_narrow<S, K, SILU, SEQ>(a, p, lane);
          continue;
        }
      }
      tile_general<S, K, SILU, SEQ, VEC>(a, p, lane);
    }
  }
  if (m.fin) {
    const int64_t pairs = m.B * a.ncg;
    for (int64_t r = w0; r < pairs; r += W) final_states_group<S, K>(a, r / a.ncg, r % a.ncg, lane);
  }
}

template <class S, int K, bool SILU, bool SEQ, bool VEC, int WB>
__global__ void __launch_bounds__(256) cl_fwd_kernel(const ClArgs a) {
  cl_fwd_body<S, K, SILU, SEQ, VEC, WB, false>(a, nullptr);
}

// The same work with whole tiles staged through LDS (tiles of kClLdsRows rows):
// per wave kClLdsRows KB of rows and 256 bytes of ids.
constexpr int kClLdsWaveVecs = kClLdsRows * 64 + 16;

template <class S, int K, bool SILU, bool SEQ, int WB>
__global__ void __launch_bounds__(256) cl_fwd_lds_kernel(const ClArgs a) {
  __shared__ u32x4 rows[kWavesPerGroup * kClLdsWaveVecs];
  cl_fwd_body<S, K, SILU, SEQ, true, WB, true>(a, (lds_u32x4*)rows);
}

// ---- the pages' tile, for comparison: load, change direction, compute, change back
//
// Ch.5 "Dao forward CUDA implementation", section "Load first, then change the
// access direction": a workgroup stages a tile of time rows x channels in LDS with
// loads along channels, each thread then owns one channel and runs its time
// steps out of LDS, writes its outputs back into the tile, and the tile is stored
// along channels again.  Here: kClTrChannels channels (one per thread) x TT rows
// plus the K-1 rows above; the outputs overwrite their own inputs in place (a
// thread's window already holds the history it needs).  All threads read and
// write the same row at once, consecutive elements, so the tile needs no padding.
// The arithmetic is the register path's term for term, so the bits are the same.
// Opt-in (CCV_CL_LDS=2), for C a multiple of 16 / element size with aligned rows.
template <class S>
struct TrTile {
  static constexpr int ES = sizeof(typename S::raw);
  static constexpr int TT = cl_tr_rows(ES);                  // time rows per tile
  static constexpr int CHUNKS = kClTrChannels * ES / 16;     // 16-byte pieces per row
};

template <class S, int K, bool SILU, bool SEQ>
__global__ void __launch_bounds__(kClTrChannels) cl_fwd_tr_kernel(const ClArgs a) {
  using raw = typename S::raw;
  using G = TrTile<S>;
  constexpr int H = K - 1, TT = G::TT, ROWS = TT + H, V = 16 / G::ES, N = kClTrChannels;
  __shared__ u32x4 tile[ROWS * G::CHUNKS];
  __shared__ int ids[ROWS];
  const Common& m = a.m;
  const int tid = threadIdx.x;
  const int64_t item = xcd_order(blockIdx.x, m.xcd_q, m.xcd_r);
  const int64_t cb = item % a.ncg, rest = item / a.ncg;
  const int64_t b = rest / a.ntt, t0 = (rest % a.ntt) * TT;
  const int64_t c0 = cb * N, L = m.L, C = m.C;
  const raw* xb = static_cast<const raw*>(m.x) + b * a.x_sb;
  const raw* ib = static_cast<const raw*>(m.init);

  // Load along channels: rows t0-H .. t0+TT-1 (history or zeros left of t = 0,
  // zeros past L or C), and the rows' sequence ids (the history's: seq_idx[b, 0]).
  for (int q = tid; q < ROWS * G::CHUNKS; q += N) {
    const int r = q / G::CHUNKS, k = q - r * G::CHUNKS;
    const int64_t t = t0 - H + r, c = c0 + (int64_t)k * V;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (c < C && t >= 0 && t < L) {
      v = load16(xb + t * a.x_sl + c);
    } else if (c < C && t < 0 && ib) {
      raw e[V];
#pragma unroll
      for (int i = 0; i < V; ++i) e[i] = ib[b * m.is_b + (c + i) * m.is_c + (t + H) * m.is_i];
      __builtin_memcpy(&v, e, 16);
    }
    tile[q] = v;
  }
  if constexpr (SEQ) {
    for (int r = tid; r < ROWS; r += N) {
      const int64_t t = t0 - H + r;
      ids[r] = (t >= 0 && t < L) ? m.seq[b * L + t] : (t < 0 && L > 0 ? m.seq[b * L] : 0);
    }
  }
  __syncthreads();

  // Change direction: this thread's channel, along time.
  const int64_t c = c0 + tid;
  raw* col = reinterpret_cast<raw*>(tile) + tid;   // element (row r, this channel) at col[r * N]
  if (c < C) {
    float w[K];
    load_params<K>(m.w, m.w_dtype, c * K, w);
    const float beta = m.bias ? load_param(m.bias, m.w_dtype, c) : 0.0f;
    float win[K];
    int wid[K];
    bool wok[K];
#pragma unroll
    for (int j = 0; j < H; ++j) {
      win[j + 1] = S::to_f(col[j * N]);
      wid[j + 1] = SEQ ? ids[j] : 0;
      wok[j + 1] = t0 - H + j >= 0 || ib != nullptr;
    }
    for (int r = 0; r < TT && t0 + r < L; ++r) {
#pragma unroll
      for (int j = 0; j < H; ++j) {
        win[j] = win[j + 1];
        wid[j] = wid[j + 1];
        wok[j] = wok[j + 1];
      }
      win[H] = S::to_f(col[(H + r) * N]);
      wid[H] = SEQ ? ids[H + r] : 0;
      wok[H] = true;
      float acc = beta;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const float f = __builtin_fmaf(w[k], win[k], acc);
        acc = (!SEQ || (wok[k] && wid[k] == wid[H])) ? f : acc;
      }
      col[(H + r) * N] = S::from_f(SILU ? silu(acc) : acc);   // over its own input
    }
    // final_states: the tile that holds the row's end writes this channel's.
    if (m.fin && t0 + TT >= L) {
      const int32_t* sr = m.seq ? m.seq + b * L : nullptr;
#pragma unroll
      for (int j = 0; j < H; ++j) {
        const int64_t src = L - H + j;
        raw v = 0;
        if (src >= 0) v = xb[src * a.x_sl + c];
        else if (ib) v = ib[b * m.is_b + c * m.is_c + (src + H) * m.is_i];
        if (!final_kept(sr, L, src, ib != nullptr)) v = 0;
        static_cast<raw*>(m.fin)[b * m.fs_b + c * m.fs_c + j * m.fs_i] = v;
      }
    }
  }
  __syncthreads();

  // Change back: store along channels.
  raw* ob = static_cast<raw*>(m.out) + b * a.o_sb;
  for (int q = tid; q < TT * G::CHUNKS; q += N) {
    const int r = q / G::CHUNKS, k = q - r * G::CHUNKS;
    const int64_t t = t0 + r, cc = c0 + (int64_t)k * V;
    if (t < L && cc < C) store16_stream(ob + t * a.o_sl + cc, tile[(H + r) * G::CHUNKS + k]);
  }
}

template <class S, int K, bool SILU, bool SEQ, bool VEC, int WB>
static int launch_one(const ClArgs& a, uint32_t grid, void* stream) {
  void* args[] = {const_cast<ClArgs*>(&a)};
  if (VEC && a.lds == 2)
    return (int)hipLaunchKernel(reinterpret_cast<const void*>(&cl_fwd_tr_kernel<S, K, SILU, SEQ>), dim3(grid),
                                dim3(kClTrChannels), args, 0, static_cast<hipStream_t>(stream));
  const void* fn = VEC && a.lds ? reinterpret_cast<const void*>(&cl_fwd_lds_kernel<S, K, SILU, SEQ, WB>)
                                : reinterpret_cast<const void*>(&cl_fwd_kernel<S, K, SILU, SEQ, VEC, WB>);
  return (int)hipLaunchKernel(fn, dim3(grid), dim3(64 * kWavesPerGroup), args, 0, static_cast<hipStream_t>(stream));
}

template <class S, int K, bool SILU, bool SEQ, bool VEC>
static int launch_w(const ClArgs& a, uint32_t grid, void* st) {
  return a.m.w_dtype == CCV_DT_F32 ? launch_one<S, K, SILU, SEQ, VEC, 4>(a, grid, st)
                                   : launch_one<S, K, SILU, SEQ, VEC, 2>(a, grid, st);
}

template <class S, int K>
static int launch_k(const ClArgs& a, bool silu, bool seq, bool vec, uint32_t grid, void* st) {
  if (silu) {
    if (seq) return vec ? launch_w<S, K, true, true, true>(a, grid, st) : launch_w<S, K, true, true, false>(a, grid, st);
    return vec ? launch_w<S, K, true, false, true>(a, grid, st) : launch_w<S, K, true, false, false>(a, grid, st);
  }
  if (seq) return vec ? launch_w<S, K, false, true, true>(a, grid, st) : launch_w<S, K, false, true, false>(a, grid, st);
  return vec ? launch_w<S, K, false, false, true>(a, grid, st) : launch_w<S, K, false, false, false>(a, grid, st);
}

template <class S>
static int launch_s(const ClArgs& a, int K, bool silu, bool seq, bool vec, uint32_t grid, void* st) {
  switch (K) {
    case 2: return launch_k<S, 2>(a, silu, seq, vec, grid, st);
    case 3: return launch_k<S, 3>(a, silu, seq, vec, grid, st);
    case 4: return launch_k<S, 4>(a, silu, seq, vec, grid, st);
  }
  return (int)hipErrorInvalidValue;
}

int launch_cl(const ClArgs& a, int dtype, int K, bool silu, bool seq, bool vec, uint32_t grid,
              void* stream) {
  switch (dtype) {
    case CCV_DT_F32: return launch_s<F32>(a, K, silu, seq, vec, grid, stream);
    case CCV_DT_F16: return launch_s<F16>(a, K, silu, seq, vec, grid, stream);
    case CCV_DT_BF16: return launch_s<BF16>(a, K, silu, seq, vec, grid, stream);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace ccv
