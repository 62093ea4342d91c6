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
// seq_idx ids are shared by all channels of a time row, so the masks are
// wave-uniform.
#include "ccv_device.hpp"

namespace ccv {

template <class S, int K, bool SILU, bool SEQ, bool VEC>
__global__ void __launch_bounds__(256) cl_fwd_kernel(const ClArgs a) {
  constexpr int V = S::V;
  constexpr int U = kClUnroll;
  constexpr int H = K - 1;
  static_assert(U >= H, "a batch of rows must cover the history window");
  using raw = typename S::raw;
  const Common& m = a.m;

  const int lane = threadIdx.x & 63;
  const uint32_t g = xcd_order(blockIdx.x, m.xcd_q, m.xcd_r);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t item = (int64_t)g * kWavesPerGroup + wave;
  if (item >= m.nwork) return;                      // whole wave leaves together

  const int64_t tt = item % a.ntt;
  const int64_t rest = item / a.ntt;
  const int64_t cg = rest % a.ncg;
  const int64_t b = rest / a.ncg;
  const int64_t L = m.L;
  const int64_t c0 = cg * (64 * V) + lane * V;      // this lane's first channel
  const int nch = (int)(m.C - c0 < V ? (m.C - c0 > 0 ? m.C - c0 : 0) : V);
  const bool full = VEC && nch == V;
  // Every lane of the wave holds a whole aligned vector (same value for the wave).
  const bool wave_full = VEC && (cg + 1) * (64 * V) <= m.C;
  const int64_t t0 = tt * a.tile;
  const int64_t t1 = (t0 + a.tile < L) ? t0 + a.tile : L;

  const raw* __restrict__ xb = static_cast<const raw*>(m.x) + b * a.x_sb + c0;
  raw* __restrict__ ob = static_cast<raw*>(m.out) + b * a.o_sb + c0;
  const raw* __restrict__ ib = static_cast<const raw*>(m.init);
  const int32_t* __restrict__ sr = SEQ ? m.seq + b * L : nullptr;

  if (t0 < t1) {
    float w[V][K], beta[V];
    if (nch == V) {
      load_params<V * K>(m.w, m.w_dtype, c0 * K, &w[0][0]);
      if (m.bias) load_params<V>(m.bias, m.w_dtype, c0, beta);
      else
#pragma unroll
        for (int i = 0; i < V; ++i) beta[i] = 0.0f;
    } else {
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const bool in = i < nch;
#pragma unroll
        for (int k = 0; k < K; ++k) w[i][k] = in ? load_param(m.w, m.w_dtype, (c0 + i) * K + k) : 0.0f;
        beta[i] = (in && m.bias) ? load_param(m.bias, m.w_dtype, c0 + i) : 0.0f;
      }
    }

    // History rows X~[t0-H .. t0-1] for this lane's channels.
    float h[H][V];
#pragma unroll
    for (int j = 0; j < H; ++j) {
      const int64_t src = t0 - H + j;
      if (src >= 0) {
        if (full) {
          S::unpack(load16(xb + src * a.x_sl), h[j]);
        } else {
#pragma unroll
          for (int i = 0; i < V; ++i) h[j][i] = i < nch ? S::to_f(xb[src * a.x_sl + i]) : 0.0f;
        }
      } else {
#pragma unroll
        for (int i = 0; i < V; ++i)
          h[j][i] = (ib && i < nch) ? S::to_f(ib[b * m.is_b + (c0 + i) * m.is_c + (src + H) * m.is_i]) : 0.0f;
      }
    }
    // Sequence ids of the history rows (wave-uniform); rows left of t = 0 have none.
    int hid[H];
    bool hok[H];
#pragma unroll
    for (int j = 0; j < H; ++j) {
      const int64_t src = t0 - H + j;
      hok[j] = src >= 0;
      hid[j] = (SEQ && src >= 0) ? sr[src] : 0;
    }

    for (int64_t t = t0; t < t1; t += U) {
      float e[U][V];
      int id[U];
      // A batch of U rows inside the tile, across a wave of whole vectors, takes the
      // straight-line path: all U row loads are issued before any arithmetic.
      const bool fast = wave_full && t + U <= t1;
      if (fast) {
        u32x4 rv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) rv[u] = load16(xb + (t + u) * a.x_sl);
        if constexpr (SEQ) {
#pragma unroll
          for (int u = 0; u < U; ++u) id[u] = sr[t + u];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) S::unpack(rv[u], e[u]);
      } else {
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
            if constexpr (SEQ) id[u] = sr[tr];
          } else {
#pragma unroll
            for (int i = 0; i < V; ++i) e[u][i] = 0.0f;
            if constexpr (SEQ) id[u] = 0;
          }
        }
      }

#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t tr = t + u;
        float y[V];
#pragma unroll
        for (int i = 0; i < V; ++i) {
          float acc = beta[i];
#pragma unroll
          for (int k = 0; k < K; ++k) {
            const int r = u - H + k;                 // source row relative to this batch
            const float xv = r >= 0 ? e[r][i] : h[H + r][i];
            if constexpr (SEQ) {
              const bool ok = r >= 0 ? (id[r] == id[u]) : (hok[H + r] && hid[H + r] == id[u]);
              acc = ok ? __builtin_fmaf(w[i][k], xv, acc) : acc;
            } else {
              acc = __builtin_fmaf(w[i][k], xv, acc);
            }
          }
          y[i] = SILU ? silu(acc) : acc;
        }
        if (fast) {
          store16(ob + tr * a.o_sl, S::pack(y));
        } else if (tr < t1) {
          if (full) {
            store16(ob + tr * a.o_sl, S::pack(y));
          } else {
#pragma unroll
            for (int i = 0; i < V; ++i)
              if (i < nch) ob[tr * a.o_sl + i] = S::from_f(y[i]);
          }
        }
      }

      // Slide the history window: the last H rows of this batch become the history.
#pragma unroll
      for (int j = 0; j < H; ++j) {
#pragma unroll
        for (int i = 0; i < V; ++i) h[j][i] = e[U - H + j][i];
        if constexpr (SEQ) {
          hid[j] = id[U - H + j];
          hok[j] = true;
        }
      }
    }
  }

  // final_states: the tile holding t = L-1 (tile 0 when L == 0) copies the last
  // K-1 extended inputs of its channels bit for bit (Ch.5, section "Three kinds
  // of boundary handled separately").
  if (m.fin && tt == a.ntt - 1) {
    raw* __restrict__ fb = static_cast<raw*>(m.fin) + b * m.fs_b;
    for (int i = 0; i < nch; ++i) {
#pragma unroll
      for (int j = 0; j < H; ++j) {
        const int64_t src = L - H + j;
        raw v;
        if (src >= 0) v = xb[src * a.x_sl + i];
        else if (ib) v = ib[b * m.is_b + (c0 + i) * m.is_c + (src + H) * m.is_i];
        else v = 0;
        fb[(c0 + i) * m.fs_c + j * m.fs_i] = v;
      }
    }
  }
}

template <class S, int K, bool SILU, bool SEQ, bool VEC>
static int launch_one(const ClArgs& a, uint32_t grid, void* stream) {
  void* args[] = {const_cast<ClArgs*>(&a)};
  return (int)hipLaunchKernel(reinterpret_cast<const void*>(&cl_fwd_kernel<S, K, SILU, SEQ, VEC>),
                              dim3(grid), dim3(64 * kWavesPerGroup), args, 0,
                              static_cast<hipStream_t>(stream));
}

template <class S, int K>
static int launch_k(const ClArgs& a, bool silu, bool seq, bool vec, uint32_t grid, void* st) {
  if (silu) {
    if (seq) return vec ? launch_one<S, K, true, true, true>(a, grid, st) : launch_one<S, K, true, true, false>(a, grid, st);
    return vec ? launch_one<S, K, true, false, true>(a, grid, st) : launch_one<S, K, true, false, false>(a, grid, st);
  }
  if (seq) return vec ? launch_one<S, K, false, true, true>(a, grid, st) : launch_one<S, K, false, true, false>(a, grid, st);
  return vec ? launch_one<S, K, false, false, true>(a, grid, st) : launch_one<S, K, false, false, false>(a, grid, st);
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
