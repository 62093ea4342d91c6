// ccv_cf.hip -- channel-first forward (x and out have unit stride in time).
//
// Computes out[b,c,t] = act(bias[c] + sum_k keep * w[c,k] * X~[b,c,t-K+1+k]) (Ch.5
// "Dao forward CUDA implementation", section "How adjacent threads and chunks
// exchange history", stencil equation for z_i; fp32 accumulation, SiLU on the
// accumulator, one rounding at the store).
//
// Work split (rethought for wave64 rather than taken from the pages' 128-thread
// blocks): one wave owns one time segment of one (b, c) row.  Lane l of the wave
// holds 16-byte vectors number (l, l + 64, l + 128, ...) of the segment, so every
// load and store instruction of the wave covers 1 KB of consecutive addresses.
// Each output needs the K-1 inputs before its vector; they come from lane l-1 by
// a DPP wave shift, and lane 0 takes them from lane 63 of the previous vector
// (v_readlane), or, for the segment's first vector, from memory just left of the
// segment, initial_states, or zeros (Ch.5, section "Three kinds of boundary
// handled separately").  Segments are independent, so long rows with few
// channels still fill the GPU: the pages' design ties the block count to B*C
// (Ch.5, section "Task split of the time-contiguous path"), which collapses for
// long sequences with few channels.  There is no LDS and no barrier.
#include "ccv_device.hpp"

namespace ccv {

template <class S, int K, bool SILU, bool SEQ, bool VEC>
__global__ void __launch_bounds__(256) cf_fwd_kernel(const CfArgs a) {
  constexpr int V = S::V;
  constexpr int U = kCfUnroll;
  using raw = typename S::raw;
  const Common& m = a.m;

  const int lane = threadIdx.x & 63;
  const uint32_t g = xcd_order(blockIdx.x, m.xcd_q, m.xcd_r);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t item = (int64_t)g * kWavesPerGroup + wave;
  if (item >= m.nwork) return;                      // whole wave leaves together

  const int64_t row = item / a.nseg;
  const int64_t seg = item - row * a.nseg;
  const int64_t b = row / m.C;
  const int64_t c = row - b * m.C;
  const int64_t L = m.L;
  const int64_t t0 = seg * a.span;

  const raw* __restrict__ xr = static_cast<const raw*>(m.x) + b * a.x_sb + c * a.x_sc;
  raw* __restrict__ orow = static_cast<raw*>(m.out) + b * a.o_sb + c * a.o_sc;
  const int32_t* __restrict__ sr = SEQ ? m.seq + b * L : nullptr;

  if (t0 < L) {
    // Lane l's u-th vector starts at element t0 + (u*64 + l)*V.  A segment that lies
    // wholly inside the row takes the straight-line path (the condition is the same
    // for the whole wave): its U loads are issued first, before the parameter and
    // history loads, so they are in flight together.
    const bool fast = VEC && t0 + a.span <= L;
    const raw* __restrict__ xl = xr + t0 + lane * V;
    const int32_t* __restrict__ sl = SEQ ? sr + t0 + lane * V : nullptr;
    u32x4 rv[U];
    u32x4 sv[U][V / 4];
    if (fast) {
#pragma unroll
      for (int u = 0; u < U; ++u) rv[u] = load16(xl + u * 64 * V);
      if constexpr (SEQ) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int q = 0; q < V / 4; ++q) sv[u][q] = load16(sl + u * 64 * V + 4 * q);
      }
    }

    float w[K];
    load_params<K>(m.w, m.w_dtype, c * K, w);
    const float beta = m.bias ? load_param(m.bias, m.w_dtype, c) : 0.0f;

    // History for lane 0 of the segment's first vector: X~[t0-K+1 .. t0-1].
    float carry[K - 1];
    int carry_id[K - 1];
    if (t0 >= K - 1) {                               // inside the row: K-1 plain loads
#pragma unroll
      for (int j = 0; j < K - 1; ++j) {
        carry[j] = S::to_f(xr[t0 - (K - 1) + j]);
        carry_id[j] = SEQ ? sr[t0 - (K - 1) + j] : 0;
      }
    } else {
#pragma unroll
      for (int j = 0; j < K - 1; ++j) {
        const int64_t src = t0 - (K - 1) + j;
        if (src >= 0) {
          carry[j] = S::to_f(xr[src]);
        } else if (m.init) {
          carry[j] = S::to_f(static_cast<const raw*>(m.init)[b * m.is_b + c * m.is_c + (src + K - 1) * m.is_i]);
        } else {
          carry[j] = 0.0f;
        }
        carry_id[j] = (SEQ && src >= 0) ? sr[src] : 0;
      }
    }
    // With seq_idx a source left of t = 0 has no id and never counts.
    bool first_ok[K - 1];
#pragma unroll
    for (int j = 0; j < K - 1; ++j) first_ok[j] = !(SEQ && lane == 0 && t0 - (K - 1) + j < 0);

    float e[U][V];
    int id[U][V];
    if (fast) {
#pragma unroll
      for (int u = 0; u < U; ++u) S::unpack(rv[u], e[u]);
      if constexpr (SEQ) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int q = 0; q < V / 4; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i) id[u][4 * q + i] = (int)dword(sv[u][q], i);
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t te = t0 + (int64_t)(u * 64 + lane) * V;
        if (VEC && te + V <= L) {
          S::unpack(load16(xr + te), e[u]);
        } else {
#pragma unroll
          for (int i = 0; i < V; ++i) e[u][i] = te + i < L ? S::to_f(xr[te + i]) : 0.0f;
        }
        if constexpr (SEQ) {
#pragma unroll
          for (int i = 0; i < V; ++i) id[u][i] = te + i < L ? sr[te + i] : 0;
        }
      }
    }

#pragma unroll
    for (int u = 0; u < U; ++u) {
      // Halo of this lane's vector: the last K-1 inputs of the previous vector.
      float h[K - 1];
      int hid[K - 1];
#pragma unroll
      for (int j = 0; j < K - 1; ++j) {
        h[j] = shift_in(carry[j], e[u][V - (K - 1) + j]);
        if constexpr (SEQ) hid[j] = shift_in(carry_id[j], id[u][V - (K - 1) + j]);
      }
#pragma unroll
      for (int j = 0; j < K - 1; ++j) {
        carry[j] = lane63(e[u][V - (K - 1) + j]);
        if constexpr (SEQ) carry_id[j] = lane63(id[u][V - (K - 1) + j]);
      }

      float y[V];
#pragma unroll
      for (int i = 0; i < V; ++i) {
        float acc = beta;
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const int j = i - (K - 1) + k;            // source offset inside the vector
          const float xv = j >= 0 ? e[u][j] : h[K - 1 + j];
          if constexpr (SEQ) {
            const int sid = j >= 0 ? id[u][j] : hid[K - 1 + j];
            const bool ok = (j >= 0 || u > 0 || first_ok[K - 1 + j]) && sid == id[u][i];
            acc = ok ? __builtin_fmaf(w[k], xv, acc) : acc;
          } else {
            acc = __builtin_fmaf(w[k], xv, acc);
          }
        }
        y[i] = SILU ? silu(acc) : acc;
      }

      if (fast) {
        store16(orow + t0 + (int64_t)(u * 64 + lane) * V, S::pack(y));
      } else {
        const int64_t te = t0 + (int64_t)(u * 64 + lane) * V;
        if (VEC && te + V <= L) {
          store16(orow + te, S::pack(y));
        } else {
#pragma unroll
          for (int i = 0; i < V; ++i)
            if (te + i < L) orow[te + i] = S::from_f(y[i]);
        }
      }
    }
  }

  // final_states: the segment holding t = L-1 (segment 0 when L == 0) copies the
  // last K-1 extended inputs bit for bit (Ch.5, section "Three kinds of boundary
  // handled separately").
  if (m.fin && (L == 0 ? seg == 0 : (t0 <= L - 1 && L - 1 < t0 + a.span)) && lane < K - 1) {
    const int64_t j = L - (K - 1) + lane;
    raw v;
    if (j >= 0) v = xr[j];
    else if (m.init) v = static_cast<const raw*>(m.init)[b * m.is_b + c * m.is_c + (j + K - 1) * m.is_i];
    else v = 0;
    static_cast<raw*>(m.fin)[b * m.fs_b + c * m.fs_c + lane * m.fs_i] = v;
  }
}

template <class S, int K, bool SILU, bool SEQ, bool VEC>
static int launch_one(const CfArgs& a, uint32_t grid, void* stream) {
  void* args[] = {const_cast<CfArgs*>(&a)};
  return (int)hipLaunchKernel(reinterpret_cast<const void*>(&cf_fwd_kernel<S, K, SILU, SEQ, VEC>),
                              dim3(grid), dim3(64 * kWavesPerGroup), args, 0,
                              static_cast<hipStream_t>(stream));
}

template <class S, int K>
static int launch_k(const CfArgs& a, bool silu, bool seq, bool vec, uint32_t grid, void* st) {
  if (silu) {
    if (seq) return vec ? launch_one<S, K, true, true, true>(a, grid, st) : launch_one<S, K, true, true, false>(a, grid, st);
    return vec ? launch_one<S, K, true, false, true>(a, grid, st) : launch_one<S, K, true, false, false>(a, grid, st);
  }
  if (seq) return vec ? launch_one<S, K, false, true, true>(a, grid, st) : launch_one<S, K, false, true, false>(a, grid, st);
  return vec ? launch_one<S, K, false, false, true>(a, grid, st) : launch_one<S, K, false, false, false>(a, grid, st);
}

template <class S>
static int launch_s(const CfArgs& a, int K, bool silu, bool seq, bool vec, uint32_t grid, void* st) {
  switch (K) {
    case 2: return launch_k<S, 2>(a, silu, seq, vec, grid, st);
    case 3: return launch_k<S, 3>(a, silu, seq, vec, grid, st);
    case 4: return launch_k<S, 4>(a, silu, seq, vec, grid, st);
  }
  return (int)hipErrorInvalidValue;
}

int launch_cf(const CfArgs& a, int dtype, int K, bool silu, bool seq, bool vec, uint32_t grid,
              void* stream) {
  switch (dtype) {
    case CCV_DT_F32: return launch_s<F32>(a, K, silu, seq, vec, grid, stream);
    case CCV_DT_F16: return launch_s<F16>(a, K, silu, seq, vec, grid, stream);
    case CCV_DT_BF16: return launch_s<BF16>(a, K, silu, seq, vec, grid, stream);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace ccv
