// ccv_cf.hip -- channel-first forward (x and out have unit stride in time).
//
// Computes out[b,c,t] = act(bias[c] + sum_k keep * w[c,k] * X~[b,c,t-K+1+k]) (Ch.5
// "Dao forward CUDA implementation", section "How adjacent threads and chunks
// exchange history", stencil equation for z_i; fp32 accumulation, SiLU on the
// accumulator, one rounding at the store).
//
// Work split (rethought for wave64 rather than taken from the pages' 128-thread
// blocks): a segment is 64 * V * U consecutive steps of one (b, c) row.  Lane l
// holds 16-byte vectors number (l, l + 64, l + 128, ...) of the segment, so every
// load and store instruction of the wave covers 1 KB of consecutive addresses.
// Each output needs the K-1 inputs before its vector; they come from lane l-1 by
// a DPP wave shift, and lane 0 takes them from lane 63 of the previous vector
// (v_readlane), or, for the segment's first vector, from memory just left of the
// segment, initial_states, or zeros (Ch.5, section "Three kinds of boundary
// handled separately").  Segments are independent, so long rows with few
// channels still fill the GPU, where the pages' design ties the block count to
// B*C (Ch.5, section "Task split of the time-contiguous path").
//
// Wave w of the grid takes segments w, w + W, w + 2W, ... (W = waves launched):
// at any moment the waves work on one compact window of the tensors, and each
// wave issues all loads of its next segment (data, weights, bias, halo) before
// the arithmetic of the current one.  x and out are streamed with non-temporal
// loads and stores.  There is no LDS and no barrier.
#include "ccv_device.hpp"

namespace ccv {

// Everything one whole segment needs, loaded ahead of its arithmetic: the lane's
// U data vectors (and sequence ids), the channel's raw weights and bias, and the
// raw history just left of the segment.  The loads are unconditional and go
// straight into their registers; nothing is converted until the arithmetic, so
// the compiler knows exactly how many memory operations are in flight and waits
// only for the ones it needs.
template <class S, int K, bool SEQ, int WB>
struct SegLoads {
  u32x4 d[kCfUnroll];
  u32x4 sid[SEQ ? kCfUnroll : 1][S::V / 4];
  uint32_t w[K];
  uint32_t bias;
  typename S::raw hist[K - 1];
  int hist_id[K - 1];
};

struct SegPos {
  int64_t b, c, t0;
};

__device__ inline SegPos row_pos(const Common& m, int64_t row, int64_t t0) {
  const int64_t b = row / m.C;
  return SegPos{b, row - b * m.C, t0};
}

// Issue the loads of whole segment p (when `valid`; otherwise harmless loads of
// zeros, so the instruction stream is the same either way).
template <class S, int K, bool SEQ, int WB, bool TAIL>
__device__ inline void issue_segment(const CfArgs& a, const SegPos& p, bool valid, int lane,
                                     SegLoads<S, K, SEQ, WB>& q) {
  constexpr int V = S::V;
  constexpr int H = K - 1;
  constexpr int ES = sizeof(typename S::raw);
  using raw = typename S::raw;
  const Common& m = a.m;
  const uintptr_t zero = reinterpret_cast<uintptr_t>(kZeroSrc);
  const uintptr_t xrow = reinterpret_cast<uintptr_t>(m.x) + (p.b * a.x_sb + p.c * a.x_sc) * ES;
  const uintptr_t srow = reinterpret_cast<uintptr_t>(m.seq) + p.b * m.L * 4;

  if constexpr (!TAIL) {
    const uintptr_t dbase = pick(valid, xrow + (p.t0 + lane * V) * ES, zero);
    const uintptr_t dstep = valid ? 64 * V * ES : 0;
#pragma unroll
    for (int u = 0; u < kCfUnroll; ++u) q.d[u] = gload16_stream(dbase + u * dstep);
    if constexpr (SEQ) {
      const uintptr_t sbase = pick(valid, srow + (p.t0 + lane * V) * 4, zero);
      const uintptr_t sstep = valid ? 64 * V * 4 : 0;
      const uintptr_t squad = valid ? 16 : 0;
#pragma unroll
      for (int u = 0; u < kCfUnroll; ++u)
#pragma unroll
        for (int r = 0; r < V / 4; ++r) q.sid[u][r] = gload<u32x4>(sbase + u * sstep + r * squad);
    }
  } else {
    // A row's last segment, shorter than the span.  Vectors that end at or before L
    // load as 16 bytes; a vector at or past L loads the segment's first vector
    // instead (in bounds; its outputs are not stored, and no halo flows from it
    // into a vector before L).  When L is not a multiple of V, the one vector that
    // straddles L is read element by element, zeros past L, so no access leaves
    // the row.  Wave-wide vector groups that start at or past L load nothing (the
    // arithmetic skips them too).
    const int64_t vrem = m.L - p.t0;               // steps of the row from t0 on
    const uintptr_t dbase = pick(valid, xrow + p.t0 * ES, zero);
    const uintptr_t sbase = pick(valid, srow + p.t0 * 4, zero);
#pragma unroll
    for (int u = 0; u < kCfUnroll; ++u) {
      if ((int64_t)u * 64 * V >= vrem) break;
      const int64_t e = (int64_t)(u * 64 + lane) * V;
      const bool whole = valid && e + V <= vrem;
      q.d[u] = gload16_stream(dbase + (whole ? (uint32_t)e * ES : 0u));
      if constexpr (SEQ) {
#pragma unroll
        for (int r = 0; r < V / 4; ++r)
          q.sid[u][r] = gload<u32x4>(sbase + (whole ? (uint32_t)e * 4 + r * 16 : 0u));
      }
      if (valid && e < vrem && e + V > vrem) {
        raw part[V];
        int32_t part_id[V];
#pragma unroll
        for (int i = 0; i < V; ++i) {
          const bool in = e + i < vrem;
          part[i] = in ? gload<raw>(dbase + (uint32_t)(e + i) * ES) : raw(0);
          part_id[i] = (SEQ && in) ? gload<int32_t>(sbase + (uint32_t)(e + i) * 4) : 0;
        }
        __builtin_memcpy(&q.d[u], part, 16);
        if constexpr (SEQ) __builtin_memcpy(&q.sid[u][0], part_id, V * 4);
      }
    }
  }
  const uintptr_t wbase = pick(valid, reinterpret_cast<uintptr_t>(m.w) + p.c * K * WB, zero);
  const uintptr_t wstep = valid ? WB : 0;
#pragma unroll
  for (int k = 0; k < K; ++k) q.w[k] = load_param_raw<WB>(wbase + k * wstep);
  q.bias = load_param_raw<WB>(pick(valid && m.bias, reinterpret_cast<uintptr_t>(m.bias) + p.c * WB, zero));
  const uintptr_t irow = reinterpret_cast<uintptr_t>(m.init) + (p.b * m.is_b + p.c * m.is_c) * ES;
#pragma unroll
  for (int j = 0; j < H; ++j) {
    const int64_t src = p.t0 - H + j;
    const uintptr_t from_init = pick(m.init != nullptr, irow + (src + H) * m.is_i * ES, zero);
    const uintptr_t from_x = xrow + src * ES;
    q.hist[j] = gload<raw>(pick(valid, pick(src >= 0, from_x, from_init), zero));
    if constexpr (SEQ)                             // the history carries seq_idx[b, 0]
      q.hist_id[j] = gload<int32_t>(pick(valid && src >= 0, srow + src * 4,
                                         pick(valid && m.init != nullptr, srow, zero)));
    else
      q.hist_id[j] = 0;
  }
}

// One output vector per lane: the K-tap stencil on fp32 values (Ch.5, stencil
// equation for z_i), SiLU, and the lane's halo carried in from lane-1 / `carry`.
template <class S, int K, bool SILU, bool SEQ>
__device__ inline void stencil_vector(const float (&e)[S::V], const int (&id)[S::V], float (&carry)[K - 1],
                                      int (&carry_id)[K - 1], bool first_vec, const bool (&first_ok)[K - 1],
                                      const float (&w)[K], float beta, float (&y)[S::V]) {
  constexpr int V = S::V;
  constexpr int H = K - 1;
  float h[H];
  int hid[H];
#pragma unroll
  for (int j = 0; j < H; ++j) {
    h[j] = shift_in(carry[j], e[V - H + j]);
    if constexpr (SEQ) hid[j] = shift_in(carry_id[j], id[V - H + j]);
  }
#pragma unroll
  for (int j = 0; j < H; ++j) {
    carry[j] = lane63(e[V - H + j]);
    if constexpr (SEQ) carry_id[j] = lane63(id[V - H + j]);
  }
#pragma unroll
  for (int i = 0; i < V; ++i) {
    float acc = beta;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int j = i - H + k;                       // source offset inside the vector
      const float xv = j >= 0 ? e[j] : h[H + j];
      if constexpr (SEQ) {
        const int sid = j >= 0 ? id[j] : hid[H + j];
        const bool ok = (j >= 0 || !first_vec || first_ok[H + j]) && sid == id[i];
        acc = ok ? __builtin_fmaf(w[k], xv, acc) : acc;
      } else {
        acc = __builtin_fmaf(w[k], xv, acc);
      }
    }
    y[i] = SILU ? silu(acc) : acc;
  }
}

template <int K, bool SEQ>
__device__ inline void first_flags(int64_t t0, int lane, bool has_init, bool (&first_ok)[K - 1]) {
  // With seq_idx, a source left of t = 0 is the history of the row's first
  // sequence (its id is seq_idx[b, 0]); without a history it never counts.
#pragma unroll
  for (int j = 0; j < K - 1; ++j) first_ok[j] = !(SEQ && !has_init && lane == 0 && t0 - (K - 1) + j < 0);
}

// Arithmetic and stores of a whole segment from its prefetched loads.
template <class S, int K, bool SILU, bool SEQ, int WB, bool TAIL>
__device__ inline void compute_whole(const CfArgs& a, const SegPos& p, int lane,
                                     const SegLoads<S, K, SEQ, WB>& q) {
  constexpr int V = S::V;
  constexpr int H = K - 1;
  using raw = typename S::raw;
  const Common& m = a.m;
  float w[K];
#pragma unroll
  for (int k = 0; k < K; ++k) w[k] = param_f32<WB>(q.w[k], m.w_dtype);
  const float beta = param_f32<WB>(q.bias, m.w_dtype);
  float carry[H];
  int carry_id[H];
#pragma unroll
  for (int j = 0; j < H; ++j) {
    carry[j] = S::to_f(q.hist[j]);
    carry_id[j] = q.hist_id[j];
  }
  bool first_ok[H];
  first_flags<K, SEQ>(p.t0, lane, m.init != nullptr, first_ok);
  raw* __restrict__ ol = static_cast<raw*>(m.out) + p.b * a.o_sb + p.c * a.o_sc + p.t0 + lane * V;
#pragma unroll
  for (int u = 0; u < kCfUnroll; ++u) {
    if (TAIL && p.t0 + (int64_t)u * 64 * V >= m.L) break;   // the wave's vectors are all past L
    float e[V], y[V];
    int id[V];
    S::unpack(q.d[u], e);
    if constexpr (SEQ) {
#pragma unroll
      for (int r = 0; r < V / 4; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) id[4 * r + i] = (int)dword(q.sid[u][r], i);
    }
    stencil_vector<S, K, SILU, SEQ>(e, id, carry, carry_id, u == 0, first_ok, w, beta, y);
    if constexpr (!TAIL) {
      store16_stream(ol + u * 64 * V, S::pack(y));
    } else {
      const int64_t left = m.L - (p.t0 + (int64_t)(u * 64 + lane) * V);
      if (left >= V) {
        store16_stream(ol + u * 64 * V, S::pack(y));
      } else if (left > 0) {                       // the vector that straddles L
#pragma unroll
        for (int i = 0; i < V; ++i)
          if (i < left) ol[u * 64 * V + i] = S::from_f(y[i]);
      }
    }
  }
}

// A segment on the element path (CCV_FORCE_SCALAR): element loads and stores,
// bounds-checked against L.
template <class S, int K, bool SILU, bool SEQ>
__device__ inline void compute_partial(const CfArgs& a, const SegPos& p, int lane) {
  constexpr int V = S::V;
  constexpr int H = K - 1;
  using raw = typename S::raw;
  const Common& m = a.m;
  const int64_t L = m.L;
  const raw* __restrict__ xr = static_cast<const raw*>(m.x) + p.b * a.x_sb + p.c * a.x_sc;
  raw* __restrict__ orow = static_cast<raw*>(m.out) + p.b * a.o_sb + p.c * a.o_sc;
  const int32_t* __restrict__ sr = SEQ ? m.seq + p.b * L : nullptr;
  float w[K];
  load_params<K>(m.w, m.w_dtype, p.c * K, w);
  const float beta = m.bias ? load_param(m.bias, m.w_dtype, p.c) : 0.0f;
  float carry[H];
  int carry_id[H];
#pragma unroll
  for (int j = 0; j < H; ++j) {
    const int64_t src = p.t0 - H + j;
    if (src >= 0) carry[j] = S::to_f(xr[src]);
    else if (m.init)
      carry[j] = S::to_f(static_cast<const raw*>(m.init)[p.b * m.is_b + p.c * m.is_c + (src + H) * m.is_i]);
    else carry[j] = 0.0f;
    carry_id[j] = SEQ ? (src >= 0 ? sr[src] : (m.init ? sr[0] : 0)) : 0;
  }
  bool first_ok[H];
  first_flags<K, SEQ>(p.t0, lane, m.init != nullptr, first_ok);
#pragma unroll
  for (int u = 0; u < kCfUnroll; ++u) {
    const int64_t te = p.t0 + (int64_t)(u * 64 + lane) * V;
    float e[V], y[V];
    int id[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const bool in = te + i < L;
      e[i] = in ? S::to_f(xr[te + i]) : 0.0f;
      id[i] = (SEQ && in) ? sr[te + i] : 0;
    }
    stencil_vector<S, K, SILU, SEQ>(e, id, carry, carry_id, u == 0, first_ok, w, beta, y);
#pragma unroll
    for (int i = 0; i < V; ++i)
      if (te + i < L) orow[te + i] = S::from_f(y[i]);
  }
}

// final_states of one row: the last K-1 extended inputs, bit for bit (Ch.5,
// section "Three kinds of boundary handled separately"); with seq_idx, those of
// the row's last sequence only (others are zero).
template <class S, int K>
__device__ inline void final_states_row(const CfArgs& a, const SegPos& p, int lane) {
  constexpr int H = K - 1;
  using raw = typename S::raw;
  const Common& m = a.m;
  if (lane >= H) return;
  const int64_t j = m.L - H + lane;
  raw v;
  if (j >= 0) v = static_cast<const raw*>(m.x)[p.b * a.x_sb + p.c * a.x_sc + j];
  else if (m.init) v = static_cast<const raw*>(m.init)[p.b * m.is_b + p.c * m.is_c + (j + H) * m.is_i];
  else v = 0;
  if (!final_kept(m.seq ? m.seq + p.b * m.L : nullptr, m.L, j, m.init != nullptr)) v = 0;
  static_cast<raw*>(m.fin)[p.b * m.fs_b + p.c * m.fs_c + lane * m.fs_i] = v;
}

template <class S, int K, bool SILU, bool SEQ, bool VEC, int WB>
__global__ void __launch_bounds__(256) cf_fwd_kernel(const CfArgs a) {
  const Common& m = a.m;
  const int lane = threadIdx.x & 63;
  // Workgroups keep the hardware's numbering: rows share only a K-1 step halo
  // between segments, and dealing consecutive segments to all 8 XCDs at once
  // spreads the concurrent streams over more memory channels than giving each
  // XCD one contiguous range does.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t w0 = (int64_t)blockIdx.x * kWavesPerGroup + wave;
  const int64_t rows = m.B * m.C;
  // With 16-byte rows whose length is not a multiple of the span, workgroups
  // appended after those of the whole segments give each row's last, shorter
  // segment a wave of its own (lanes past L store nothing, the vector that
  // straddles L moves element by element); that wave also writes the row's final
  // states.  They share the launch, so they run beside the whole segments instead
  // of after them.
  const bool tails = VEC && m.L > 0 && a.nseg > a.nfull;
  if constexpr (VEC) {
    const int64_t wmain = (a.nwaves + kWavesPerGroup - 1) / kWavesPerGroup * kWavesPerGroup;
    if (w0 >= wmain) {
      const int64_t r = w0 - wmain;
      if (!tails || r >= rows) return;              // whole wave leaves together
      const SegPos p = row_pos(m, r, a.nfull * a.span);
      SegLoads<S, K, SEQ, WB> q;
      issue_segment<S, K, SEQ, WB, true>(a, p, true, lane, q);
      compute_whole<S, K, SILU, SEQ, WB, true>(a, p, lane, q);
      if (m.fin) final_states_row<S, K>(a, p, lane);
      return;
    }
  }
  if (w0 >= a.nwaves) return;                       // whole wave leaves together
  const int64_t W = a.nwaves;

  // Phase 1: whole segments, two sets of loads in flight.  The next segment's
  // loads are issued before the current segment's arithmetic; the body is
  // written twice so the sets swap roles without register copies.  Segment i is
  // (row i / nfull, segment i % nfull), and row r is (b, c) = (r / C, r % C); the
  // cursor steps by W segments with additions only, the quotients of W taken once.
  const int64_t nfull = VEC ? a.nfull : 0;
  const int64_t n1 = rows * nfull;
  if constexpr (VEC) if (w0 < n1) {
    const int64_t drow = W / nfull, dseg = W - drow * nfull;
    const int64_t db = drow / m.C, dc = drow - db * m.C;
    const int64_t row0 = w0 / nfull;
    int64_t seg = w0 - row0 * nfull, b = row0 / m.C, c = row0 - b * m.C;
    auto advance = [&]() {
      seg += dseg;
      const int64_t carry = seg >= nfull ? 1 : 0;
      seg -= carry * nfull;
      c += dc + carry;                              // < 2C: at most one wrap
      b += db;
      if (c >= m.C) {
        c -= m.C;
        ++b;
      }
    };
    SegLoads<S, K, SEQ, WB> qa, qb;
    int64_t i = w0;
    SegPos pa{b, c, seg * a.span}, pb;
    issue_segment<S, K, SEQ, WB, false>(a, pa, true, lane, qa);
    while (true) {
      const int64_t i1 = i + W;
      if (i1 >= n1) {                               // last segment of this wave
        compute_whole<S, K, SILU, SEQ, WB, false>(a, pa, lane, qa);
        break;
      }
      advance();
      pb = SegPos{b, c, seg * a.span};
      issue_segment<S, K, SEQ, WB, false>(a, pb, true, lane, qb);
      compute_whole<S, K, SILU, SEQ, WB, false>(a, pa, lane, qa);
      const int64_t i2 = i1 + W;
      if (i2 >= n1) {
        compute_whole<S, K, SILU, SEQ, WB, false>(a, pb, lane, qb);
        break;
      }
      advance();
      pa = SegPos{b, c, seg * a.span};
      issue_segment<S, K, SEQ, WB, false>(a, pa, true, lane, qa);
      compute_whole<S, K, SILU, SEQ, WB, false>(a, pb, lane, qb);
      i = i2;
    }
  }

  // Phase 2 (element path only): every segment, element by element.
  if constexpr (!VEC) {
    const int64_t n2 = m.L > 0 ? rows * a.nseg : 0;
    for (int64_t j = w0; j < n2; j += W) {
      const int64_t row = j / a.nseg;
      compute_partial<S, K, SILU, SEQ>(a, row_pos(m, row, (j % a.nseg) * a.span), lane);
    }
  }

  // Phase 3: final states (the appended waves write them when there are tails).
  if (m.fin && !tails)
    for (int64_t r = w0; r < rows; r += W) final_states_row<S, K>(a, row_pos(m, r, 0), lane);
}

template <class S, int K, bool SILU, bool SEQ, bool VEC, int WB>
static int launch_one(const CfArgs& a, uint32_t grid, void* stream) {
  void* args[] = {const_cast<CfArgs*>(&a)};
  return (int)hipLaunchKernel(reinterpret_cast<const void*>(&cf_fwd_kernel<S, K, SILU, SEQ, VEC, WB>),
                              dim3(grid), dim3(64 * kWavesPerGroup), args, 0,
                              static_cast<hipStream_t>(stream));
}

template <class S, int K, bool SILU, bool SEQ, bool VEC>
static int launch_w(const CfArgs& a, uint32_t grid, void* st) {
  return a.m.w_dtype == CCV_DT_F32 ? launch_one<S, K, SILU, SEQ, VEC, 4>(a, grid, st)
                                   : launch_one<S, K, SILU, SEQ, VEC, 2>(a, grid, st);
}

template <class S, int K>
static int launch_k(const CfArgs& a, bool silu, bool seq, bool vec, uint32_t grid, void* st) {
  if (silu) {
    if (seq) return vec ? launch_w<S, K, true, true, true>(a, grid, st) : launch_w<S, K, true, true, false>(a, grid, st);
    return vec ? launch_w<S, K, true, false, true>(a, grid, st) : launch_w<S, K, true, false, false>(a, grid, st);
  }
  if (seq) return vec ? launch_w<S, K, false, true, true>(a, grid, st) : launch_w<S, K, false, true, false>(a, grid, st);
  return vec ? launch_w<S, K, false, false, true>(a, grid, st) : launch_w<S, K, false, false, false>(a, grid, st);
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
