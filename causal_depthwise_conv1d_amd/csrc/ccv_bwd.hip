// ccv_bwd.hip -- the backward of the causal depthwise conv1d: dx, dinitial_states,
// dweight and dbias from dout and dfinal_states (Ch.4 "Dao interface and source
// map", section "How autograd links forward and backward"; the formulas are
// stated in ccv.h beside ccv_bwd).
//
// Gradient kernel.  One lane owns one (b, c) row and a group of tpi consecutive
// tiles of T time steps.  For each tile [t0, t_end) it walks
// u = t0 .. t_end + K - 2 once, with three register windows over the
// positions u-K+1 .. u: the extended input X~, the sequence ids, and dz.  At
// each u < L it recomputes the pre-activation z[u] exactly as the forward does
// (bias first, k ascending, fused multiply-adds) and forms dz[u] = dout[u] *
// act'(z[u]); for u inside the tile it adds the tap products dz[u] * X~[u-K+1+k]
// to its fp32 partial dweight and dbias.  Position j = u-K+1 then has every dz it
// reads (dz[j .. j+K-1]), so dX~[j] is finished and stored: to dx when j lies in
// the tile, to dinitial_states when j < 0 in the row's first tile.  Recomputing
// z over the K-1 steps past the tile is the halo; nothing from the forward is
// stored.  The lane's partial sums over its group go to the workspace as one
// row.  In the element kernel lanes take consecutive channels and read global
// memory directly; in the LDS kernels a wave stages each tile of 64 channels in
// LDS with 16-byte loads first (see bwd_lds_kernel).  For channel-first data
// without seq_idx a third kernel keeps everything in registers: 64-lane segments
// of one row with the halos passed between lanes (see bwd_cf_reg_kernel).
//
// Reduction kernel.  The partials of all (b, tile group) are summed per (tap or bias,
// channel) by a tree of fixed shape: each level adds groups of kBwdFanIn
// consecutive rows in order, one lane per group and column, until one row is
// left, which is rounded once to the weight dtype (the fp32-accumulate-then-
// convert of the section cited above).  The shape depends only on the problem,
// so dweight and dbias repeat bit for bit; a level reads coalesced rows.
#include "ccv_bwd_launch.hpp"
#include "ccv_device.hpp"

namespace ccv {
namespace {

// d silu(z) / dz = s (1 + z (1 - s)) with s = sigmoid(z), on the hardware exp2 and
// rcp as the forward's SiLU; z (1 - s) = z - z s and s + s t are each one fused
// multiply-add.
__device__ inline float silu_slope(float z) {
  const float s = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.44269504088896341f));
  const float t = __builtin_fmaf(-z, s, z);
  return __builtin_fmaf(s, t, s);
}

// The walk of one lane over one tile (see the header comment), shared by both
// kernels so that they compute the same bits.  `src` gives X~ at positions
// >= t0 - K + 1 (history included), dout at positions >= t0, the sequence id at
// positions in [0, L) from t0 - K + 1 to t0 + T + K - 2 (and at 0 when t0 = 0),
// and takes dx.
// FULL (a tile of TT steps with t0 + TT + K - 1 <= L, not writing
// d(initial_states)) fixes the trip count and every condition at compile time,
// so the walk unrolls completely; the arithmetic is the same.
template <class S, int K, bool SILU, bool SEQ, bool FULL, int TT, class Src>
__device__ inline void walk_tile(const BwdArgs& a, int64_t b, int64_t c, int64_t t0, Src& src,
                                 const float (&w)[K], float beta, float (&pw)[K], float& pb) {
  using raw = typename S::raw;
  constexpr int H = K - 1;
  const int64_t L = a.L;
  const int64_t t_end = FULL ? t0 + TT : (t0 + a.T < L ? t0 + a.T : L);
  const bool has_init = a.init != nullptr;       // with seq_idx: the history is the first sequence's
  const int hist_id = (SEQ && has_init && L > 0 && t0 < H) ? src.id(0) : 0;   // read left of t = 0 only

  // Slots 0 .. H-1 hold positions u-H .. u-1 before step u; slot H takes u.
  float xw[K], dzw[K];
  int idw[K];
#pragma unroll
  for (int i = 0; i < H; ++i) {
    const int64_t j = t0 - H + i;
    xw[i] = src.x(j);
    idw[i] = SEQ ? (j >= 0 ? src.id(j) : hist_id) : 0;
    dzw[i] = 0.0f;                                 // dz left of the tile is never read
  }
  const int64_t n_steps = FULL ? TT + H : t_end + H - t0;
  constexpr int kUnroll = FULL ? TT + H : 1;
#pragma unroll kUnroll
  for (int64_t i = 0; i < n_steps; ++i) {
    const int64_t u = t0 + i;
    float xu = 0.0f, dzu = 0.0f;
    int idu = 0;
    if (FULL || u < L) {
      xu = src.x(u);
      if constexpr (SEQ) idu = src.id(u);
      bool keep[H];
      float z = beta;
#pragma unroll
      for (int k = 0; k < H; ++k) {
        keep[k] = !SEQ || ((u - H + k >= 0 || has_init) && idw[k] == idu);
        if (keep[k]) z = __builtin_fmaf(w[k], xw[k], z);
      }
      z = __builtin_fmaf(w[H], xu, z);
      const float go = src.g(u);
      dzu = SILU ? go * silu_slope(z) : go;
      if (FULL ? i < TT : u < t_end) {
#pragma unroll
        for (int k = 0; k < H; ++k)
          if (keep[k]) pw[k] = __builtin_fmaf(dzu, xw[k], pw[k]);
        pw[H] = __builtin_fmaf(dzu, xu, pw[H]);
        pb += dzu;
      }
    }
    xw[H] = xu;
    dzw[H] = dzu;
    idw[H] = idu;

    // dX~ at j = u - H reads dz[j .. u] = slots 0 .. H.
    const int64_t j = u - H;
    const bool to_dx = FULL ? i >= H : j >= t0;
    const bool to_init = !FULL && j < 0 && a.dinit != nullptr;
    if (to_dx || to_init) {
      float acc = 0.0f;
#pragma unroll
      for (int k = 0; k < K; ++k) {                // output t = j + H - k uses tap k on X~[j]
        const int64_t t = j + H - k;
        const bool keep = (FULL || (t >= 0 && t < L)) && (!SEQ || idw[0] == idw[H - k]);
        if (keep) acc = __builtin_fmaf(w[k], dzw[H - k], acc);
      }
      if (!FULL && a.dfs && j >= L - H && (!SEQ || L == 0 || idw[0] == src.id(L - 1)))
        acc += S::to_f(static_cast<const raw*>(a.dfs)[b * a.fs_b + c * a.fs_c + (j - (L - H)) * a.fs_i]);
      if (FULL || j >= 0)                          // a whole tile never reaches left of t = 0
        src.put_dx(j, acc);
      else
        static_cast<raw*>(a.dinit)[b * a.di_b + c * a.di_c + (j + H) * a.di_i] = S::from_f(acc);
    }
#pragma unroll
    for (int i = 0; i < H; ++i) {
      xw[i] = xw[i + 1];
      dzw[i] = dzw[i + 1];
      idw[i] = idw[i + 1];
    }
  }

}

// The lane's partial row: parameter gradients summed over its group of tiles.
template <int K>
__device__ inline void store_partials(const BwdArgs& a, int64_t b, int64_t g, int64_t c, const float (&pw)[K],
                                      float pb) {
  float* part = a.part + ((b * a.ngr + g) * (K + 1)) * a.C + c;
#pragma unroll
  for (int k = 0; k < K; ++k) part[k * a.C] = pw[k];
  part[K * a.C] = pb;
}

// Element path: strided global loads and stores (any layout).
template <class S, int K>
struct GlobalSrc {
  using raw = typename S::raw;
  const raw* xr;
  const raw* gr;
  raw* dxr;
  const raw* init;          // the row's initial_states, or nullptr
  const int32_t* sr;        // the row of seq_idx, or nullptr
  int64_t x_sl, d_sl, g_sl, is_i;
  __device__ float x(int64_t p) const {
    if (p >= 0) return S::to_f(xr[p * x_sl]);
    return init ? S::to_f(init[(p + K - 1) * is_i]) : 0.0f;
  }
  __device__ float g(int64_t p) const { return S::to_f(gr[p * d_sl]); }
  __device__ void put_dx(int64_t j, float v) const { dxr[j * g_sl] = S::from_f(v); }
  __device__ int id(int64_t p) const { return sr[p]; }
};

template <class S, int K, bool SILU, bool SEQ>
__global__ void __launch_bounds__(kBwdBlock) bwd_kernel(const BwdArgs a) {
  using raw = typename S::raw;
  const int64_t id = (int64_t)blockIdx.x * kBwdBlock + threadIdx.x;
  if (id >= a.lanes) return;
  const int64_t bg = id / a.C;
  const int64_t c = id - bg * a.C;
  const int64_t b = bg / a.ngr;
  const int64_t g = bg - b * a.ngr;
  GlobalSrc<S, K> src{static_cast<const raw*>(a.x) + b * a.x_sb + c * a.x_sc,
                      static_cast<const raw*>(a.dout) + b * a.d_sb + c * a.d_sc,
                      static_cast<raw*>(a.dx) + b * a.g_sb + c * a.g_sc,
                      a.init ? static_cast<const raw*>(a.init) + b * a.is_b + c * a.is_c : nullptr,
                      SEQ ? a.seq + b * a.L : nullptr, a.x_sl, a.d_sl, a.g_sl, a.is_i};
  float w[K], pw[K], pb = 0.0f;
  load_params<K>(a.w, a.w_dtype, c * K, w);
  const float beta = a.bias ? load_param(a.bias, a.w_dtype, c) : 0.0f;
#pragma unroll
  for (int k = 0; k < K; ++k) pw[k] = 0.0f;
  const int64_t tt1 = (g + 1) * a.tpi < a.ntt ? (g + 1) * a.tpi : a.ntt;
  for (int64_t tt = g * a.tpi; tt < tt1; ++tt)
    walk_tile<S, K, SILU, SEQ, false, 0>(a, b, c, tt * a.T, src, w, beta, pw, pb);
  store_partials<K>(a, b, g, c, pw, pb);
}

// Geometry of the LDS path's tiles: 64 channels x T steps, staged with V steps of
// margin on either side for the halos.
template <class S>
struct LdsGeom {
  static constexpr int V = S::V;
  // The tile length: 32 steps keeps a 16-bit tile's LDS near 11 KB, so about 14
  // waves fit on a CU; the K-1 step halo is recomputed per tile.
  static constexpr int T = 32;
  static constexpr int ES = sizeof(typename S::raw);
  static constexpr int XN = T + 2 * V;                  // staged x positions: [t0 - V, t0 + T + V)
  static constexpr int GN = T + V;                      // staged dout positions: [t0, t0 + T + V)
  // channel-first pitches (elements), odd in dwords
  static constexpr int XP = ((XN * ES / 4) | 1) * 4 / ES;
  static constexpr int GP = ((GN * ES / 4) | 1) * 4 / ES;
  static constexpr int CF_WORDS = 64 * (XP + GP) * ES / 4;
  static constexpr int CL_WORDS = (XN + GN) * 64 * ES / 4;
};

template <class S, int PS>
struct LdsSrc {
  using raw = typename S::raw;
  raw* xs;                 // this lane's channel in the staged x tile, at position t0 - V
  const raw* gs;           // ... in the staged dout tile, at position t0
  const int32_t* ids;      // the staged sequence ids, at position t0 - V (with seq_idx)
  int64_t t0;              // PS: elements between consecutive positions
  __device__ float x(int64_t p) const { return S::to_f(xs[(p - t0 + S::V) * PS]); }
  __device__ float g(int64_t p) const { return S::to_f(gs[(p - t0) * PS]); }
  __device__ void put_dx(int64_t j, float v) const { xs[(j - t0 + S::V) * PS] = S::from_f(v); }
  // All lanes of the workgroup share (b, t): the id is wave-uniform, so the masks
  // built from it are scalar.
  __device__ int id(int64_t p) const { return __builtin_amdgcn_readfirstlane(ids[p - t0 + S::V]); }
};

__device__ inline void lds_put16(void* p, u32x4 v) {
  uint32_t* d = static_cast<uint32_t*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) d[i] = dword(v, i);
}

__device__ inline u32x4 lds_get16(const void* p) {
  const uint32_t* d = static_cast<const uint32_t*>(p);
  return u32x4{d[0], d[1], d[2], d[3]};
}

// One tile's staged vectors: x over [t0 - V, t0 + T + V) and dout over
// [t0, t0 + T + V), NX + NG 16-byte vectors per lane; with seq_idx also the ids
// over [t0 - V, t0 + T + V), one per lane (XN <= 64).
template <class S>
struct Staged {
  static constexpr int NX = LdsGeom<S>::XN / S::V, NG = LdsGeom<S>::GN / S::V;
  u32x4 x[NX], g[NG];
  int32_t id;
};

// Issues every load of tile t0 (absent vectors, outside [0, L) or past C, load
// from the zero array; L and C are multiples of V on this path), with no wait.
// Channel-first: NX (NG) consecutive lanes read one channel's run, so each
// instruction covers whole runs of consecutive addresses.  Channel-last: 64 / V
// consecutive lanes read one step's 64 channels.  `ln` is the lane index made
// opaque to the compiler per tile, so that it recomputes the row offsets rather
// than keeping one per load in registers for the whole kernel.
// The V channels ck .. ck+V-1 of one channel-last step row (element ck at `p`),
// zeros from channel C on, by element loads (the vector that straddles C when C
// is not a multiple of V).
template <class raw, int V>
__device__ inline u32x4 load_channels_upto(const raw* p, int64_t ck, int64_t C) {
  raw part[V];
#pragma unroll
  for (int i = 0; i < V; ++i) part[i] = ck + i < C ? p[i] : raw(0);
  u32x4 v;
  __builtin_memcpy(&v, part, 16);
  return v;
}

// ODD (channel-last only): step rows that are not 16-byte aligned (C not a
// multiple of V, or an offset channel view): unaligned 16-byte loads, and the
// vector that straddles C element by element.
template <class S, bool CL, bool SEQ, bool ODD>
__device__ inline void stage_issue(const BwdArgs& a, const typename S::raw* xb, const typename S::raw* gb,
                                   const int32_t* sr, int64_t c0, int64_t t0, int ln, Staged<S>& st) {
  constexpr int V = S::V, NX = Staged<S>::NX, NG = Staged<S>::NG, NS = 64 / V;
  const int64_t L = a.L, C = a.C;
  const uintptr_t zero = reinterpret_cast<uintptr_t>(kZeroSrc);
  if constexpr (SEQ) {                             // the ids first: the walk reads them from LDS
    const int64_t p = t0 - V + ln;
    st.id = gload<int32_t>(pick(ln < LdsGeom<S>::XN && p >= 0 && p < L, reinterpret_cast<uintptr_t>(sr + p), zero));
  }
  if constexpr (!CL) {
    constexpr int ES = sizeof(typename S::raw);
    if (a.off24 && c0 + 64 <= C && t0 >= V && t0 + LdsGeom<S>::T + V <= L) {
      // An interior tile: every vector exists.  A wave-uniform base plus a 24-bit
      // byte offset per lane (one multiply-add).
      const uintptr_t xw = reinterpret_cast<uintptr_t>(xb + c0 * a.x_sc + (t0 - V));
      const uintptr_t gw = reinterpret_cast<uintptr_t>(gb + c0 * a.d_sc + t0);
      const uint32_t xs = (uint32_t)(a.x_sc * ES), gs = (uint32_t)(a.d_sc * ES);
#pragma unroll
      for (int i = 0; i < NX; ++i) {
        const uint32_t q = (uint32_t)ln + 64u * i, r = q / NX;
        st.x[i] = gload16_stream(xw + (__umul24(r, xs) + (q - r * NX) * 16u));
      }
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        const uint32_t q = (uint32_t)ln + 64u * i, r = q / NG;
        st.g[i] = gload16_stream(gw + (__umul24(r, gs) + (q - r * NG) * 16u));
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const int q = ln + 64 * i, r = q / NX;
      const int64_t p = t0 - V + (q - r * NX) * V;
      st.x[i] = gload<u32x4>(pick(c0 + r < C && p >= 0 && p < L,
                                  reinterpret_cast<uintptr_t>(xb + (c0 + r) * a.x_sc + p), zero));
    }
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const int q = ln + 64 * i, r = q / NG;
      const int64_t p = t0 + (q - r * NG) * V;
      st.g[i] = gload<u32x4>(pick(c0 + r < C && p < L, reinterpret_cast<uintptr_t>(gb + (c0 + r) * a.d_sc + p), zero));
    }
  } else {
    const int64_t ck = c0 + (ln % NS) * V;         // the lane's first channel
    const int s0 = ln / NS;                        // and first step
    const bool whole = ODD ? ck + V <= C : ck < C;
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const int64_t p = t0 - V + s0 + i * V;
      st.x[i] = gload<u32x4>(pick(whole && p >= 0 && p < L, reinterpret_cast<uintptr_t>(xb + p * a.x_sl + ck), zero));
    }
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const int64_t p = t0 + s0 + i * V;
      st.g[i] = gload<u32x4>(pick(whole && p < L, reinterpret_cast<uintptr_t>(gb + p * a.d_sl + ck), zero));
    }
    if constexpr (ODD) {
      if (ck < C && ck + V > C) {                  // the vector that straddles C
#pragma unroll
        for (int i = 0; i < NX; ++i) {
          const int64_t p = t0 - V + s0 + i * V;
          if (p >= 0 && p < L) st.x[i] = load_channels_upto<typename S::raw, V>(xb + p * a.x_sl + ck, ck, C);
        }
#pragma unroll
        for (int i = 0; i < NG; ++i) {
          const int64_t p = t0 + s0 + i * V;
          if (p < L) st.g[i] = load_channels_upto<typename S::raw, V>(gb + p * a.d_sl + ck, ck, C);
        }
      }
    }
  }
}

// Writes a tile's staged vectors to LDS (channel-first: channel-major rows of
// pitch XP / GP; channel-last: step-major, 64 channels to a step).
template <class S, bool CL, bool SEQ>
__device__ inline void stage_put(typename S::raw* lx, typename S::raw* lg, int32_t* lids, int ln,
                                 const Staged<S>& st) {
  using G = LdsGeom<S>;
  constexpr int V = S::V, NX = Staged<S>::NX, NG = Staged<S>::NG, NS = 64 / V;
  if constexpr (SEQ)
    if (ln < G::XN) lids[ln] = st.id;
  if constexpr (!CL) {
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const int q = ln + 64 * i, r = q / NX;
      lds_put16(lx + r * G::XP + (q - r * NX) * V, st.x[i]);
    }
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const int q = ln + 64 * i, r = q / NG;
      lds_put16(lg + r * G::GP + (q - r * NG) * V, st.g[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < NX; ++i) lds_put16(lx + (ln / NS + i * V) * 64 + (ln % NS) * V, st.x[i]);
#pragma unroll
    for (int i = 0; i < NG; ++i) lds_put16(lg + (ln / NS + i * V) * 64 + (ln % NS) * V, st.g[i]);
  }
}

// LDS path: a wave takes a group of consecutive tiles of one (b, 64 channels).
// Tile n's loads are issued before tile n-1's walk (software pipelining within
// the wave; the walk reads nothing from global memory except dfinal_states in a
// row's last tile, which has no successor in flight: the sequence ids are staged
// in LDS with the tile).  A tile is written to LDS, walked from LDS, and its dx, parked in the
// LDS slots of the x values that the walk no longer needs, is stored back with
// 16-byte stores.  Channel-first tiles are channel-major with an odd dword pitch
// (the walk's reads, one channel per lane, fall in distinct banks); channel-last
// tiles step-major.
template <class S, int K, bool SILU, bool SEQ, bool CL, bool ODD>
__global__ void __launch_bounds__(64) bwd_lds_kernel(const BwdArgs a) {
  using raw = typename S::raw;
  using G = LdsGeom<S>;
  constexpr int V = G::V, H = K - 1, NS = 64 / V;
  // Prefetch where a work item has several tiles (channel-last).
  constexpr bool PREFETCH = CL;
  constexpr int WORDS = CL ? G::CL_WORDS : G::CF_WORDS;   // LDS per wave bounds the waves per CU
  __shared__ uint32_t lds[WORDS + (SEQ ? 64 : 0)];
  raw* lx = reinterpret_cast<raw*>(lds);
  raw* lg = lx + (CL ? G::XN * 64 : 64 * G::XP);
  int32_t* lids = reinterpret_cast<int32_t*>(lds + WORDS);

  const int lane = threadIdx.x;
  const int64_t ncg = (a.C + 63) / 64;
  // Channel-last: each XCD takes one contiguous range of items (neighbouring channel
  // groups of the same rows, and the next tile group's halo rows), as in the
  // channel-last forward; channel-first keeps the hardware's round-robin order.
  const int64_t item = CL ? xcd_order(blockIdx.x, gridDim.x >> 3, gridDim.x & 7) : blockIdx.x;
  const int64_t bg = item / ncg;
  const int64_t c0 = (item - bg * ncg) * 64;
  const int64_t b = bg / a.ngr;
  const int64_t g = bg - b * a.ngr;
  const int64_t L = a.L, C = a.C;
  const raw* xb = static_cast<const raw*>(a.x) + b * a.x_sb;
  const raw* gb = static_cast<const raw*>(a.dout) + b * a.d_sb;
  raw* db = static_cast<raw*>(a.dx) + b * a.g_sb;
  const int64_t c = c0 + lane;
  constexpr int cs = CL ? 1 : G::XP, gcs = CL ? 1 : G::GP, ps = CL ? 64 : 1;

  // Parameters first: they are the only loads the walk needs besides LDS.
  float w[K], pw[K], pb = 0.0f;
  load_params<K>(a.w, a.w_dtype, (c < C ? c : 0) * K, w);
  const float beta = a.bias ? load_param(a.bias, a.w_dtype, c < C ? c : 0) : 0.0f;
#pragma unroll
  for (int k = 0; k < K; ++k) pw[k] = 0.0f;

  const int64_t tt0 = g * a.tpi;
  const int64_t tt1 = (g + 1) * a.tpi < a.ntt ? (g + 1) * a.tpi : a.ntt;
  Staged<S> st;
  // dx of the previous tile, read out of LDS after its walk and stored after the
  // next tile is in LDS: the hardware waits for loads in issue order, so stores
  // issued just before the wait for the next tile's loads would be waited for too.
  constexpr int ND = G::T / V;                     // dx vectors per lane and tile
  u32x4 dxv[ND];
  int64_t dx_t0 = -1;
  int dx_n = 0;
  auto store_dx = [&](int ln) {
    if constexpr (!CL) {
      if (a.off24 && c0 + 64 <= C && dx_n == G::T) {   // as the interior staging
        const uintptr_t dw = reinterpret_cast<uintptr_t>(db + c0 * a.g_sc + dx_t0);
        const uint32_t ds = (uint32_t)(a.g_sc * sizeof(raw));
#pragma unroll
        for (int i = 0; i < ND; ++i) {
          const uint32_t q = (uint32_t)ln + 64u * i, r = q / ND;
          gstore16_stream(dw + (__umul24(r, ds) + (q - r * ND) * 16u), dxv[i]);
        }
        return;
      }
    }
#pragma unroll
    for (int i = 0; i < ND; ++i) {
      if constexpr (!CL) {
        const int q = ln + 64 * i, r = q / ND, k = q - r * ND;
        if (c0 + r < C && k * V < dx_n) store16_stream(db + (c0 + r) * a.g_sc + dx_t0 + k * V, dxv[i]);
      } else {
        const int64_t ck = c0 + (ln % NS) * V;
        const int s = ln / NS + i * V;
        if constexpr (ODD) {
          if (s < dx_n && ck + V <= C) {
            store16_stream(db + (dx_t0 + s) * a.g_sl + ck, dxv[i]);
          } else if (s < dx_n && ck < C) {          // the vector that straddles C
            raw part[V];
            __builtin_memcpy(part, &dxv[i], 16);
#pragma unroll
            for (int e = 0; e < V; ++e)
              if (ck + e < C) db[(dx_t0 + s) * a.g_sl + ck + e] = part[e];
          }
        } else {
          if (ck < C && s < dx_n) store16_stream(db + (dx_t0 + s) * a.g_sl + ck, dxv[i]);
        }
      }
    }
  };

  const int32_t* sr = SEQ ? a.seq + b * L : nullptr;
  if constexpr (PREFETCH) stage_issue<S, CL, SEQ, ODD>(a, xb, gb, sr, c0, tt0 * a.T, lane, st);
  for (int64_t tt = tt0; tt < tt1; ++tt) {
    const int64_t t0 = tt * a.T;
    int ln = lane;
    asm volatile("" : "+v"(ln));
    if constexpr (!PREFETCH) stage_issue<S, CL, SEQ, ODD>(a, xb, gb, sr, c0, t0, ln, st);
    __syncthreads();                               // the previous tile's dx has left LDS
    stage_put<S, CL, SEQ>(lx, lg, lids, ln, st);
    if (t0 == 0 && a.init && c < C) {              // the history left of t = 0
#pragma unroll
      for (int i = 0; i < H; ++i)
        lx[lane * cs + (V - H + i) * ps] =
            static_cast<const raw*>(a.init)[b * a.is_b + c * a.is_c + i * a.is_i];
    }
    if (dx_t0 >= 0) store_dx(ln);
    if constexpr (PREFETCH)
      if (tt + 1 < tt1) stage_issue<S, CL, SEQ, ODD>(a, xb, gb, sr, c0, t0 + a.T, ln, st);
    __syncthreads();

    // With seq_idx, a tile right of the history whose rows t0-H .. t0+T+H-1 (those
    // inside [0, L)) all carry one id keeps every term, so the unmasked walk gives
    // the same bits (every mask and the dfinal_states condition read true).
    bool one_seq = false;
    if constexpr (SEQ) {
      const int64_t p = t0 - V + lane;             // the lane's staged position
      const int64_t hi = t0 + G::T + H < L ? t0 + G::T + H : L;
      const int ref = lids[V];                     // the id at t0
      const bool same = lane >= G::XN || p < t0 - H || p >= hi || lids[lane] == ref;
      one_seq = t0 >= H && t0 < L && __all(same);
    }
    if (c < C) {
      LdsSrc<S, ps> src{lx + lane * cs, lg + lane * gcs, lids, t0};
      const bool inner = t0 + G::T + H <= L && (t0 > 0 || !a.dinit);   // an interior tile
      if (SEQ && one_seq) {
        if (inner)
          walk_tile<S, K, SILU, false, true, G::T>(a, b, c, t0, src, w, beta, pw, pb);
        else
          walk_tile<S, K, SILU, false, false, 0>(a, b, c, t0, src, w, beta, pw, pb);
      } else if (inner) {
        walk_tile<S, K, SILU, SEQ, true, G::T>(a, b, c, t0, src, w, beta, pw, pb);
      } else {
        walk_tile<S, K, SILU, SEQ, false, 0>(a, b, c, t0, src, w, beta, pw, pb);
      }
    }
    __syncthreads();

    // Read this tile's dx (the steps [t0, t0 + dx_n)) out of LDS, in the staging's
    // lane mapping; vectors past dx_n are read but never stored.
#pragma unroll
    for (int i = 0; i < ND; ++i) {
      if constexpr (!CL) {
        const int q = ln + 64 * i, r = q / ND, k = q - r * ND;
        dxv[i] = lds_get16(lx + r * G::XP + (k + 1) * V);
      } else {
        dxv[i] = lds_get16(lx + (ln / NS + i * V + V) * 64 + (ln % NS) * V);
      }
    }
    dx_t0 = t0;
    dx_n = (int)((t0 + a.T < L ? t0 + a.T : L) - t0);
    if constexpr (!PREFETCH) {                     // no load in flight: store at once
      store_dx(ln);
      dx_t0 = -1;
    }
  }
  if (dx_t0 >= 0) store_dx(lane);
  if (c < C) store_partials<K>(a, b, g, c, pw, pb);
}

// ---- channel-first, registers only ------------------------------------------------
//
// For x, dout and dx unit-stride in time (16-byte aligned rows, L a multiple of V).
// The forward's channel-first layout of work: a segment is
// 64 lanes x U vectors x V steps of one (b, c) row; lane l holds vectors
// l, l + 64, ..., so every load and store moves 1 KB of consecutive addresses.
// The K-1 inputs before a lane's vector come from lane l-1 (DPP shift right) or,
// for lane 0, from lane 63 of the previous vector or the segment's history; z
// and dz are recomputed per element exactly as in walk_tile.  dx needs the dz of
// the K-1 steps after the element: from lane l+1 (DPP shift left), for lane 63
// from lane 0 of the next vector, and for the segment's last vector from dz
// recomputed over the K-1 steps past the segment.  So dx comes out with the same
// bits as in the other paths.  The parameter gradients: each lane sums its
// elements in step order, then a fixed-order 64-lane sum over DPP lane patterns
// (wave_sum) gives the segment's sum in lane 0, written as one partial row per
// (b, segment).  With seq_idx each lane also loads the ids of its elements, and
// the ids before and after its vector travel with x and dz: the same keep() as
// the walk's decides every term of z, of dx and of the parameter sums, and which
// dfinal_states entries and history taps count.
// x and dout vectors and dx are touched once and use streaming (non-temporal)
// accesses, as do the LDS kernels' interior staging loads and dx stores; the
// vectors just past a segment, which the next segment reads again, are ordinary
// loads.
constexpr int kBwdRegUnroll = 4;                  // vectors per lane and segment

// Lane l receives lane l+1's value; lane 63 receives `carry`.  DPP wave_shl:1.
__device__ inline float shift_out(float carry, float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      __builtin_bit_cast(int, carry), __builtin_bit_cast(int, v), 0x130, 0xf, 0xf, false));
}

// v plus the value of lane p(i) for the DPP lane pattern CTRL (row_mask and
// bank_mask full: every lane reads a lane of its own row).
template <int CTRL>
__device__ inline float dpp_pair_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

// Sum over the 64 lanes in a fixed order, valid in lane 0.  Within each row of 16
// lanes: swap neighbours (quad_perm 1,0,3,2), swap pairs (quad_perm 2,3,0,1), then
// the half-row and row mirrors, each of which pairs a lane with one holding the
// sum of the other quad / half; partners add the same two values, so after the
// four steps every lane of a row holds the row's sum with the same bits.  Lane 0
// then adds the sums of rows 1, 2 and 3 in that order.
__device__ inline float wave_sum(float v) {
  v = dpp_pair_add<0xB1>(v);
  v = dpp_pair_add<0x4E>(v);
  v = dpp_pair_add<0x141>(v);
  v = dpp_pair_add<0x140>(v);
  const int bits = __builtin_bit_cast(int, v);
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(bits, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(bits, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(bits, 48));
  return ((v + r1) + r2) + r3;
}

// Everything one segment reads, loaded ahead of its arithmetic: the lane's x and
// dout vectors, the vectors just past the segment, the K-1 inputs before it, the
// channel's parameters (as the aligned dwords that hold them, so that the loads do
// not depend on the weight dtype) and dfinal_states.  Absent data loads from the
// zero array; nothing is converted until the arithmetic.
template <class S, int K, bool SEQ>
struct RegLoads {
  u32x4 xv[kBwdRegUnroll], gv[kBwdRegUnroll], hx, hg;
  typename S::raw hist[K - 1], dfs[K - 1];
  uint32_t w[K], bias;
  // with seq_idx: the ids of each vector's elements and of the V steps past the
  // segment, the ids of the K-1 steps before it (seq_idx[b, 0] for the history left
  // of t = 0), and the row's first and last ids
  u32x4 iv[SEQ ? kBwdRegUnroll : 1][S::V / 4], hi[S::V / 4];
  int32_t hist_id[K - 1], first_id, last_id;
};

// Ids as ints from the vectors that hold them.
template <int V>
__device__ inline void unpack_ids(const u32x4 (&v)[V / 4], int (&id)[V]) {
#pragma unroll
  for (int r = 0; r < V / 4; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) id[4 * r + i] = (int)dword(v[r], i);
}

__device__ inline int shift_out(int carry, int v) {
  return __builtin_amdgcn_update_dpp(carry, v, 0x130, 0xf, 0xf, false);
}

struct RegPos {
  int64_t b, c, seg;
};

// Where a segment lies in its row: inside with the K-1 steps past it
// (t0 + span + K - 1 <= L; with ODD rows, the V steps past it), ending exactly at
// L (every vector inside, nothing past it), or anything else (the row's last,
// partial segment).
enum { kSegInner = 0, kSegLast = 1, kSegEdge = 2 };

// ODD: rows that are not 16-byte aligned (L not a multiple of V, or an offset
// view).  Their 16-byte accesses are unaligned (the GPU serves them), the one
// vector that straddles L moves element by element, and loads whose address is
// the same in every lane go element by element: the compiler may turn such a
// 16-byte load into a scalar load, which ignores the address's low two bits.

// Elements e .. e+V-1 of a row (element 0 at `base`) as one 16-byte vector: a
// single load when they all lie before `n`, else element by element with zeros
// from n on, so no access leaves the row.
template <class raw, int V>
__device__ inline u32x4 load_row_vec(uintptr_t base, int64_t e, int64_t n) {
  if (e + V <= n) return gload16_stream(base + e * (int64_t)sizeof(raw));
  raw part[V];
#pragma unroll
  for (int i = 0; i < V; ++i) part[i] = e + i < n ? gload<raw>(base + (e + i) * (int64_t)sizeof(raw)) : raw(0);
  u32x4 v;
  __builtin_memcpy(&v, part, 16);
  return v;
}

// The ids of steps t .. t+V-1 of a row of seq_idx (step 0 at `base`), zeros from n on.
template <int V>
__device__ inline void load_row_ids(uintptr_t base, int64_t t, int64_t n, u32x4 (&out)[V / 4]) {
  if (t + V <= n) {
#pragma unroll
    for (int r = 0; r < V / 4; ++r) out[r] = gload<u32x4>(base + t * 4 + r * 16);
    return;
  }
  int32_t part[V];
#pragma unroll
  for (int i = 0; i < V; ++i) part[i] = t + i < n ? gload<int32_t>(base + (t + i) * 4) : 0;
  __builtin_memcpy(&out[0], part, V * 4);
}

// Elements t .. t+N-1 of a row (zeros from n on) in the low elements of a 16-byte
// vector, by element loads (for addresses that are the same in every lane).
template <class T, int N>
__device__ inline u32x4 load_row_head(uintptr_t base, int64_t t, int64_t n) {
  T part[16 / sizeof(T)] = {};
#pragma unroll
  for (int j = 0; j < N; ++j) part[j] = t + j < n ? gload<T>(base + (t + j) * (int64_t)sizeof(T)) : T(0);
  u32x4 v;
  __builtin_memcpy(&v, part, 16);
  return v;
}

template <class S, int K, bool SEQ, int MODE, bool ODD>
__device__ inline void reg_issue(const BwdArgs& a, const RegPos& p, int lane, RegLoads<S, K, SEQ>& q) {
  using raw = typename S::raw;
  constexpr bool EDGE = MODE == kSegEdge;
  constexpr int V = S::V, U = kBwdRegUnroll, H = K - 1, SPAN = 64 * V * U, ES = sizeof(raw);
  const int64_t L = a.L;
  const int64_t t0 = p.seg * SPAN, t1 = t0 + SPAN;
  const uintptr_t zero = reinterpret_cast<uintptr_t>(kZeroSrc);
  const raw* xr = static_cast<const raw*>(a.x) + p.b * a.x_sb + p.c * a.x_sc;
  const raw* gr = static_cast<const raw*>(a.dout) + p.b * a.d_sb + p.c * a.d_sc;
  const uint32_t lo = (uint32_t)lane * (V * ES);
  const uintptr_t xs = reinterpret_cast<uintptr_t>(xr + t0), gs = reinterpret_cast<uintptr_t>(gr + t0);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t o = lo + (uint32_t)(u * 64 * V * ES);
    if constexpr (EDGE && ODD) {
      const int64_t e = (int64_t)(u * 64 + lane) * V;
      q.xv[u] = load_row_vec<raw, V>(xs, e, L - t0);
      q.gv[u] = load_row_vec<raw, V>(gs, e, L - t0);
    } else if constexpr (EDGE) {
      const bool ok = t0 + (int64_t)(u * 64 + lane) * V < L;
      q.xv[u] = gload16_stream(pick(ok, xs + o, zero));
      q.gv[u] = gload16_stream(pick(ok, gs + o, zero));
    } else {                                       // every vector and the halo lie inside the row
      q.xv[u] = gload16_stream(xs + o);
      q.gv[u] = gload16_stream(gs + o);
    }
  }
  if constexpr (ODD && MODE != kSegLast) {         // the H steps past the segment (all it reads)
    q.hx = load_row_head<raw, H>(reinterpret_cast<uintptr_t>(xr), t1, L);
    q.hg = load_row_head<raw, H>(reinterpret_cast<uintptr_t>(gr), t1, L);
  } else if constexpr (EDGE) {
    q.hx = gload<u32x4>(pick(t1 < L, reinterpret_cast<uintptr_t>(xr + t1), zero));
    q.hg = gload<u32x4>(pick(t1 < L, reinterpret_cast<uintptr_t>(gr + t1), zero));
  } else if constexpr (MODE == kSegLast) {
    q.hx = q.hg = u32x4{0u, 0u, 0u, 0u};         // nothing past L; not read
  } else {
    q.hx = gload<u32x4>(reinterpret_cast<uintptr_t>(xr + t1));
    q.hg = gload<u32x4>(reinterpret_cast<uintptr_t>(gr + t1));
  }
  const uintptr_t ir = reinterpret_cast<uintptr_t>(static_cast<const raw*>(a.init) + p.b * a.is_b + p.c * a.is_c);
  const uintptr_t fr = reinterpret_cast<uintptr_t>(static_cast<const raw*>(a.dfs) + p.b * a.fs_b + p.c * a.fs_c);
#pragma unroll
  for (int j = 0; j < H; ++j) {
    const int64_t src = t0 - H + j;
    const uintptr_t from_init = pick(a.init != nullptr, ir + (src + H) * a.is_i * ES, zero);
    q.hist[j] = gload<raw>(pick(src >= 0, reinterpret_cast<uintptr_t>(xr + src), from_init));
    q.dfs[j] = gload<raw>(pick(a.dfs != nullptr, fr + j * a.fs_i * ES, zero));
  }
  if constexpr (SEQ) {
    const uintptr_t sr = reinterpret_cast<uintptr_t>(a.seq + p.b * L);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t t = t0 + (int64_t)(u * 64 + lane) * V;
      if constexpr (EDGE && ODD) {
        load_row_ids<V>(sr, t, L, q.iv[u]);
      } else {
        const uintptr_t at = pick(!EDGE || t < L, sr + t * 4, zero);
#pragma unroll
        for (int r = 0; r < V / 4; ++r) q.iv[u][r] = gload<u32x4>(at + (EDGE && t >= L ? 0 : r * 16));
      }
    }
    if constexpr (ODD) {                           // ids of the H steps past the segment
#pragma unroll
      for (int r = 0; r < V / 4; ++r) q.hi[r] = u32x4{0u, 0u, 0u, 0u};
      if constexpr (MODE != kSegLast) q.hi[0] = load_row_head<int32_t, H>(sr, t1, L);
    } else {
      const uintptr_t ah = pick(MODE != kSegLast && t1 < L, sr + t1 * 4, zero);
#pragma unroll
      for (int r = 0; r < V / 4; ++r) q.hi[r] = gload<u32x4>(ah + (MODE != kSegLast && t1 < L ? r * 16 : 0));
    }
#pragma unroll
    for (int j = 0; j < H; ++j) {
      const int64_t src = t0 - H + j;              // the history carries seq_idx[b, 0]
      q.hist_id[j] = gload<int32_t>(pick(src >= 0, sr + src * 4, pick(a.init != nullptr, sr, zero)));
    }
    q.first_id = gload<int32_t>(sr);
    q.last_id = gload<int32_t>(sr + (L - 1) * 4);
  }
  const int64_t wb = a.w_dtype == CCV_DT_F32 ? 4 : 2;
  const uintptr_t wl = reinterpret_cast<uintptr_t>(a.w) + p.c * K * wb;
#pragma unroll
  for (int k = 0; k < K; ++k) q.w[k] = gload<uint32_t>((wl + k * wb) & ~(uintptr_t)3);
  q.bias = gload<uint32_t>(pick(a.bias != nullptr, (reinterpret_cast<uintptr_t>(a.bias) + p.c * wb) & ~(uintptr_t)3, zero));
}

// A parameter from the aligned dword that holds it (element i of the array).
__device__ inline float reg_param(uint32_t d, int dtype, int64_t i) {
  if (dtype == CCV_DT_F32) return __builtin_bit_cast(float, d);
  const uint32_t h = (i & 1) ? d >> 16 : d & 0xffffu;
  return dtype == CCV_DT_BF16 ? __builtin_bit_cast(float, h << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// The arithmetic and stores of one segment from its loads.  kSegInner: no
// position needs a check and dfinal_states does not reach the segment.  kSegLast:
// no position needs a check, but lane 63 of the last vector holds the row's last
// H steps: it skips the taps that would read dz past L and adds dfinal_states,
// exactly as the checked form does.  kSegEdge: every check in place.
template <class S, int K, bool SILU, bool SEQ, int MODE, bool ODD>
__device__ inline void reg_compute(const BwdArgs& a, const RegPos& p, int lane, const RegLoads<S, K, SEQ>& q) {
  using raw = typename S::raw;
  constexpr bool EDGE = MODE == kSegEdge, LAST = MODE == kSegLast;
  constexpr int V = S::V, U = kBwdRegUnroll, H = K - 1, SPAN = 64 * V * U, ES = sizeof(raw);
  const int64_t L = a.L;
  const int64_t b = p.b, c = p.c, seg = p.seg;
  const int64_t t0 = seg * SPAN, t1 = t0 + SPAN;
  const uint32_t lo = (uint32_t)lane * (V * ES);
  raw* dxr = static_cast<raw*>(a.dx) + b * a.g_sb + c * a.g_sc;
  const bool has_dfs = EDGE && a.dfs != nullptr;
  const bool tail = LAST && lane == 63;            // the row's last H steps, in the last vector
  const bool tail_dfs = tail && a.dfs != nullptr;

  float w[K], hist[H], dfs[H];
#pragma unroll
  for (int k = 0; k < K; ++k) w[k] = reg_param(q.w[k], a.w_dtype, c * K + k);
  const float beta = a.bias ? reg_param(q.bias, a.w_dtype, c) : 0.0f;
#pragma unroll
  for (int j = 0; j < H; ++j) {
    hist[j] = S::to_f(q.hist[j]);
    dfs[j] = S::to_f(q.dfs[j]);
  }

  float pw[K], pb = 0.0f;
#pragma unroll
  for (int k = 0; k < K; ++k) pw[k] = 0.0f;
  float carry[H];                                  // X~ of the H steps before lane 0's vector
  int carry_id[H];                                 // and their ids
#pragma unroll
  for (int j = 0; j < H; ++j) {
    carry[j] = hist[j];
    carry_id[j] = SEQ ? q.hist_id[j] : 0;
  }
  float dzp[V], dz0[H];                            // dz of the previous vector; lane 0's first H of vector 0
  int idp[V], id0[H];                              // their ids

  // dx of vector u with dz d[] (ids di[]) and the dz of the H steps after each
  // lane's vector (next[], ids nid[]), stored when inside [0, L).  With seq_idx an
  // output's tap counts when its id is the element's.
  auto put_dx = [&](int u, const float (&d)[V], const int (&di)[V], const float (&next)[H],
                    const int (&nid)[H]) {
    const int64_t base = t0 + (int64_t)(u * 64 + lane) * V;
    const bool skip_next = LAST && u == U - 1 && tail;
    float y[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
      float acc = 0.0f;
#pragma unroll
      for (int k = 0; k < K; ++k) {                // output t = base + i + H - k uses tap k
        const int j = i + H - k;
        const float dv = j < V ? d[j] : next[j - V];
        const bool same = !SEQ || (j < V ? di[j] : nid[j - V]) == di[i];
        if (j >= V && LAST) {
          const float f = __builtin_fmaf(w[k], dv, acc);
          acc = skip_next || !same ? acc : f;
        } else if (!EDGE || base + i + H - k < L) {
          const float f = __builtin_fmaf(w[k], dv, acc);
          acc = same ? f : acc;
        }
      }
      const bool fin_kept = !SEQ || di[i] == q.last_id;   // final_states keep the last sequence's steps
      if (has_dfs) {                               // the last H steps take dfinal_states
        const int64_t t = base + i;
#pragma unroll
        for (int m = 0; m < H; ++m)
          if (t == L - H + m && fin_kept) acc += dfs[m];
      }
      if (LAST && u == U - 1 && i >= V - H) {
        if (tail_dfs && fin_kept) acc += dfs[i - (V - H)];
      }
      y[i] = acc;
    }
    if constexpr (ODD && EDGE) {
      raw* const dst = reinterpret_cast<raw*>(reinterpret_cast<uintptr_t>(dxr + t0) + lo + u * 64 * V * ES);
      if (base + V <= L) {
        store16_stream(dst, S::pack(y));
      } else if (base < L) {                       // the vector that straddles L
#pragma unroll
        for (int i = 0; i < V; ++i)
          if (base + i < L) dst[i] = S::from_f(y[i]);
      }
    } else {
      const u32x4 pk = S::pack(y);
      if (!EDGE || base < L)
        store16_stream(reinterpret_cast<raw*>(reinterpret_cast<uintptr_t>(dxr + t0) + lo + u * 64 * V * ES), pk);
    }
  };

  // Lane 0 of the row's first vector: whether each of the H history steps before
  // it has an id (without a history, steps left of t = 0 have none and never count).
  const bool lead = lane == 0 && t0 == 0 && a.init == nullptr;
  bool done = false;                               // ODD: the rest of the segment lies past L
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if constexpr (ODD && EDGE) {
      if (u > 0 && t0 + (int64_t)u * 64 * V >= L) {
        // Group u and those after it lie past L: none of their steps has an output
        // or a parameter-gradient term, and the taps of group u-1 that would read
        // their dz are outside [0, L) and skipped by position.  Store group u-1
        // and stop (a wave-uniform exit).
        float next[H];
        int nid[H];
#pragma unroll
        for (int m = 0; m < H; ++m) {
          next[m] = shift_out(0.0f, dzp[m]);
          nid[m] = SEQ ? shift_out(0, idp[m]) : 0;
        }
        put_dx(u - 1, dzp, idp, next, nid);
        done = true;
        break;
      }
    }
    const int64_t tv = t0 + (int64_t)(u * 64 + lane) * V;   // this lane's vector's first step
    const bool okv = !EDGE || tv < L;
    float e[V], g[V];
    S::unpack(q.xv[u], e);
    S::unpack(q.gv[u], g);
    int id[V], hid[H];
    if constexpr (SEQ) unpack_ids<V>(q.iv[u], id);
    float h[H];
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
    float dz[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
      float xk[K];                                 // X~[t - H + k]
      bool keep[K];
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int j = i - H + k;
        xk[k] = j >= 0 ? e[j] : h[i + k];
        if constexpr (SEQ)
          keep[k] = j >= 0 ? id[j] == id[i] : !(lead && u == 0) && hid[i + k] == id[i];
        else
          keep[k] = true;
      }
      float z = beta;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const float f = __builtin_fmaf(w[k], xk[k], z);
        z = keep[k] ? f : z;
      }
      const float d = SILU ? g[i] * silu_slope(z) : g[i];
      const bool ok = ODD && EDGE ? tv + i < L : okv;   // ODD: the straddling vector's steps past L
      dz[i] = ok ? d : 0.0f;
      if (ok) {
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const float f = __builtin_fmaf(dz[i], xk[k], pw[k]);
          pw[k] = keep[k] ? f : pw[k];
        }
        pb += dz[i];
      }
    }
    if (u == 0) {
#pragma unroll
      for (int m = 0; m < H; ++m) {
        dz0[m] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, dz[m]), 0));
        id0[m] = SEQ ? __builtin_amdgcn_readlane(id[m], 0) : 0;
      }
    }
    if (u > 0) {
      float next[H];
      int nid[H];
#pragma unroll
      for (int m = 0; m < H; ++m) {
        next[m] = shift_out(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, dz[m]), 0)),
                            dzp[m]);
        nid[m] = SEQ ? shift_out(__builtin_amdgcn_readlane(id[m], 0), idp[m]) : 0;
      }
      put_dx(u - 1, dzp, idp, next, nid);
    }
#pragma unroll
    for (int i = 0; i < V; ++i) {
      dzp[i] = dz[i];
      idp[i] = SEQ ? id[i] : 0;
    }
  }
  // dz of the H steps past the segment (zero past L), for the last vector's lane 63.
  if (done) {
  } else if constexpr (LAST) {
    const float none[H] = {};
    const int none_id[H] = {};
    float next[H];
    int nid[H];
#pragma unroll
    for (int m = 0; m < H; ++m) {
      next[m] = shift_out(none[m], dzp[m]);
      nid[m] = SEQ ? shift_out(none_id[m], idp[m]) : 0;
    }
    put_dx(U - 1, dzp, idp, next, nid);
  } else {
    float e[V], g[V];
    S::unpack(q.hx, e);
    S::unpack(q.hg, g);
    int ida[V];                                    // ids of the steps past the segment
    if constexpr (SEQ) unpack_ids<V>(q.hi, ida);
    float hz[H];
#pragma unroll
    for (int m = 0; m < H; ++m) {
      float z = beta;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int j = m - H + k;                   // relative to t1
        const float f = __builtin_fmaf(w[k], j >= 0 ? e[j] : carry[H + j], z);
        z = !SEQ || (j >= 0 ? ida[j] : carry_id[H + j]) == ida[m] ? f : z;
      }
      const float d = SILU ? g[m] * silu_slope(z) : g[m];
      hz[m] = !EDGE || t1 < L ? d : 0.0f;
    }
    float next[H];
    int nid[H];
#pragma unroll
    for (int m = 0; m < H; ++m) {
      next[m] = shift_out(hz[m], dzp[m]);
      nid[m] = SEQ ? shift_out(ida[m], idp[m]) : 0;
    }
    put_dx(U - 1, dzp, idp, next, nid);
  }

  // d(initial_states): the history positions j = -H .. -1 of the row's first
  // segment; with seq_idx the history is the first sequence's (id seq_idx[b, 0]).
  if (t0 == 0 && a.dinit && lane < H) {
    const int j = lane - H;
    float acc = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int t = j + H - k;                     // < H: in lane 0's first vector
      float dv = 0.0f;
      int tid = 0;
#pragma unroll
      for (int m = 0; m < H; ++m) {
        dv = t == m ? dz0[m] : dv;
        tid = t == m ? id0[m] : tid;
      }
      if (t >= 0 && t < L && (!SEQ || tid == q.first_id)) acc = __builtin_fmaf(w[k], dv, acc);
    }
    if (has_dfs && (!SEQ || q.first_id == q.last_id)) {
#pragma unroll
      for (int m = 0; m < H; ++m)
        if (j == L - H + m) acc += dfs[m];
    }
    static_cast<raw*>(a.dinit)[b * a.di_b + c * a.di_c + (j + H) * a.di_i] = S::from_f(acc);
  }

  // The segment's parameter gradients: one partial row entry per (b, segment).
  float sw[K];
#pragma unroll
  for (int k = 0; k < K; ++k) sw[k] = wave_sum(pw[k]);
  const float sb = wave_sum(pb);
  if (lane == 0) {
    float* part = a.part + ((b * a.ngr + seg) * (K + 1)) * a.C + c;
#pragma unroll
    for (int k = 0; k < K; ++k) part[k * a.C] = sw[k];
    part[K * a.C] = sb;
  }
}

// With seq_idx: whether every step the segment's arithmetic reads carries one id
// (the segment's own steps, the K-1 before it, which at t = 0 must be a given
// history, and the V steps past it that feed the last vector's dx).  Then every
// mask of the walk reads true, and the unmasked arithmetic gives the same bits.
// The ids are loaded here on their own, so that neither form of the arithmetic
// holds them (or the other form's values) in registers.
template <class S, int K, int MODE, bool ODD>
__device__ inline bool reg_one_sequence(const BwdArgs& a, const RegPos& p, int lane) {
  constexpr bool EDGE = MODE == kSegEdge;
  constexpr int V = S::V, U = kBwdRegUnroll, H = K - 1, SPAN = 64 * V * U;
  const int64_t L = a.L, t0 = p.seg * SPAN, t1 = t0 + SPAN;
  if (t0 == 0 && a.init == nullptr) return false;  // the history left of t = 0 never counts
  const uintptr_t zero = reinterpret_cast<uintptr_t>(kZeroSrc);
  const uintptr_t sr = reinterpret_cast<uintptr_t>(a.seq + p.b * L);
  const int ref = __builtin_amdgcn_readfirstlane(gload<int32_t>(sr + t0 * 4));   // the id at t0
  bool ok = true;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t t = t0 + (int64_t)(u * 64 + lane) * V;
    if constexpr (ODD && EDGE) {
      u32x4 iv[V / 4];
      load_row_ids<V>(sr, t, L, iv);
#pragma unroll
      for (int r = 0; r < V / 4; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) ok = ok && (t + 4 * r + i >= L || (int)dword(iv[r], i) == ref);
    } else {
      const bool in = !EDGE || t < L;
#pragma unroll
      for (int r = 0; r < V / 4; ++r) {
        const u32x4 v = gload<u32x4>(pick(in, sr + t * 4 + r * 16, zero));
#pragma unroll
        for (int i = 0; i < 4; ++i) ok = ok && ((EDGE && t + 4 * r + i >= L) || (int)dword(v, i) == ref);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < H; ++j) {                   // at t0 = 0 the history carries seq_idx[b, 0]
    const int64_t src = t0 - H + j;
    ok = ok && gload<int32_t>(src >= 0 ? sr + src * 4 : sr) == ref;
  }
  if constexpr (MODE != kSegLast && ODD) {        // the V steps past the segment, as dwords
#pragma unroll
    for (int i = 0; i < V; ++i) ok = ok && (t1 + i >= L || gload<int32_t>(sr + (t1 + i) * 4) == ref);
  } else if constexpr (MODE != kSegLast) {
#pragma unroll
    for (int r = 0; r < V / 4; ++r) {
      const u32x4 v = gload<u32x4>(pick(t1 < L, sr + t1 * 4 + r * 16, zero));
#pragma unroll
      for (int i = 0; i < 4; ++i) ok = ok && (t1 + 4 * r + i >= L || (int)dword(v, i) == ref);
    }
  }
  return __all(ok);
}

// One segment: its loads, then its arithmetic, in the form for where it lies (and,
// with seq_idx, unmasked when it holds one sequence).
template <class S, int K, bool SILU, bool SEQ, int MODE, bool ODD>
__device__ inline void reg_segment_in(const BwdArgs& a, const RegPos& p, int lane) {
  if constexpr (SEQ) {
    if (reg_one_sequence<S, K, MODE, ODD>(a, p, lane)) {
      RegLoads<S, K, false> q;
      reg_issue<S, K, false, MODE, ODD>(a, p, lane, q);
      reg_compute<S, K, SILU, false, MODE, ODD>(a, p, lane, q);
      return;
    }
  }
  RegLoads<S, K, SEQ> q;
  reg_issue<S, K, SEQ, MODE, ODD>(a, p, lane, q);
  reg_compute<S, K, SILU, SEQ, MODE, ODD>(a, p, lane, q);
}

template <class S, int K, bool SILU, bool SEQ, bool ODD>
__device__ inline void reg_segment(const BwdArgs& a, const RegPos& p, int lane) {
  const int64_t t1 = (p.seg + 1) * (64 * kBwdRegUnroll * S::V);
  if (t1 + (ODD ? S::V : K - 1) <= a.L)
    reg_segment_in<S, K, SILU, SEQ, kSegInner, ODD>(a, p, lane);
  else if (t1 == a.L)
    reg_segment_in<S, K, SILU, SEQ, kSegLast, ODD>(a, p, lane);
  else
    reg_segment_in<S, K, SILU, SEQ, kSegEdge, ODD>(a, p, lane);
}

__device__ inline RegPos reg_pos(const BwdArgs& a, int64_t i) {
  const int64_t row = i / a.ntt;
  const int64_t b = row / a.C;
  return RegPos{b, row - b * a.C, i - row * a.ntt};
}

// Work item i = segment (row i / nseg, segment i % nseg), row = b * C + c, one
// wave per item: the hardware keeps as many waves resident as the registers allow
// and starts the next as one ends.  A segment's loads are issued together and
// waited for once; other waves' arithmetic hides that latency.  (Issuing the next
// segment's loads before the current one's arithmetic, in a wave that loops over
// items, needs about 100 more registers, halves the waves per CU, and measured
// slower; so did a fixed grid of 16 resident waves per CU looping over items, and,
// with seq_idx, items of 4 channels of a segment sharing its ids in registers.)
template <class S, int K, bool SILU, bool SEQ, bool ODD>
__global__ void __launch_bounds__(kBwdBlock) bwd_cf_reg_kernel(const BwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t i = (int64_t)blockIdx.x * (kBwdBlock / 64) + wave;
  if (i < a.items) reg_segment<S, K, SILU, SEQ, ODD>(a, reg_pos(a, i), lane);
}

__device__ inline void store_param(void* p, int dtype, int64_t i, float v) {
  if (dtype == CCV_DT_F32)
    static_cast<float*>(p)[i] = v;
  else if (dtype == CCV_DT_BF16)
    static_cast<uint16_t*>(p)[i] = BF16::from_f(v);
  else
    static_cast<uint16_t*>(p)[i] = F16::from_f(v);
}

// The in-order sum of rows q0 .. q1-1 of column s, from zero: a whole group's loads
// are all issued before the additions.
__device__ inline float sum_rows(const float* in, int64_t width, int64_t s, int64_t q0, int64_t q1) {
  float acc = 0.0f;
  if (q1 - q0 == kBwdFanIn) {
    float v[kBwdFanIn];
#pragma unroll
    for (int q = 0; q < kBwdFanIn; ++q) v[q] = in[(q0 + q) * width + s];
#pragma unroll
    for (int q = 0; q < kBwdFanIn; ++q) acc += v[q];
  } else {
    for (int64_t q = q0; q < q1; ++q) acc += in[q * width + s];
  }
  return acc;
}

__global__ void __launch_bounds__(kBwdBlock) bwd_reduce_kernel(const BwdReduceArgs r) {
  const int64_t width = (int64_t)(r.K + 1) * r.C;
  const int64_t id = (int64_t)blockIdx.x * kBwdBlock + threadIdx.x;
  const int64_t groups = (r.n_in + kBwdFanIn - 1) / kBwdFanIn;
  if (id >= groups * width) return;
  const int64_t g = id / width;
  const int64_t s = id - g * width;
  const int64_t q0 = g * kBwdFanIn;
  const int64_t q1 = q0 + kBwdFanIn < r.n_in ? q0 + kBwdFanIn : r.n_in;
  r.out[g * width + s] = sum_rows(r.in, width, s, q0, q1);
}

__global__ void __launch_bounds__(64 * kBwdFinalWaves) bwd_reduce_final_kernel(const BwdReduceArgs r) {
  __shared__ float sums[kBwdFinalWaves][64];
  const int64_t width = (int64_t)(r.K + 1) * r.C;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int64_t s = (int64_t)blockIdx.x * 64 + lane;
  float acc = 0.0f;                                // no rows (B = 0): zeros
  if (s < width) {
    const int64_t q0 = (int64_t)wv * kBwdFanIn;
    const int64_t q1 = q0 + kBwdFanIn < r.n_in ? q0 + kBwdFanIn : r.n_in;
    acc = sum_rows(r.in, width, s, q0, q1);
  }
  sums[wv][lane] = acc;
  __syncthreads();
  if (wv != 0 || s >= width) return;
  float tot = 0.0f;
  for (int w = 0; w < nw; ++w) tot += sums[w][lane];
  const int64_t slot = s / r.C;
  const int64_t c = s - slot * r.C;
  if (slot < r.K)
    store_param(r.dw, r.w_dtype, c * r.K + slot, tot);
  else if (r.db)
    store_param(r.db, r.w_dtype, c, tot);
}

template <class S, int K, bool SILU, bool SEQ>
int launch_one(const BwdArgs& a, int path, uint32_t grid, void* st) {
  void* args[] = {const_cast<BwdArgs*>(&a)};
  const void* fn;
  int block = 64;
  if (path == kBwdPathRegCf) {
    fn = reinterpret_cast<const void*>(&bwd_cf_reg_kernel<S, K, SILU, SEQ, false>);
    block = kBwdBlock;
  } else if (path == kBwdPathRegCfOdd) {
    fn = reinterpret_cast<const void*>(&bwd_cf_reg_kernel<S, K, SILU, SEQ, true>);
    block = kBwdBlock;
  } else if (path == kBwdPathLdsCf)
    fn = reinterpret_cast<const void*>(&bwd_lds_kernel<S, K, SILU, SEQ, false, false>);
  else if (path == kBwdPathLdsCl)
    fn = reinterpret_cast<const void*>(&bwd_lds_kernel<S, K, SILU, SEQ, true, false>);
  else if (path == kBwdPathLdsClOdd)
    fn = reinterpret_cast<const void*>(&bwd_lds_kernel<S, K, SILU, SEQ, true, true>);
  else {
    fn = reinterpret_cast<const void*>(&bwd_kernel<S, K, SILU, SEQ>);
    block = kBwdBlock;
  }
  return (int)hipLaunchKernel(fn, dim3(grid), dim3(block), args, 0, static_cast<hipStream_t>(st));
}

template <class S, int K>
int launch_k(const BwdArgs& a, bool silu, bool seq, int path, uint32_t grid, void* st) {
  if (silu)
    return seq ? launch_one<S, K, true, true>(a, path, grid, st) : launch_one<S, K, true, false>(a, path, grid, st);
  return seq ? launch_one<S, K, false, true>(a, path, grid, st) : launch_one<S, K, false, false>(a, path, grid, st);
}

template <class S>
int launch_s(const BwdArgs& a, int K, bool silu, bool seq, int path, uint32_t grid, void* st) {
  switch (K) {
    case 2: return launch_k<S, 2>(a, silu, seq, path, grid, st);
    case 3: return launch_k<S, 3>(a, silu, seq, path, grid, st);
    case 4: return launch_k<S, 4>(a, silu, seq, path, grid, st);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace

int bwd_tile_steps(int dtype) { return dtype == CCV_DT_F32 ? LdsGeom<F32>::T : LdsGeom<BF16>::T; }

int bwd_reg_span(int dtype) { return 64 * kBwdRegUnroll * (dtype == CCV_DT_F32 ? F32::V : BF16::V); }

int launch_bwd(const BwdArgs& a, int dtype, int K, bool silu, bool seq, int path, uint32_t grid,
               void* stream) {
  switch (dtype) {
    case CCV_DT_F32: return launch_s<F32>(a, K, silu, seq, path, grid, stream);
    case CCV_DT_F16: return launch_s<F16>(a, K, silu, seq, path, grid, stream);
    case CCV_DT_BF16: return launch_s<BF16>(a, K, silu, seq, path, grid, stream);
  }
  return (int)hipErrorInvalidValue;
}

int launch_bwd_reduce(const BwdReduceArgs& r, uint32_t grid, void* stream) {
  void* args[] = {const_cast<BwdReduceArgs*>(&r)};
  return (int)hipLaunchKernel(reinterpret_cast<const void*>(&bwd_reduce_kernel), dim3(grid), dim3(kBwdBlock),
                              args, 0, static_cast<hipStream_t>(stream));
}

int launch_bwd_reduce_final(const BwdReduceArgs& r, uint32_t grid, int waves, void* stream) {
  if (waves < 1 || waves > kBwdFinalWaves) return (int)hipErrorInvalidValue;
  void* args[] = {const_cast<BwdReduceArgs*>(&r)};
  return (int)hipLaunchKernel(reinterpret_cast<const void*>(&bwd_reduce_final_kernel), dim3(grid),
                              dim3(64 * waves), args, 0, static_cast<hipStream_t>(stream));
}

}  // namespace ccv
