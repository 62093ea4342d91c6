// ccv_device.hpp -- device-side helpers shared by the two forward kernels:
// storage types, fp32 <-> storage conversion, SiLU, lane shifts, and the
// XCD-aware workgroup order.  gfx950 (CDNA4, wave64) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ccv_launch.hpp"

namespace ccv {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Element i of a 16-byte vector as a plain 32-bit value.  Never apply
// __builtin_bit_cast to a vector subscript directly: clang reads element 0 for
// every i when the operand is a vector-element lvalue.
__device__ inline uint32_t dword(const u32x4 v, int i) {
  const uint32_t w = v[i];
  return w;
}

// The fp32 value itself, materialised in a register.  Before a down-convert this
// keeps the compiler from fusing the last multiply (or FMA) with the conversion
// into one mixed-precision instruction (v_fma_mixlo_*), which rounds the exact
// product once to 16 bits instead of rounding it to fp32 first; the two differ in
// about one output in 2^14, so fused and unfused code paths would disagree.
// The empty asm statement emits no instruction.
__device__ inline float as_f32(float v) {
  asm("" : "+v"(v));
  return v;
}

// ---- storage types: V elements fill one 16-byte vector ---------------------------

struct F32 {
  using raw = uint32_t;
  static constexpr int V = 4;
  __device__ static inline float to_f(raw r) { return __builtin_bit_cast(float, r); }
  __device__ static inline void unpack(const u32x4 v, float* e) {
#pragma unroll
    for (int i = 0; i < 4; ++i) e[i] = __builtin_bit_cast(float, dword(v, i));
  }
  __device__ static inline u32x4 pack(const float* y) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __builtin_bit_cast(uint32_t, y[i]);
    return v;
  }
  __device__ static inline raw from_f(float y) { return __builtin_bit_cast(uint32_t, y); }
};

// bfloat16: the upper half of a binary32.  Widening is a shift; narrowing uses the
// gfx950 packed convert (round to nearest even, NaN stays NaN).
struct BF16 {
  using raw = uint16_t;
  static constexpr int V = 8;
  __device__ static inline float to_f(raw r) { return __builtin_bit_cast(float, (uint32_t)r << 16); }
  __device__ static inline void unpack(const u32x4 v, float* e) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = dword(v, i);
      e[2 * i] = __builtin_bit_cast(float, w << 16);
      e[2 * i + 1] = __builtin_bit_cast(float, w & 0xffff0000u);
    }
  }
  __device__ static inline u32x4 pack(const float* y) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x2 p = {as_f32(y[2 * i]), as_f32(y[2 * i + 1])};
      v[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2));
    }
    return v;
  }
  __device__ static inline raw from_f(float y) {
    return __builtin_bit_cast(uint16_t, (__bf16)as_f32(y));
  }
};

// IEEE binary16: hardware converts both ways (round to nearest even).
struct F16 {
  using raw = uint16_t;
  static constexpr int V = 8;
  __device__ static inline float to_f(raw r) { return (float)__builtin_bit_cast(_Float16, r); }
  __device__ static inline void unpack(const u32x4 v, float* e) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x2 p = __builtin_convertvector(__builtin_bit_cast(f16x2, dword(v, i)), f32x2);
      e[2 * i] = p[0];
      e[2 * i + 1] = p[1];
    }
  }
  __device__ static inline u32x4 pack(const float* y) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x2 p = {as_f32(y[2 * i]), as_f32(y[2 * i + 1])};
      v[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(p, f16x2));
    }
    return v;
  }
  __device__ static inline raw from_f(float y) { return __builtin_bit_cast(uint16_t, (_Float16)as_f32(y)); }
};

// Weight / bias element of any storage dtype, widened exactly to fp32.
__device__ inline float load_param(const void* p, int dtype, int64_t i) {
  if (dtype == CCV_DT_F32) return static_cast<const float*>(p)[i];
  const uint16_t h = static_cast<const uint16_t*>(p)[i];
  if (dtype == CCV_DT_BF16) return __builtin_bit_cast(float, (uint32_t)h << 16);
  return (float)__builtin_bit_cast(_Float16, h);
}

// n consecutive parameters starting at element i0, widened to fp32.  One branch
// on the dtype, then n independent loads, so they are in flight together.
template <int N>
__device__ inline void load_params(const void* p, int dtype, int64_t i0, float* out) {
  if (dtype == CCV_DT_F32) {
    const float* q = static_cast<const float*>(p) + i0;
#pragma unroll
    for (int k = 0; k < N; ++k) out[k] = q[k];
  } else {
    const uint16_t* q = static_cast<const uint16_t*>(p) + i0;
    uint16_t h[N];
#pragma unroll
    for (int k = 0; k < N; ++k) h[k] = q[k];
#pragma unroll
    for (int k = 0; k < N; ++k)
      out[k] = dtype == CCV_DT_BF16 ? __builtin_bit_cast(float, (uint32_t)h[k] << 16)
                                    : (float)__builtin_bit_cast(_Float16, h[k]);
  }
}

// SiLU on the fp32 accumulator: z * 1 / (1 + 2^(-z * log2(e))), with the hardware
// base-2 exponential and reciprocal (about 1 ulp each).  IEEE edge cases fall out:
// silu(+inf) = +inf, silu(-inf) = NaN (as z * sigmoid(z) evaluates), NaN -> NaN.
__device__ inline float silu(float z) {
  const float e = __builtin_amdgcn_exp2f(z * -1.44269504088896341f);
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

// Lane l receives lane l-1's value; lane 0 receives `carry`.  DPP wave_shr:1
// (whole-wave shift right by one lane); every lane of the wave must be active.
__device__ inline float shift_in(float carry, float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      __builtin_bit_cast(int, carry), __builtin_bit_cast(int, v), 0x138, 0xf, 0xf, false));
}
__device__ inline int shift_in(int carry, int v) {
  return __builtin_amdgcn_update_dpp(carry, v, 0x138, 0xf, 0xf, false);
}
__device__ inline float lane63(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ inline int lane63(int v) { return __builtin_amdgcn_readlane(v, 63); }

// Workgroups are dealt round-robin to the 8 XCDs (workgroup g runs on XCD g % 8).
// Renumber them so that each XCD owns one contiguous range of work: neighbouring
// work items (which re-read each other's K-1 halo) then share that XCD's L2.
// With G workgroups, q = G / 8 and r = G % 8, XCD x holds q + (x < r) of them.
__device__ inline uint32_t xcd_order(uint32_t g, uint32_t q, uint32_t r) {
  const uint32_t x = g & 7u, s = g >> 3;
  return x * q + (x < r ? x : r) + s;
}

// With seq_idx, final_states are the history of the row's last sequence: the
// entry from extended position j survives when its sequence id (seq_idx[b, j], or
// seq_idx[b, 0] for the history left of t = 0) is the id at t = L-1.  seq_row is
// the row of seq_idx, or nullptr.
__device__ inline bool final_kept(const int32_t* seq_row, int64_t L, int64_t j, bool has_init) {
  if (!seq_row || L == 0) return true;
  if (j < 0 && !has_init) return false;            // the zero history
  return seq_row[j >= 0 ? j : 0] == seq_row[L - 1];
}

__device__ inline u32x4 load16(const void* p) { return *static_cast<const u32x4*>(p); }
__device__ inline void store16(void* p, u32x4 v) { *static_cast<u32x4*>(p) = v; }

// Streaming (non-temporal) 16-byte accesses for data touched once: x and out.
__device__ inline u32x4 load16_stream(const void* p) {
  return __builtin_nontemporal_load(static_cast<const u32x4*>(p));
}
__device__ inline void store16_stream(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, static_cast<u32x4*>(p));
}

// Zeros to load from where an operand is absent (no bias, history left of t = 0
// without initial_states), so that every load is unconditional.  2 KB: a wave
// whose lanes add their own offset (up to 64 lanes x 32 bytes) stays inside it.
static __device__ const uint32_t kZeroSrc[512] = {};

// Loads through global-address-space pointers made from integer addresses, and a
// select of addresses without a branch: the prefetch below stays one straight
// sequence of global loads.
template <class T>
__device__ inline T gload(uintptr_t addr) {
  return *reinterpret_cast<const T __attribute__((address_space(1)))*>(addr);
}
__device__ inline u32x4 gload16_stream(uintptr_t addr) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 __attribute__((address_space(1)))*>(addr));
}
__device__ inline void gstore16_stream(uintptr_t addr, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4 __attribute__((address_space(1)))*>(addr));
}
__device__ inline uintptr_t pick(bool c, uintptr_t a, uintptr_t b) {
  const uintptr_t mask = (uintptr_t)0 - (uintptr_t)c;
  return (a & mask) | (b & ~mask);
}

// Raw weight / bias element: WB == 4 for fp32 parameters, 2 for bf16 / fp16.
template <int WB>
__device__ inline uint32_t load_param_raw(uintptr_t addr) {
  if constexpr (WB == 4) return gload<uint32_t>(addr);
  else return gload<uint16_t>(addr);
}

// A lane's block of NB bytes of consecutive parameters (its V channels' weights or
// biases), as dwords: 16-byte loads when NB is a multiple of 16 (the block then
// starts 16-byte aligned), else 8-byte loads (fp32 data with 16-bit parameters:
// blocks of 8 or 24 bytes, starting 8-byte aligned).
template <int NB>
__device__ inline void load_param_block(uintptr_t p, uint32_t (&d)[NB / 4]) {
  static_assert(NB % 8 == 0, "parameter blocks are whole 8-byte units");
  if constexpr (NB % 16 == 0) {
#pragma unroll
    for (int i = 0; i < NB / 16; ++i) {
      const u32x4 v = gload<u32x4>(p + 16 * i);
#pragma unroll
      for (int j = 0; j < 4; ++j) d[4 * i + j] = dword(v, j);
    }
  } else {
#pragma unroll
    for (int i = 0; i < NB / 8; ++i) {
      const u32x2 v = gload<u32x2>(p + 8 * i);
      d[2 * i] = v[0];
      d[2 * i + 1] = v[1];
    }
  }
}

// Raw parameter e of a block loaded by load_param_block (WB bytes each).
template <int WB, int ND>
__device__ inline uint32_t block_param_raw(const uint32_t (&d)[ND], int e) {
  if constexpr (WB == 4) return d[e];
  else return (d[e / 2] >> (16 * (e % 2))) & 0xffffu;
}

template <int WB>
__device__ inline float param_f32(uint32_t r, int dtype) {
  if constexpr (WB == 4) {
    return __builtin_bit_cast(float, r);
  } else {
    const float bf = __builtin_bit_cast(float, r << 16);
    const float hf = (float)__builtin_bit_cast(_Float16, (uint16_t)r);
    return dtype == CCV_DT_BF16 ? bf : hf;
  }
}

}  // namespace ccv
