// ccv_checks.hpp -- host-side argument checks shared by the forward, update and
// backward entry points: element sizes, offset overflow, alignment and
// self-overlap of strided views, and the target's CU count.  Host only, no HIP.
#pragma once

#include <stdint.h>
#include <stdlib.h>

#include <algorithm>

#include "ccv.h"

namespace ccv {
namespace checks {

inline int elt_size(int dt) { return dt == CCV_F32 ? 4 : 2; }

// Compute units to size a grid for: CCV_CU_COUNT when set to a positive count,
// else `device` (what the runtime reports for the call's GPU) when positive, else
// 256, MI355X's count.
inline int cu_count(int device) {
  const char* v = getenv("CCV_CU_COUNT");
  const int n = v && *v ? atoi(v) : 0;
  return n > 0 ? n : (device > 0 ? device : 256);
}

// Largest element offset of an [n0, n1, n2] view with strides s (all >= 0), or
// -1 when it does not fit in int64.
inline int64_t max_offset(const int64_t n[3], const int64_t s[3]) {
  int64_t total = 0;
  for (int d = 0; d < 3; ++d) {
    if (n[d] <= 1) continue;
    int64_t p;
    if (__builtin_mul_overflow(n[d] - 1, s[d], &p)) return -1;
    if (__builtin_add_overflow(total, p, &total)) return -1;
  }
  return total;
}

inline bool fits_bytes(int64_t max_off, int es) {
  int64_t bytes;
  return max_off >= 0 && !__builtin_mul_overflow(max_off + 1, (int64_t)es, &bytes);
}

// True when no two index triples of an [n0, n1, n2] view with strides s share an
// offset, shown by the usual sufficient test: taking the dimensions of extent > 1
// in ascending stride order, each stride exceeds the largest offset reachable
// with the dimensions before it.  (Call after max_offset succeeded, so the
// partial sums cannot overflow.)
inline bool non_overlapping(const int64_t n[3], const int64_t s[3]) {
  int order[3] = {0, 1, 2};
  std::sort(order, order + 3, [&](int p, int q) { return s[p] < s[q]; });
  int64_t reach = 0;
  for (int i = 0; i < 3; ++i) {
    const int d = order[i];
    if (n[d] <= 1) continue;
    if (s[d] <= reach) return false;
    reach += (n[d] - 1) * s[d];
  }
  return true;
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// The element stride of a dimension keeps 16-byte alignment (or is never used).
inline bool stride_ok16(int64_t n, int64_t s, int es) { return n <= 1 || ((s * es) & 15) == 0; }

}  // namespace checks
}  // namespace ccv
