// Shared host/device helpers of libcpattn: argument checks and fast division.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "cp_attn.h"

namespace cpattn {

// ---------------------------------------------------------------- host-side checks

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Half-open byte ranges [a, a+na) and [b, b+nb) intersect.
inline bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

inline bool layout_dtype_ok(int dtype) { return dtype == CP_DTYPE_BF16 || dtype == CP_DTYPE_FP16; }

// a * b with overflow detection against a cap; returns false on overflow.
inline bool mul_capped(int64_t a, int64_t b, int64_t cap, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > cap / a) return false;
  *out = a * b;
  return *out <= cap;
}

// Element counts of the layout kernels are indexed in 32-bit arithmetic over
// 16-byte vectors; 2^31 vectors (32 GiB) per launch is the supported extent.
constexpr int64_t kMaxVectors = (int64_t(1) << 31) - 1;

inline int hip_status(hipError_t e) { return e == hipSuccess ? CP_OK : CP_ERR_HIP; }

// Compute units of the current device (cached per device; 256 if unknown).
inline int num_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// ---------------------------------------------------------------- fast division
// Division of n < 2^31 by a runtime divisor d in [1, 2^31): q = (umulhi(n, m) + n) >> s
// with s = ceil(log2 d) and m = floor(2^32 * (2^s - d) / d) + 1 (Granlund and
// Montgomery, "Division by invariant integers using multiplication", 1994).
struct FastDiv {
  uint32_t d, m, s;
  FastDiv() : d(1), m(1), s(0) {}
  explicit FastDiv(uint32_t div) : d(div) {
    s = 0;
    while ((uint64_t(1) << s) < div) ++s;
    m = uint32_t(((uint64_t(1) << 32) * ((uint64_t(1) << s) - div)) / div + 1);
  }
  __device__ __forceinline__ uint32_t div(uint32_t n) const {
    return (__umulhi(n, m) + n) >> s;
  }
  __device__ __forceinline__ void divmod(uint32_t n, uint32_t& q, uint32_t& r) const {
    q = div(n);
    r = n - q * d;
  }
};

}  // namespace cpattn
