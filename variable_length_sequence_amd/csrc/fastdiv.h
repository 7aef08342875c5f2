// Division of 32-bit unsigned integers by a divisor fixed at launch time,
// done as a multiply-high and shifts (Granlund & Montgomery, "Division by
// Invariant Integers using Multiplication", 1994, Figure 4.1).  Used by the
// copy kernels to split a flat index into (chunk, offset) without the slow
// integer-division sequence.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define VL_HD __host__ __device__ __forceinline__
#else
#define VL_HD inline
#endif

namespace vl {

struct FastDiv {
  uint32_t d;  // divisor, >= 1
  uint32_t m;  // magic multiplier
  uint32_t l;  // ceil(log2(d))

  FastDiv() : d(1), m(0), l(0) {}
  explicit FastDiv(uint32_t div) : d(div) {
    l = 0;
    while ((uint64_t(1) << l) < div) ++l;
    // m = floor(2^32 * (2^l - d) / d) + 1
    m = uint32_t(((uint64_t(1) << 32) * ((uint64_t(1) << l) - div)) / div + 1);
  }

  VL_HD uint32_t div(uint32_t n) const {
    if (l == 0) return n;  // d == 1
    uint32_t t = uint32_t((uint64_t(m) * n) >> 32);
    return (t + ((n - t) >> 1)) >> (l - 1);
  }
};

}  // namespace vl
