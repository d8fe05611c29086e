// fastdiv.h -- division by a divisor fixed at launch time, for dividends
// 0 <= n < 2^31, by one high multiply, an add and a shift (the round-up
// method of T. Granlund and P. L. Montgomery, "Division by invariant integers
// using multiplication", PLDI 1994, section 4: with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, floor(n / d) = (mulhi(m, n) + n) >> l,
// the sum staying below 2^32 because mulhi(m, n) < n).  Plain C++: the host
// builds the constants, the kernels apply them with __umulhi.
#pragma once

#include <stdint.h>

namespace ra {

struct FastDiv {
  uint32_t d;   // the divisor, >= 1
  uint32_t m;   // multiplier
  uint32_t l;   // shift, ceil(log2 d)
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while (l < 32 && (uint64_t(1) << l) < d) ++l;
  const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1;
  return FastDiv{d, (uint32_t)m, l};
}

// floor(n / d) given hi = mulhi(m, n) (the top 32 bits of the 64-bit product)
inline uint32_t fastdiv_apply(const FastDiv& f, uint32_t hi, uint32_t n) { return (hi + n) >> f.l; }

}  // namespace ra
