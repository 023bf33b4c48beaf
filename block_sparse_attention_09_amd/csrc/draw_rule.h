// The keep decision of one SIP draw, shared by the sampler kernel and a host
// harness of the tests (the same code on both sides).
//
// Block j is kept iff its 53-bit uniform u = w0 * 2^21 + (w1 >> 11), made of
// its two Philox words, is below pi_j * 2^53.  With x = pi_j * 2^32 (exact:
// pi scaled by a power of two) and f = floor(min(x, 2^32 - 1)):
//   w0 < f  implies  u < (w0 + 1) * 2^21 <= f * 2^21 <= pi * 2^53  (kept);
//   w0 > f  implies  u >= (f + 1) * 2^21 > pi * 2^53                (dropped,
//           for pi < 1; pi = 1 gives f = 2^32 - 1 and no w0 above it).
// Only w0 == f (probability 2^-32) needs the 53-bit compare, which is exact in
// float64 (u < 2^53 and x * 2^21 are both representable).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace abatt {

__host__ __device__ inline bool sip_keep(uint32_t w0, uint32_t w1, double x) {
  const uint32_t f = x < 4294967295.0 ? (uint32_t)x : 0xffffffffu;
  bool keep = w0 < f;
  if (w0 == f) {
    const double u = (double)(((uint64_t)w0 << 21) | (w1 >> 11));
    keep = u < x * 2097152.0;
  }
  return keep;
}

}  // namespace abatt
