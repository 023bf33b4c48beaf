// The keep decision of one SIP draw, shared by the sampler kernel and a host
// harness of the tests (the same code on both sides).
//
// Block j is kept iff its 32-bit uniform integer w (one Philox word) is below
// x = pi_j * 2^32.  Both sides of the compare are exact in float64: w < 2^32
// is an integer, and x is pi scaled by a power of two.  So the block enters
// with probability ceil(x) / 2^32: never for pi = 0, always for pi = 1, and
// within 2^-32 of pi in between.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace abatt {

__host__ __device__ inline bool sip_keep(uint32_t w, double x) {
  return (double)w < x;
}

}  // namespace abatt
