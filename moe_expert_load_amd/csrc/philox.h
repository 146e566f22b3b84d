// Philox4x64-10, the counter-based generator of J. K. Salmon, M. A. Moraes, R. O. Dror
// and D. E. Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11), section 4,
// with the 4x64 multipliers and Weyl key increments given there.  Word 0 of the block
// at counter (c0, c1, c2, c3) under key (k0, k1).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace uep {

__device__ __forceinline__ uint64_t philox4x64_10_w0(uint64_t c0, uint64_t c1, uint64_t c2,
                                                     uint64_t c3, uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const uint64_t hi0 = __umul64hi(M0, c0), lo0 = M0 * c0;
    const uint64_t hi1 = __umul64hi(M1, c2), lo1 = M1 * c2;
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
    k0 += W0;
    k1 += W1;
  }
  return c0;
}

}  // namespace uep
