// Philox4x64-10, the counter-based generator of J. K. Salmon, M. A. Moraes, R. O. Dror
// and D. E. Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11), section 4,
// with the 4x64 multipliers and Weyl key increments given there.  The block (words
// 0..3) at counter (c0, c1, c2, c3) under key (k0, k1).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace uep {

// 64 x 64 -> 128-bit product from four 32 x 32 + 64 multiply-adds (v_mad_u64_u32),
// sharing the partial products between the high and the low word.  No partial sum
// overflows: (2^32 - 1)^2 + (2^32 - 1) < 2^64.
__device__ __forceinline__ void mulhilo64(uint64_t a, uint64_t b, uint64_t& hi, uint64_t& lo) {
  const uint32_t a0 = (uint32_t)a, a1 = (uint32_t)(a >> 32);
  const uint32_t b0 = (uint32_t)b, b1 = (uint32_t)(b >> 32);
  const uint64_t p00 = (uint64_t)a0 * b0;
  const uint64_t p10 = (uint64_t)a1 * b0 + (p00 >> 32);
  const uint64_t p01 = (uint64_t)a0 * b1 + (uint32_t)p10;
  hi = (uint64_t)a1 * b1 + (p10 >> 32) + (p01 >> 32);
  lo = (p01 << 32) | (uint32_t)p00;
}

__device__ __forceinline__ void philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3,
                                              uint64_t k0, uint64_t k1, uint64_t (&w)[4]) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    uint64_t hi0, lo0, hi1, lo1;
    mulhilo64(M0, c0, hi0, lo0);
    mulhilo64(M1, c2, hi1, lo1);
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
    k0 += W0;
    k1 += W1;
  }
  w[0] = c0;
  w[1] = c1;
  w[2] = c2;
  w[3] = c3;
}

// word 0 alone (the last round's other product is dead code then)
__device__ __forceinline__ uint64_t philox4x64_10_w0(uint64_t c0, uint64_t c1, uint64_t c2,
                                                     uint64_t c3, uint64_t k0, uint64_t k1) {
  uint64_t w[4];
  philox4x64_10(c0, c1, c2, c3, k0, k1, w);
  return w[0];
}

}  // namespace uep
