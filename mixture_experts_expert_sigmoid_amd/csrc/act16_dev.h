// bf16 -> f16 activation conversion in the K order of the 4-bit kernels'
// weight expansion (gemm_w4.h), shared with the decode front end
// (front.hip). Exact for |x| in [2^-14, 65504]; values beyond 65504 are
// reported through the error word.
#pragma once
#include "common.h"

namespace moe {

// 8 bf16 (k0..k7) -> 8 f16 in the order k0, k4, k1, k5, k2, k6, k3, k7
__device__ __forceinline__ f16x8 bf16x8_f16p(i32x4 v) {
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t u = (uint32_t)v[i];
    f[2 * i] = __uint_as_float(u << 16);
    f[2 * i + 1] = __uint_as_float(u & 0xFFFF0000u);
  }
  return (f16x8){(_Float16)f[0], (_Float16)f[4], (_Float16)f[1], (_Float16)f[5],
                 (_Float16)f[2], (_Float16)f[6], (_Float16)f[3], (_Float16)f[7]};
}

// true if one of the 8 bf16 values has |v| > 65504 (f16 would make it
// infinite: the next bf16 magnitude above 65280 is 65536) or is not finite
__device__ __forceinline__ bool bf16x8_f16_overflow(i32x4 v) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t u = (uint32_t)v[i];
    m = max(m, max(u & 0x7FFFu, (u >> 16) & 0x7FFFu));
  }
  return m >= 0x4780u;
}

}  // namespace moe
