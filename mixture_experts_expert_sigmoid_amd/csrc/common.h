// Device helpers shared by the gfx950 kernels: vector types, bf16 / e4m3fn
// conversions and wave64 reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// err_word bit for a routing id outside [0, num_experts_global); equal to
// MOE_DEVERR_GLOBAL_ID_OOB of the public header.
#define MOE_DEVERR_BIT_OOB 0x1

namespace moe {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// fp32 -> OCP e4m3fn code, round to nearest even, magnitudes >= 448
// saturated to +-448, NaN -> 0x7F.
__device__ __forceinline__ uint32_t f32_to_e4m3(float f) {
  uint32_t u = __float_as_uint(f);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return 0x7Fu;
  if (a >= 0x43E00000u) return sign | 0x7Eu;        // |f| >= 448
  if (a < 0x3C800000u) {                            // |f| < 2^-6: subnormal
    // multiples of 2^-9; rint is round-half-even; 8 -> first normal code
    float m = __builtin_rintf(__uint_as_float(a) * 512.0f);
    return sign | (uint32_t)m;
  }
  // normal: keep 3 mantissa bits, round the remaining 20 to nearest even
  uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
  return sign | ((r >> 20) - (120u << 3));          // rebias 127 -> 7
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// max over the 16 lanes that share lane / 16 (xor over lane bits 0..3)
__device__ __forceinline__ float max16(float v) {
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

}  // namespace moe
