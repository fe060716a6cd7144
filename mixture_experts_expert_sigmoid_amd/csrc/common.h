// Device helpers shared by the gfx950 kernels: vector types, bf16 / e4m3fn
// conversions and wave64 reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// err_word bits, equal to the public header's MOE_DEVERR_*: a routing id
// outside [0, num_experts_global); a 4-bit layer's bf16 activation (x or h)
// beyond the f16 range of its matrix-core operands; a 4-bit weight scale
// outside the range whose products expand exactly to f16.
#define MOE_DEVERR_BIT_OOB 0x1
#define MOE_DEVERR_BIT_F16_RANGE 0x2
#define MOE_DEVERR_BIT_W4_SCALE 0x4

namespace moe {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
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

// Cross-lane reductions in registers. Within a row of 16 lanes: DPP
// quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror, row_mirror (each lane
// meets every other lane of its row once). Across rows: gfx950's
// v_permlane16_swap / v_permlane32_swap exchange rows so that lane l meets
// l ^ 16 and l ^ 32. Every lane ends with the same result; the combination
// order is fixed, so sums are deterministic. (A __shfl_xor butterfly goes
// through LDS, one round trip per step.)
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}

template <typename T, typename Op>
__device__ __forceinline__ T row16_reduce(T v, Op op) {
  v = op(v, __builtin_bit_cast(T, dpp_u32<0xB1>(__builtin_bit_cast(uint32_t, v))));
  v = op(v, __builtin_bit_cast(T, dpp_u32<0x4E>(__builtin_bit_cast(uint32_t, v))));
  v = op(v, __builtin_bit_cast(T, dpp_u32<0x141>(__builtin_bit_cast(uint32_t, v))));
  v = op(v, __builtin_bit_cast(T, dpp_u32<0x140>(__builtin_bit_cast(uint32_t, v))));
  return v;
}

// op(v[l], v[l ^ 16]) and op(v[l], v[l ^ 32]), lower row first
template <typename T, typename Op>
__device__ __forceinline__ T xor16_reduce(T v, Op op) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return op(__builtin_bit_cast(T, (uint32_t)p[0]), __builtin_bit_cast(T, (uint32_t)p[1]));
}
template <typename T, typename Op>
__device__ __forceinline__ T xor32_reduce(T v, Op op) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return op(__builtin_bit_cast(T, (uint32_t)p[0]), __builtin_bit_cast(T, (uint32_t)p[1]));
}

template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T v, Op op) {
  return xor32_reduce(xor16_reduce(row16_reduce(v, op), op), op);
}

struct OpMax { __device__ float operator()(float a, float b) const { return fmaxf(a, b); } };
struct OpSum { __device__ float operator()(float a, float b) const { return a + b; } };
struct OpMinI { __device__ int operator()(int a, int b) const { return a < b ? a : b; } };

__device__ __forceinline__ float wave_max(float v) { return wave_reduce(v, OpMax{}); }
__device__ __forceinline__ float wave_sum(float v) { return wave_reduce(v, OpSum{}); }
__device__ __forceinline__ int wave_min_i32(int v) { return wave_reduce(v, OpMinI{}); }

// max over the 16 lanes that share lane / 16
__device__ __forceinline__ float max16(float v) { return row16_reduce(v, OpMax{}); }

// max over the 4 lanes that share lane % 16
__device__ __forceinline__ float max_across_rows(float v) {
  return xor32_reduce(xor16_reduce(v, OpMax{}), OpMax{});
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// fp32 sigmoid of an fp32 logit for ranking keys: evaluated in fp64 and
// rounded once to fp32 -- 1 / (1 + e) for x >= 0 and e / (1 + e) below,
// e = exp(-|x|) from the device library's double exp. Either form is
// within a few fp64 ulp of sigma(x), so the key is sigma(x) correctly
// rounded to fp32 unless sigma(x) lies within that distance of an fp32
// rounding midpoint; it saturates to exactly 1 and flushes to 0 where fp32
// does.
__device__ __forceinline__ float sigmoid_key(float x) {
  const double z = (double)x;
  const double e = exp(-fabs(z));
  return (float)(z >= 0.0 ? 1.0 / (1.0 + e) : e / (1.0 + e));
}

}  // namespace moe
