// Per-token, per-128-column e4m3fn activation quantisation, device part
// shared by quant.hip and front.hip. The activation side of blockwise
// 128x128 FP8 ("[Moe] Fix flashinfer_trtllm silently dropping swiglu_limit
// clamped SwiGLU activation", sglang PR #39920, "Modifications":
// DeepSeekFp8): s = amax/448 (s = 1 for an all-zero group), q =
// e4m3fn(round-to-nearest-even(x / s)) with saturation, both divisions
// correctly rounded fp32.
#pragma once
#include "common.h"

namespace moe {

// The unit index is the same for every lane of the wave: make it a scalar so
// that row = wi / nc is scalar arithmetic (32-bit whenever wi fits, as it
// does for any realistic batch) instead of a 64-bit division per lane.
__device__ __forceinline__ void unit_row_col(long wi, int nc, long& row, int& chunk) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)wi);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(wi >> 32));
  if (hi == 0) {
    const uint32_t r = lo / (uint32_t)nc;
    row = r;
    chunk = (int)(lo - r * (uint32_t)nc);
  } else {
    const long w = ((long)hi << 32) | lo;
    row = w / nc;
    chunk = (int)(w - row * nc);
  }
}

// One wave per (row, 512-column chunk): lane l converts the 8 columns
// chunk*512 + 8l .. +7 with one 16-byte load; the 16 lanes of a DPP row
// (lane / 16) hold one 128-column group, so the group amax is a row
// reduction in registers. The quotient x / s is a correctly rounded fp32
// division; it is clamped to +-448 and rounded to nearest-even e4m3fn by
// v_cvt_pk_fp8_f32 (identical to RNE with saturation for clamped inputs).
// Unit wi = row * ceil(H / 512) + chunk; all 64 lanes of the wave call it.
__device__ __forceinline__ void quant_act_unit(const uint16_t* __restrict__ x, long wi, int H,
                                               uint8_t* __restrict__ xq,
                                               float* __restrict__ xs) {
  const int nc = (H + 511) >> 9;
  const int lane = lane_id();
  long row;
  int chunk;
  unit_row_col(wi, nc, row, chunk);
  const int col = chunk * 512 + 8 * lane;
  const bool on = col < H;              // whole 16-lane rows (H % 128 == 0)
  float f[8];
  i32x4 v = {0, 0, 0, 0};
  if (on) v = *(const i32x4*)(x + row * H + col);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_bits_to_f32((uint32_t)v[i] & 0xFFFFu);
    f[2 * i + 1] = bf16_bits_to_f32((uint32_t)v[i] >> 16);
  }
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(f[i]));
  a = max16(a);
  const float sc = a > 0.0f ? a / 448.0f : 1.0f;
  // x / sc: with r = 1 / sc correctly rounded, q0 = x r, the residual
  // x - q0 sc (exact by FMA) and one correction q0 + (x - q0 sc) r give the
  // correctly rounded quotient whenever it is normal, and the same e4m3 code
  // always, for every bf16 x = 0 or |x| >= 2^-64 and sc >= 2^-64: checked
  // exhaustively over all bf16 amax / x pairs on the host. Other lanes
  // divide. Three operations per value instead of the division's ten.
  bool fast = sc >= 0x1p-64f;
#pragma unroll
  for (int i = 0; i < 8; ++i) fast = fast && (f[i] == 0.0f || fabsf(f[i]) >= 0x1p-64f);
  float qv[8];
  if (fast) {
    const float r = 1.0f / sc;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float q0 = __fmul_rn(f[i], r);
      qv[i] = __builtin_fmaf(__builtin_fmaf(-q0, sc, f[i]), r, q0);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) qv[i] = f[i] / sc;
  }
  uint32_t w[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = __builtin_amdgcn_fmed3f(qv[4 * h + i], -448.0f, 448.0f);
    int c = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
    w[h] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], c, true);
  }
  if (on) {
    *(uint2*)(xq + row * H + col) = make_uint2(w[0], w[1]);
    if ((lane & 15) == 0) xs[row * (H >> 7) + (col >> 7)] = sc;
  }
}

// MXFP8 activations for the GEMM1 of the MXFP4 W4A8 layers: per row and 32
// columns, amax (fp32, exact for bf16 inputs), e = the smallest integer
// with amax <= 448 * 2^e (raised to -127, e.g. for an all-zero group),
// stored as the e8m0 code e + 127, and codes = e4m3 RNE of x * 2^-e (an
// exact product of magnitude <= 448, so the conversion never saturates).
// With amax = m * 2^E (1 <= m < 2, biased exponent field B = E + 127):
// 448 = 1.75 * 2^8, so e = E - 8 when m <= 1.75 and E - 7 otherwise, i.e.
// e = B - 135 + (mantissa field > 0x600000). Same units as quant_act_unit:
// one wave per (row, 512 columns); the 4 lanes of a DPP quad hold one
// 32-column group.
__device__ __forceinline__ void quant_mx_unit(const uint16_t* __restrict__ x, long wi, int H,
                                              uint8_t* __restrict__ xq,
                                              uint8_t* __restrict__ xe) {
  const int nc = (H + 511) >> 9;
  const int lane = lane_id();
  long row;
  int chunk;
  unit_row_col(wi, nc, row, chunk);
  const int col = chunk * 512 + 8 * lane;
  const bool on = col < H;              // whole quads (H % 32 == 0)
  float f[8];
  i32x4 v = {0, 0, 0, 0};
  if (on) v = *(const i32x4*)(x + row * H + col);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_bits_to_f32((uint32_t)v[i] & 0xFFFFu);
    f[2 * i + 1] = bf16_bits_to_f32((uint32_t)v[i] >> 16);
  }
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(f[i]));
  a = fmaxf(a, __builtin_bit_cast(float, dpp_u32<0xB1>(__builtin_bit_cast(uint32_t, a))));
  a = fmaxf(a, __builtin_bit_cast(float, dpp_u32<0x4E>(__builtin_bit_cast(uint32_t, a))));
  const uint32_t ab = __builtin_bit_cast(uint32_t, a);
  int e = (int)(ab >> 23) - 135 + ((ab & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  e = max(e, -127);
  const float inv = __builtin_bit_cast(float, (uint32_t)(127 - e) << 23);   // 2^-e
  uint32_t w[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    int c = __builtin_amdgcn_cvt_pk_fp8_f32(f[4 * h] * inv, f[4 * h + 1] * inv, 0, false);
    w[h] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(f[4 * h + 2] * inv, f[4 * h + 3] * inv,
                                                     c, true);
  }
  if (on) {
    *(uint2*)(xq + row * H + col) = make_uint2(w[0], w[1]);
    if ((lane & 3) == 0) xe[row * (H >> 5) + (col >> 5)] = (uint8_t)(e + 127);
  }
}

}  // namespace moe
