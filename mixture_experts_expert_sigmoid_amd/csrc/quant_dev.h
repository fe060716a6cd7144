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
  const long row = wi / nc;
  const int col = (int)(wi - row * nc) * 512 + 8 * lane;
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
  uint32_t w[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = __builtin_amdgcn_fmed3f(f[4 * h + i] / sc, -448.0f, 448.0f);
    int c = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
    w[h] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], c, true);
  }
  if (on) {
    *(uint2*)(xq + row * H + col) = make_uint2(w[0], w[1]);
    if ((lane & 15) == 0) xs[row * (H >> 7) + (col >> 7)] = sc;
  }
}

}  // namespace moe
