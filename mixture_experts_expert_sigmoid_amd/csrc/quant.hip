// Per-token, per-128-column e4m3fn activation quantisation, and the LoRA
// down-projection z = x A^T of the rows of each local expert.
//
// Quantisation: the activation side of blockwise 128x128 FP8 ("[Moe] Fix
// flashinfer_trtllm silently dropping swiglu_limit clamped SwiGLU
// activation", sglang PR #39920, "Modifications": DeepSeekFp8): s = amax/448
// (s = 1 for an all-zero group), q = e4m3fn(round-to-nearest-even(x / s))
// with saturation, both divisions correctly rounded fp32.
//
// LoRA: the delta on gate/up must be in true units ("FlashInfer 0.6.18
// SM100a+SM103a MoE-LoRA AOT" release notes, "Changes since 1b699bf");
// z is kept in fp32 and consumed by the GEMM1 epilogue.
#include "common.h"
#include "launch.h"

namespace moe {

// One wave per (row, 512-column chunk): lane l converts the 8 columns
// chunk*512 + 8l .. +7 with one 16-byte load; the 16 lanes of a DPP row
// (lane / 16) hold one 128-column group, so the group amax is a row
// reduction in registers. The quotient x / s is a correctly rounded fp32
// division; it is clamped to +-448 and rounded to nearest-even e4m3fn by
// v_cvt_pk_fp8_f32 (identical to RNE with saturation for clamped inputs).
__global__ __launch_bounds__(256) void quant_act_kernel(
    const uint16_t* __restrict__ x, long T, int H, uint8_t* __restrict__ xq,
    float* __restrict__ xs) {
  const int nc = (H + 511) >> 9;
  const long wi = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wi >= T * nc) return;
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

hipError_t launch_quant_act(const void* x, long T, int H, void* xq, float* xs,
                            hipStream_t s) {
  long n = T * (long)((H + 511) / 512);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_act_kernel, dim3((unsigned)((n + 3) / 4)), dim3(256),
                     0, s, (const uint16_t*)x, T, H, (uint8_t*)xq, xs);
  return hipGetLastError();
}

// One wave per sorted row of a LoRA-carrying group.
template <int R>
__global__ __launch_bounds__(256) void lora_z_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ A, int rank,
    long T, int H, int top_k, int n_lora_groups, long p_cap,
    const int* __restrict__ offsets, const int* __restrict__ sorted_pair,
    float* __restrict__ z) {
  const long r = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = lane_id();
  if (r >= p_cap || r >= offsets[n_lora_groups]) return;
  // group of row r: largest g with offsets[g] <= r
  int lo = 0, hi = n_lora_groups - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (offsets[mid] <= r) lo = mid; else hi = mid - 1;
  }
  const int g = lo;
  const int p = sorted_pair[r];
  const long t = p / top_k;
  const uint16_t* xr = x + t * H;
  const uint16_t* Ag = A + (long)g * rank * H;
  float acc[R];
#pragma unroll
  for (int q = 0; q < R; ++q) acc[q] = 0.0f;
  for (int h0 = lane * 8; h0 < H; h0 += 512) {
    i32x4 xv = *(const i32x4*)(xr + h0);
    float xf[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xf[2 * i] = bf16_bits_to_f32((uint32_t)xv[i] & 0xFFFFu);
      xf[2 * i + 1] = bf16_bits_to_f32((uint32_t)xv[i] >> 16);
    }
#pragma unroll
    for (int q = 0; q < R; ++q) {
      if (q < rank) {
        i32x4 av = *(const i32x4*)(Ag + (long)q * H + h0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[q] += xf[2 * i] * bf16_bits_to_f32((uint32_t)av[i] & 0xFFFFu);
          acc[q] += xf[2 * i + 1] * bf16_bits_to_f32((uint32_t)av[i] >> 16);
        }
      }
    }
  }
#pragma unroll
  for (int q = 0; q < R; ++q) {
    if (q < rank) {
      float v = wave_sum(acc[q]);
      if (lane == 0) z[r * rank + q] = v;
    }
  }
}

hipError_t launch_lora_z(const void* x_bf16, const void* A, int rank, long T,
                         int H, int top_k, int n_lora_groups, long p_cap,
                         const int* offsets, const int* sorted_pair, float* z,
                         hipStream_t s) {
  if (p_cap == 0 || n_lora_groups == 0) return hipSuccess;
  dim3 grid((unsigned)((p_cap + 3) / 4)), block(256);
#define LZ(R)                                                                 \
  hipLaunchKernelGGL(lora_z_kernel<R>, grid, block, 0, s,                     \
                     (const uint16_t*)x_bf16, (const uint16_t*)A, rank, T, H, \
                     top_k, n_lora_groups, p_cap, offsets, sorted_pair, z)
  if (rank <= 8) LZ(8);
  else if (rank <= 16) LZ(16);
  else LZ(32);
#undef LZ
  return hipGetLastError();
}

}  // namespace moe
