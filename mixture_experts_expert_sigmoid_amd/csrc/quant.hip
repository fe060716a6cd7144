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

// One wave per (row, 128-column group): each lane converts two columns.
__global__ __launch_bounds__(256) void quant_act_kernel(
    const uint32_t* __restrict__ x, long T, int H, uint16_t* __restrict__ xq,
    float* __restrict__ xs) {
  const int ng = H >> 7;
  const long gi = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gi >= T * ng) return;
  const int lane = lane_id();
  const long row = gi / ng;
  const int grp = (int)(gi - row * ng);
  const long off = row * H + grp * 128 + 2 * lane;     // element offset
  uint32_t v = x[off >> 1];
  float f0 = bf16_bits_to_f32(v & 0xFFFFu), f1 = bf16_bits_to_f32(v >> 16);
  float amax = wave_max(fmaxf(fabsf(f0), fabsf(f1)));
  float s = amax > 0.0f ? amax / 448.0f : 1.0f;
  uint32_t q0 = f32_to_e4m3(f0 / s), q1 = f32_to_e4m3(f1 / s);
  xq[off >> 1] = (uint16_t)(q0 | (q1 << 8));
  if (lane == 0) xs[row * ng + grp] = s;
}

hipError_t launch_quant_act(const void* x, long T, int H, void* xq, float* xs,
                            hipStream_t s) {
  long n = T * (long)(H / 128);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_act_kernel, dim3((unsigned)((n + 3) / 4)), dim3(256),
                     0, s, (const uint32_t*)x, T, H, (uint16_t*)xq, xs);
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
