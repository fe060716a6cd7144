// Routing-weighted combine of the per-pair fp32 expert outputs:
//   out[t][:] = sum over t's local slots j (ascending) of w[t][j] * y[row]
//             + shared_w * y[shared row of t]   (added last)
// in fp32 ("sm100: Fused INT4 grouped + SiLU Triton kernel", batchgen PR
// #239, commit text: slot-specific routing-weight reduction with fp32
// accumulation). A fixed slot order makes the result independent of which
// expert tile finished first. Each thread owns 4 consecutive columns.
#include "common.h"
#include "launch.h"

namespace moe {

__global__ __launch_bounds__(256) void combine_kernel(
    const float* __restrict__ y, long T, int H, int top_k, int shared,
    const int* __restrict__ pair_row, const float* __restrict__ topk_w,
    float shared_w, float* __restrict__ out) {
  const int cpr = H >> 2;                       // float4 columns per row
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= T * cpr) return;
  const long t = i / cpr;
  const int c4 = (int)(i - t * cpr);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < top_k; ++j) {
    int r = pair_row[t * top_k + j];
    if (r >= 0) {
      float wj = topk_w[t * top_k + j];
      f32x4 v = *(const f32x4*)(y + (long)r * H + 4 * c4);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = fmaf(wj, v[q], acc[q]);
    }
  }
  if (shared) {
    int r = pair_row[T * top_k + t];
    if (r >= 0) {
      f32x4 v = *(const f32x4*)(y + (long)r * H + 4 * c4);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = fmaf(shared_w, v[q], acc[q]);
    }
  }
  *(f32x4*)(out + t * H + 4 * c4) = acc;
}

hipError_t launch_combine(const float* y, long T, int H, int top_k, int shared,
                          const int* pair_row, const float* topk_w,
                          float shared_w, float* out, hipStream_t s) {
  long n = T * (long)(H / 4);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + 255) / 256)),
                     dim3(256), 0, s, y, T, H, top_k, shared, pair_row, topk_w,
                     shared_w, out);
  return hipGetLastError();
}

}  // namespace moe
