// Routing-weighted combine of the per-pair fp32 expert outputs:
//   out[t][:] = sum over t's local slots j (ascending) of w[t][j] * y[row]
//             + shared_w * y[shared row of t]   (added last)
// in fp32 ("sm100: Fused INT4 grouped + SiLU Triton kernel", batchgen PR
// #239, commit text: slot-specific routing-weight reduction with fp32
// accumulation). A fixed slot order makes the result independent of which
// expert tile finished first. Each thread owns 4 consecutive columns.
#include "gemm_common.h"

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

// The same combine over the partial sums of the FP8 / 4-bit GEMM2's split-K
// kernel (slots [kSkSlots][p_rows][H]): each y element is first summed over
// the slots of its tile in slot order. The tile schedule is rebuilt exactly as
// the GEMM built it (32-row tiles, 256-column tiles, I / 128 K blocks). One
// workgroup per (token, 2048 columns); its token's pairs are looked up once.
constexpr int kCsCols = 2048;
__global__ __launch_bounds__(512) void combine_sk_kernel(
    const float* __restrict__ part, long T, int H, int top_k, int shared,
    const int* __restrict__ pair_row, const float* __restrict__ topk_w,
    float shared_w, float* __restrict__ out, int grid, long p_rows, int I, int G,
    const int* __restrict__ offsets) {
  __shared__ int s_cum[kMaxGroups + 1];
  __shared__ int s_off[kMaxGroups + 1];
  __shared__ int s_wsum[8];
  __shared__ int s_row[65], s_mt[65];
  __shared__ float s_w[65];
  const int NT = (H + 255) >> 8, NS = I >> 7;
  tile_prefix<kSkBM>(offsets, G, s_cum, s_wsum);
  for (int i = threadIdx.x; i <= G; i += 512) s_off[i] = offsets[i];
  const long U = (long)s_cum[G] * NT * NS;
  const int W = sk_workgroups((long)s_cum[G] * NT, NS, grid);
  const int chunks = (H + kCsCols - 1) / kCsCols;
  const long t = blockIdx.x / chunks;
  const int col0 = (int)(blockIdx.x - t * chunks) * kCsCols;
  const int np = top_k + shared;               // slots j, then the shared pair
  __syncthreads();
  if ((int)threadIdx.x < np) {
    const int j = threadIdx.x;
    const int r = j < top_k ? pair_row[t * top_k + j] : pair_row[T * top_k + t];
    s_row[j] = r;
    s_w[j] = j < top_k ? topk_w[t * top_k + j] : shared_w;
    int mt = 0;
    if (r >= 0) {
      const int g = group_of_row(s_off, G, r);
      mt = s_cum[g] + (r - s_off[g]) / kSkBM;
    }
    s_mt[j] = mt;
  }
  __syncthreads();
  const int col = col0 + 4 * threadIdx.x;
  if (col >= H) return;
  const int nt = col >> 8;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < np; ++j) {               // ascending slot, shared last
    const int r = s_row[j];
    if (r < 0) continue;
    const int nsl = sk_nslots(((long)s_mt[j] * NT + nt) * NS, NS, U, W);
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    for (int sl = 0; sl < nsl; ++sl) {
      const f32x4 p = *(const f32x4*)(part + ((long)sl * p_rows + r) * H + col);
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] += p[q];
    }
    const float wj = s_w[j];
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = fmaf(wj, v[q], acc[q]);
  }
  *(f32x4*)(out + t * H + col) = acc;
}

hipError_t launch_combine(const float* y, long T, int H, int top_k, int shared,
                          const int* pair_row, const float* topk_w,
                          float shared_w, float* out, hipStream_t s, int sk_grid,
                          long p_cap, int I, int G, const int* offsets) {
  long n = T * (long)(H / 4);
  if (n == 0) return hipSuccess;
  if (sk_grid > 0) {
    const long nwg = T * ((H + kCsCols - 1) / kCsCols);
    hipLaunchKernelGGL(combine_sk_kernel, dim3((unsigned)nwg), dim3(512), 0, s, y, T, H,
                       top_k, shared, pair_row, topk_w, shared_w, out, sk_grid, p_cap,
                       I, G, offsets);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + 255) / 256)),
                     dim3(256), 0, s, y, T, H, top_k, shared, pair_row, topk_w,
                     shared_w, out);
  return hipGetLastError();
}

}  // namespace moe
