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

// The same combine over GEMM2's block-floating-point rows (FP8 and 4-bit
// layers): y16 [p_rows][H] int16 and ye [p_rows][H / 16], value = y16 *
// 2^ye (exact in fp32; -32768 stands for a value that was not finite and
// reads as NaN), then the same fp32 multiply-adds in the same order. Each
// thread owns 8 consecutive columns, one scale exponent.
__global__ __launch_bounds__(256) void combine16_kernel(
    const uint16_t* __restrict__ y16, const int8_t* __restrict__ ye, long T, int H,
    int top_k, int shared, const int* __restrict__ pair_row,
    const float* __restrict__ topk_w, float shared_w, float* __restrict__ out) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const int cpr = H >> 3;                       // 8-column runs per row
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= T * cpr) return;
  long t = i / cpr;
  const int c8 = (int)(i - t * cpr);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // kPairs pairs at a time (ascending slot, the shared pair last): their
  // rows and weights are loaded together, then their y runs, then they are
  // accumulated in pair order
  constexpr int kPairs = 8;
  const int np = top_k + shared;
  if ((cpr & 63) == 0 && T * top_k + T < (1L << 31)) {
    // a wave never straddles two tokens: the token, its pair rows and
    // weights are wave-uniform (scalar loads); the y loads stay branch-free
    // (a pair with no local row reads row 0, its value unused). Loading only
    // the local pairs' rows (a branch per pair) helped the expert-parallel
    // share at T = 8192 but cost 1.5-2 us per call at decode sizes.
    t = (long)__builtin_amdgcn_readfirstlane((int)t);
    for (int j0 = 0; j0 < np; j0 += kPairs) {
      int r[kPairs];
      float w[kPairs];
#pragma unroll
      for (int u = 0; u < kPairs; ++u) {
        const int j = min(j0 + u, np - 1);
        const int jr = (int)(j < top_k ? t * top_k + j : T * top_k + t);
        r[u] = j0 + u < np ? pair_row[jr] : -1;
        const float wl = topk_w[t * top_k + min(j, top_k - 1)];
        w[u] = j < top_k ? wl : shared_w;
      }
      i16x8 v[kPairs];
      int e[kPairs];
#pragma unroll
      for (int u = 0; u < kPairs; ++u) {
        const long rr = max(r[u], 0);
        v[u] = *(const i16x8*)(y16 + rr * H + 8 * c8);
        e[u] = ye[rr * (H >> 4) + (c8 >> 1)];
      }
#pragma unroll
      for (int u = 0; u < kPairs; ++u)
        if (r[u] >= 0) {
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const float yv = v[u][q] == -32768 ? __builtin_nanf("")
                                               : __builtin_amdgcn_ldexpf((float)v[u][q], e[u]);
            acc[q] = fmaf(w[u], yv, acc[q]);
          }
        }
    }
    float* o = out + t * H + 8 * c8;
    *(f32x4*)o = (f32x4){acc[0], acc[1], acc[2], acc[3]};
    *(f32x4*)(o + 4) = (f32x4){acc[4], acc[5], acc[6], acc[7]};
    return;
  }
  for (int j0 = 0; j0 < np; j0 += kPairs) {
    int r[kPairs];
    float w[kPairs];
#pragma unroll
    for (int u = 0; u < kPairs; ++u) {
      const int j = min(j0 + u, np - 1);
      const long jr = j < top_k ? t * top_k + j : T * top_k + t;
      r[u] = pair_row[jr];
      const float wl = topk_w[t * top_k + min(j, top_k - 1)];
      w[u] = j < top_k ? wl : shared_w;
    }
    i16x8 v[kPairs];
    int e[kPairs];
    // a pair without a local row reads row 0 instead (the launch has
    // p_rows >= 1; the value is not used), so no load waits on a branch
#pragma unroll
    for (int u = 0; u < kPairs; ++u) {
      const long rr = max(r[u], 0);
      v[u] = *(const i16x8*)(y16 + rr * H + 8 * c8);
      e[u] = ye[rr * (H >> 4) + (c8 >> 1)];
    }
#pragma unroll
    for (int u = 0; u < kPairs; ++u)
      if (j0 + u < np && r[u] >= 0) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float yv = v[u][q] == -32768 ? __builtin_nanf("")
                                             : __builtin_amdgcn_ldexpf((float)v[u][q], e[u]);
          acc[q] = fmaf(w[u], yv, acc[q]);
        }
      }
  }
  float* o = out + t * H + 8 * c8;
  *(f32x4*)o = (f32x4){acc[0], acc[1], acc[2], acc[3]};
  *(f32x4*)(o + 4) = (f32x4){acc[4], acc[5], acc[6], acc[7]};
}

// The same combine over the partial sums of the FP8 / 4-bit GEMM2's split-K
// kernel (slots [kSkSlots][p_rows][H]): each y element is first summed over
// the slots of its tile in slot order. The tile schedule is rebuilt exactly as
// the GEMM built it (32-row tiles, 256-column tiles, I / 128 K blocks). One
// workgroup per (token, 2048 columns); its token's pairs are looked up once.
constexpr int kCsCols = 2048;
constexpr int kCsPairs = 4;
__global__ __launch_bounds__(512) void combine_sk_kernel(
    const float* __restrict__ part, long T, int H, int top_k, int shared,
    const int* __restrict__ pair_row, const float* __restrict__ topk_w,
    float shared_w, float* __restrict__ out, int grid, long p_rows, int I, int G,
    const int* __restrict__ offsets, int mode) {
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
  // SK_DEVICE: the GEMM kernels chose split-K or plain rows by the same rule
  // on the same tile count; plain rows are slot 0 of the partial layout
  const bool split = mode != SK_DEVICE || sk_rule((long)s_cum[G] * NT, NS);
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
  // pairs kCsPairs at a time (ascending slot, shared last): the partial
  // slots of all of them are loaded first, then summed per pair in slot
  // order and accumulated in pair order
  for (int j0 = 0; j0 < np; j0 += kCsPairs) {
    int nsl[kCsPairs];
    f32x4 p[kCsPairs][kSkSlots];
#pragma unroll
    for (int u = 0; u < kCsPairs; ++u) {
      const int j = j0 + u;
      const int r = j < np ? s_row[j] : -1;
      nsl[u] = r < 0 ? 0
                     : split ? sk_nslots(((long)s_mt[j] * NT + nt) * NS, NS, U, W) : 1;
#pragma unroll
      for (int sl = 0; sl < kSkSlots; ++sl)
        if (sl < nsl[u]) p[u][sl] = *(const f32x4*)(part + ((long)sl * p_rows + r) * H + col);
    }
#pragma unroll
    for (int u = 0; u < kCsPairs; ++u) {
      if (nsl[u] == 0) continue;
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int sl = 0; sl < kSkSlots; ++sl)
        if (sl < nsl[u]) {
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] += p[u][sl][q];
        }
      const float wj = s_w[j0 + u];
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = fmaf(wj, v[q], acc[q]);
    }
  }
  *(f32x4*)(out + t * H + col) = acc;
}

hipError_t launch_combine(const float* y, long T, int H, int top_k, int shared,
                          const int* pair_row, const float* topk_w,
                          float shared_w, float* out, hipStream_t s, int sk_grid,
                          long p_cap, int I, int G, const int* offsets, int sk_mode,
                          bool y16) {
  long n = T * (long)(H / 4);
  if (n == 0) return hipSuccess;
  if (sk_grid == 0 && y16 && p_cap > 0) {   // (p_cap == 0: no rows, out = 0 below)
    const uint16_t* yh = (const uint16_t*)y;
    const int8_t* ye = (const int8_t*)(yh + p_cap * H);
    const long n8 = T * (long)(H / 8);
    hipLaunchKernelGGL(combine16_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s,
                       yh, ye, T, H, top_k, shared, pair_row, topk_w, shared_w, out);
    return hipGetLastError();
  }
  if (sk_grid > 0) {
    const long nwg = T * ((H + kCsCols - 1) / kCsCols);
    hipLaunchKernelGGL(combine_sk_kernel, dim3((unsigned)nwg), dim3(512), 0, s, y, T, H,
                       top_k, shared, pair_row, topk_w, shared_w, out, sk_grid, p_cap,
                       I, G, offsets, sk_mode);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + 255) / 256)),
                     dim3(256), 0, s, y, T, H, top_k, shared, pair_row, topk_w,
                     shared_w, out);
  return hipGetLastError();
}

}  // namespace moe
