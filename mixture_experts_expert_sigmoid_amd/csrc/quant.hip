// Per-token, per-128-column e4m3fn activation quantisation (and the MXFP8
// variant of the MXFP4 W4A8 layers, quant_dev.h), and the LoRA
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
#include <algorithm>

#include "launch.h"
#include "quant_dev.h"

namespace moe {

__global__ __launch_bounds__(256) void quant_act_kernel(
    const uint16_t* __restrict__ x, long T, int H, uint8_t* __restrict__ xq,
    float* __restrict__ xs) {
  const int nc = (H + 511) >> 9;
  const long wi = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wi >= T * nc) return;
  quant_act_unit(x, wi, H, xq, xs);
}

hipError_t launch_quant_act(const void* x, long T, int H, void* xq, float* xs,
                            hipStream_t s) {
  long n = T * (long)((H + 511) / 512);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_act_kernel, dim3((unsigned)((n + 3) / 4)), dim3(256),
                     0, s, (const uint16_t*)x, T, H, (uint8_t*)xq, xs);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void quant_act_mx_kernel(
    const uint16_t* __restrict__ x, long T, int H, uint8_t* __restrict__ xq,
    uint8_t* __restrict__ xe) {
  const int nc = (H + 511) >> 9;
  const long wi = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wi >= T * nc) return;
  quant_mx_unit(x, wi, H, xq, xe);
}

hipError_t launch_quant_act_mx(const void* x, long T, int H, void* xq, void* xe,
                               hipStream_t s) {
  long n = T * (long)((H + 511) / 512);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_act_mx_kernel, dim3((unsigned)((n + 3) / 4)), dim3(256),
                     0, s, (const uint16_t*)x, T, H, (uint8_t*)xq, (uint8_t*)xe);
  return hipGetLastError();
}

// Exclusive prefix over the first G groups of ceil(rows_g / 16) into
// s_cum[0..G] (256 threads, G <= 1024: four groups per thread).
__device__ __forceinline__ void lora_tile_prefix(const int* offsets, int G, int* s_cum,
                                                 int* s_wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int c[4], v = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = 4 * tid + i;
    c[i] = g < G ? (offsets[g + 1] - offsets[g] + 15) >> 4 : 0;
    v += c[i];
  }
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  int run = incl - v;
  for (int w = 0; w < wave; ++w) run += s_wsum[w];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = 4 * tid + i;
    if (g < G) s_cum[g] = run;
    run += c[i];
  }
  if (tid == 0) s_cum[G] = s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3];
  __syncthreads();
}

// token of pair p: p / top_k for the routed pairs p < T top_k, p - T top_k
// for the shared expert's rows
__device__ __forceinline__ long pair_token(long p, long T, int top_k) {
  const long npr = T * top_k;
  return p < npr ? p / top_k : p - npr;
}

// The K loop of one 16-row block: acc[n] = x rows . A rows 16 n .. 16 n + 15
// over this wave's quarter of H on v_mfma_f32_16x16x32_bf16 (x the first
// operand), 8 K steps per round with all their loads issued before the
// MFMAs. xr / Ag: the lane's row and rank-row pointers at the quarter's
// start + 8 (lane / 16).
template <int NQ>
__device__ __forceinline__ void lora_z_rows(const uint16_t* xr, const uint16_t* Ag, int rank,
                                            int H, f32x4 (&acc)[NQ]) {
  const int lr = lane_id() & 15;
  const int hq = H >> 2;
#pragma unroll
  for (int n = 0; n < NQ; ++n) acc[n] = (f32x4){0.f, 0.f, 0.f, 0.f};
  for (int h0 = 0; h0 < hq; h0 += 256) {
    i32x4 xv[8], av[NQ][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int h = min(h0 + 32 * j, hq - 32);   // hq % 32 == 0
      xv[j] = *(const i32x4*)(xr + h);
#pragma unroll
      for (int n = 0; n < NQ; ++n) {
        const int q = 16 * n + lr;
        av[n][j] = (i32x4){0, 0, 0, 0};
        if (q < rank) av[n][j] = *(const i32x4*)(Ag + (long)q * H + h);
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (h0 + 32 * j >= hq) break;
#pragma unroll
      for (int n = 0; n < NQ; ++n)
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xv[j]),
                                                        __builtin_bit_cast(bf16x8, av[n][j]),
                                                        acc[n], 0, 0, 0);
    }
  }
}

// One workgroup (4 waves) per 16-row tile of one expert's sorted rows (tile
// t of expert g covers rows offsets[g] + 16 (t - s_cum[g]) ..):
// z[16 rows][16 ranks] = X A_g^T on v_mfma_f32_16x16x32_bf16 (bf16
// products, fp32 accumulation), A_g read once per tile instead of once per
// row. Wave w covers the w-th quarter of H; the four partials are added in
// wave order through LDS. (One adapter for every row.)
template <int NQ>    // 16-column blocks covering the rank
__global__ __launch_bounds__(256) void lora_z_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ A, int rank,
    long T, int H, int top_k, int n_lora_groups,
    const int* __restrict__ offsets, const int* __restrict__ sorted_pair,
    bool gather, float* __restrict__ z) {
  __shared__ f32x4 red[4][NQ][64];
  __shared__ int s_cum[1025];
  __shared__ int s_wsum[4];
  lora_tile_prefix(offsets, n_lora_groups, s_cum, s_wsum);
  const int tile = blockIdx.x;
  if (tile >= s_cum[n_lora_groups]) return;      // uniform over the workgroup
  int g = 0, hi = n_lora_groups - 1;             // last g with s_cum[g] <= tile
  while (g < hi) {
    const int mid = (g + hi + 1) >> 1;
    if (s_cum[mid] <= tile) g = mid; else hi = mid - 1;
  }
  const long r0 = offsets[g] + 16L * (tile - s_cum[g]);
  const int m = (int)min(16L, (long)offsets[g + 1] - r0);
  const int wave = threadIdx.x >> 6, lane = lane_id(), lr = lane & 15, lg = lane >> 4;
  const int hq = H >> 2;                         // this wave's quarter of H
  const long rl = r0 + min(lr, m - 1);           // this lane's operand row
  // operand row: the token of the pair (gathered x), or the sorted row itself
  const uint16_t* xr = x + (gather ? pair_token(sorted_pair[rl], T, top_k) : rl) * H +
                       wave * hq + 8 * lg;
  const uint16_t* Ag = A + (long)g * rank * H + wave * hq + 8 * lg;
  f32x4 acc[NQ];
  lora_z_rows<NQ>(xr, Ag, rank, H, acc);
#pragma unroll
  for (int n = 0; n < NQ; ++n) red[wave][n][lane] = acc[n];
  __syncthreads();
  if (wave == 0) {
    // acc[n][r]: row 4 (lane / 16) + r, rank 16 n + lane % 16
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
      const f32x4 v = ((red[0][n][lane] + red[1][n][lane]) + red[2][n][lane]) + red[3][n][lane];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tr = 4 * lg + r;
        const int q = 16 * n + lr;
        if (tr < m && q < rank) z[(r0 + tr) * rank + q] = v[r];
      }
    }
  }
}

// A batch of adapters, grouped by adapter: one work item per (local group g,
// adapter a) pair, a = -1 standing for the rows without an adapter (z = 0).
// The item walks g's sorted rows in windows of 256, compacts those of
// adapter a into LDS (ballot prefix) and runs the K loop above on 16 of
// them at a time, so each adapter's A is read once per 16 of its rows
// instead of once per 16-row tile that meets it. zad[r] gets a (-1: none).
template <int NQ>
__global__ __launch_bounds__(256) void lora_z_batch_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ A, int rank,
    long T, int H, int top_k, int n_lora_groups, const int* __restrict__ offsets,
    const int* __restrict__ sorted_pair, bool gather, int n_adapters,
    const int* __restrict__ adapter_ids, float* __restrict__ z, int* __restrict__ zad) {
  __shared__ f32x4 red[4][NQ][64];
  __shared__ int s_rows[256];
  __shared__ int s_cnt[4];
  const int wave = threadIdx.x >> 6, lane = lane_id(), lr = lane & 15, lg = lane >> 4;
  const int hq = H >> 2;                         // each wave's quarter of H
  const int items = n_lora_groups * (n_adapters + 1);
  for (int it = blockIdx.x; it < items; it += gridDim.x) {
    const int g = it / (n_adapters + 1), a = it - g * (n_adapters + 1) - 1;
    const int rb = offsets[g], re = offsets[g + 1];
    for (int w0 = rb; w0 < re; w0 += 256) {
      const int r = w0 + (int)threadIdx.x;
      bool take = false;
      if (r < re) {
        int ad = adapter_ids[pair_token(sorted_pair[r], T, top_k)];
        if (ad < 0 || ad >= n_adapters) ad = -1;
        take = ad == a;
      }
      const unsigned long long bal = __ballot(take);
      if (lane == 0) s_cnt[wave] = __popcll(bal);
      __syncthreads();
      int before = 0, cnt = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        before += w < wave ? s_cnt[w] : 0;
        cnt += s_cnt[w];
      }
      if (take) s_rows[before + __popcll(bal & ((1ull << lane) - 1ull))] = r;
      __syncthreads();
      if (a < 0) {                               // rows without an adapter
        for (int i = threadIdx.x; i < cnt * rank; i += 256)
          z[(long)s_rows[i / rank] * rank + i % rank] = 0.0f;
        if (zad)
          for (int i = threadIdx.x; i < cnt; i += 256) zad[s_rows[i]] = -1;
      } else {
        const uint16_t* Ag = A + ((long)a * n_lora_groups + g) * rank * H + wave * hq + 8 * lg;
        for (int c0 = 0; c0 < cnt; c0 += 16) {
          const int m = min(16, cnt - c0);
          const int rl = s_rows[c0 + min(lr, m - 1)];
          const uint16_t* xr = x + (gather ? pair_token(sorted_pair[rl], T, top_k) : (long)rl) * H +
                               wave * hq + 8 * lg;
          f32x4 acc[NQ];
          lora_z_rows<NQ>(xr, Ag, rank, H, acc);
#pragma unroll
          for (int n = 0; n < NQ; ++n) red[wave][n][lane] = acc[n];
          __syncthreads();
          if (wave == 0) {
            // acc[n][r]: row 4 (lane / 16) + r of the 16, rank 16 n + lane % 16
#pragma unroll
            for (int n = 0; n < NQ; ++n) {
              const f32x4 v = ((red[0][n][lane] + red[1][n][lane]) + red[2][n][lane]) + red[3][n][lane];
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) {
                const int tr = 4 * lg + rr;
                const int q = 16 * n + lr;
                if (tr < m && q < rank) z[(long)s_rows[c0 + tr] * rank + q] = v[rr];
              }
            }
            if (zad && lane < m) zad[s_rows[c0 + lane]] = a;
          }
          __syncthreads();                       // red is reused by the next 16 rows
        }
      }
      __syncthreads();                           // s_rows / s_cnt are reused
    }
  }
}

hipError_t launch_lora_z(const void* x_bf16, const void* A, int rank, long T,
                         int H, int top_k, int n_lora_groups, long p_cap,
                         const int* offsets, const int* sorted_pair, bool gather,
                         int n_adapters, const int* adapter_ids, float* z,
                         int* zad, hipStream_t s) {
  if (p_cap == 0 || n_lora_groups == 0) return hipSuccess;
  if (n_adapters > 1) {
    const long items = (long)n_lora_groups * (n_adapters + 1);
    dim3 grid((unsigned)std::min<long>(items, 2048)), block(256);
    if (rank <= 16)
      hipLaunchKernelGGL(lora_z_batch_kernel<1>, grid, block, 0, s, (const uint16_t*)x_bf16,
                         (const uint16_t*)A, rank, T, H, top_k, n_lora_groups, offsets,
                         sorted_pair, gather, n_adapters, adapter_ids, z, zad);
    else
      hipLaunchKernelGGL(lora_z_batch_kernel<2>, grid, block, 0, s, (const uint16_t*)x_bf16,
                         (const uint16_t*)A, rank, T, H, top_k, n_lora_groups, offsets,
                         sorted_pair, gather, n_adapters, adapter_ids, z, zad);
    return hipGetLastError();
  }
  // tiles <= one per non-empty expert plus one per 16 rows
  const long tiles = std::min<long>(p_cap, n_lora_groups + p_cap / 16);
  dim3 grid((unsigned)tiles), block(256);
#define LZ(NQ)                                                                \
  hipLaunchKernelGGL(lora_z_kernel<NQ>, grid, block, 0, s,                    \
                     (const uint16_t*)x_bf16, (const uint16_t*)A, rank, T, H, \
                     top_k, n_lora_groups, offsets, sorted_pair, gather, z)
  if (rank <= 16) LZ(1);
  else LZ(2);
#undef LZ
  return hipGetLastError();
}

}  // namespace moe
