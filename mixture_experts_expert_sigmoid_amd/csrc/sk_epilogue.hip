// GEMM1's epilogue after the split-K (stream-K) schedule of the FP8 and
// 4-bit grouped GEMMs: the partial-slot sum in slot order, then the fused
// epilogue's arithmetic. Epilogue semantics: "[Moe] Fix flashinfer_trtllm
// silently dropping swiglu_limit clamped SwiGLU activation" (sglang PR
// #39920, "Modifications"); "fix(sm90): support parameterized SwiGLU in FP8
// MegaMoE" (DeepGEMM PR #445, "Summary"); global scales and the LoRA delta
// in true units: "FlashInfer 0.6.18 SM100a+SM103a MoE-LoRA AOT" release
// notes, "Changes since 1b699bf".
#include "gemm_common.h"

namespace moe {

// GEMM1 after stream-K: one wave per (sorted row r, 128 h columns nt) sums
// the partial slots of r's tile in slot order, then applies the fused
// epilogue's arithmetic (global scales, LoRA delta in true units,
// parameterized SwiGLU, then FP8H: e4m3 re-quantisation per 128 columns,
// else bf16 round-to-nearest-even); lane l owns h columns nt*128 + 2l, 2l + 1.
template <bool FP8H>
__global__ __launch_bounds__(kThreads) void gemm1_sk_epilogue_kernel(GemmParams P, int grid) {
  __shared__ int s_cum[kMaxGroups + 1];
  __shared__ int s_off[kMaxGroups + 1];
  __shared__ int s_wsum[8];
  const int G = P.G, I = P.I;
  const int NT = I >> 7, NS = P.K >> 7;
  tile_prefix<kSkBM>(P.offsets, G, s_cum, s_wsum);
  for (int i = threadIdx.x; i <= G; i += kThreads) s_off[i] = P.offsets[i];
  __syncthreads();
  // SK_DEVICE: the plain kernel ran the fused epilogue instead
  if (P.sk_mode == SK_DEVICE && !sk_rule((long)s_cum[G] * NT, NS)) return;
  const long U = (long)s_cum[G] * NT * NS;
  const int W = sk_workgroups((long)s_cum[G] * NT, NS, grid);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long items = (long)s_off[G] * NT;
  for (long it = (long)blockIdx.x * 8 + wave; it < items; it += (long)gridDim.x * 8) {
    const int r = (int)(it / NT), nt = (int)(it - (long)r * NT);
    const int g = group_of_row(s_off, G, r);
    const int mt = s_cum[g] + (r - s_off[g]) / kSkBM;
    const int nsl = sk_nslots(((long)mt * NT + nt) * NS, NS, U, W);
    const int c = nt * 128 + 2 * lane;
    float a[2][2] = {{0.f, 0.f}, {0.f, 0.f}};       // [gate | up][column]
    // the tile's slots (at most kSkSlots): every load issued, then the
    // additions in slot order
    f32x2 vg[kSkSlots], vu[kSkSlots];
#pragma unroll
    for (int sl = 0; sl < kSkSlots; ++sl)
      if (sl < nsl) {
        const float* pr = P.part + ((long)sl * P.p_rows + r) * P.N;
        vg[sl] = *(const f32x2*)(pr + c);
        vu[sl] = *(const f32x2*)(pr + I + c);
      }
#pragma unroll
    for (int sl = 0; sl < kSkSlots; ++sl)
      if (sl < nsl) {
        a[0][0] += vg[sl][0]; a[0][1] += vg[sl][1];
        a[1][0] += vu[sl][0]; a[1][1] += vu[sl][1];
      }
    if (P.gscale) {
      const float gsg = P.gscale[2 * g], gsu = P.gscale[2 * g + 1];
      a[0][0] *= gsg; a[0][1] *= gsg;
      a[1][0] *= gsu; a[1][1] *= gsu;
    }
    if (P.z && g < P.lora_groups) {
      // ranks in steps of 8 whose loads are all issued before the FMAs
      // (ascending q, as in the fused epilogue): one 16-byte load per B row
      // when the rank is a multiple of 8; a batch of adapters takes the
      // row's adapter's B (a row without one has z = 0)
      const int R = P.lora_rank;
      const int ad = P.n_adapters > 1 ? max(P.zad[r], 0) : 0;
      const uint16_t* Bg = P.lora_B + ((long)ad * P.lora_groups + g) * 2 * I * R;
      const float* zr = P.z + (long)r * R;
      for (int q0 = 0; q0 < R; q0 += 8) {
        float zq[8];
        uint32_t bw[2][2][4];                    // [gate | up][column][rank pair]
#pragma unroll
        for (int i = 0; i < 8; ++i) zq[i] = zr[min(q0 + i, R - 1)];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const uint16_t* br = Bg + (long)(hh * I + c + j) * R;
            if ((R & 7) == 0) {
              const i32x4 v = *(const i32x4*)(br + q0);
#pragma unroll
              for (int i = 0; i < 4; ++i) bw[hh][j][i] = (uint32_t)v[i];
            } else {
#pragma unroll
              for (int i = 0; i < 4; ++i)
                bw[hh][j][i] = (uint32_t)br[min(q0 + 2 * i, R - 1)] |
                               ((uint32_t)br[min(q0 + 2 * i + 1, R - 1)] << 16);
            }
          }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if (q0 + i < R) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
              for (int j = 0; j < 2; ++j) {
                const uint32_t w = bw[hh][j][i >> 1];
                const float b = bf16_bits_to_f32((i & 1) ? w >> 16 : w & 0xFFFFu);
                a[hh][j] = fmaf(zq[i], P.lora_scale * b, a[hh][j]);
              }
          }
        }
      }
    }
    const float L = P.limit, al = P.alpha, be = P.beta;
    float hv[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float gg = fminf(a[0][j], L);
      const float uu = fminf(fmaxf(a[1][j], -L), L);
      const float sg = __builtin_amdgcn_rcpf(1.0f + expf(-al * gg));
      hv[j] = gg * sg * (uu + be);
    }
    if constexpr (FP8H) {
      const float am = wave_max(fmaxf(fabsf(hv[0]), fabsf(hv[1])));
      const float sc = am > 0.0f ? am / 448.0f : 1.0f;
      const float inv = 1.0f / sc;
      const float q0 = __builtin_amdgcn_fmed3f(hv[0] * inv, -448.0f, 448.0f);
      const float q1 = __builtin_amdgcn_fmed3f(hv[1] * inv, -448.0f, 448.0f);
      const int v = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
      *(uint16_t*)(P.h + (long)r * I + c) = (uint16_t)v;
      if (lane == 0) P.hs[(long)r * NT + nt] = sc;
      if (P.h_lora)
        *(uint32_t*)(P.h_lora + (long)r * I + c) =
            f32_to_bf16_bits(hv[0]) | (f32_to_bf16_bits(hv[1]) << 16);
    } else {
      *(uint32_t*)((uint16_t*)P.h + (long)r * I + c) =
          f32_to_bf16_bits(hv[0]) | (f32_to_bf16_bits(hv[1]) << 16);
    }
  }
}

hipError_t launch_gemm1_sk_epilogue(const GemmParams& P, int sk_grid, bool fp8h, hipStream_t s) {
  const long items = P.p_rows * (P.I >> 7);     // upper bound: rows used <= p_rows
  if (items == 0) return hipSuccess;
  const long nwg = std::min<long>((items + 7) / 8, (long)num_cus() * 4);
  if (fp8h)
    gemm1_sk_epilogue_kernel<true><<<dim3((unsigned)nwg), dim3(kThreads), 0, s>>>(P, sk_grid);
  else
    gemm1_sk_epilogue_kernel<false><<<dim3((unsigned)nwg), dim3(kThreads), 0, s>>>(P, sk_grid);
  return hipGetLastError();
}

}  // namespace moe
