// Grouped expert GEMMs on CDNA4 MFMA: GEMM1 over the fused [gate | up]
// weight with the parameterized-SwiGLU epilogue (plus optional per-half
// global scales, LoRA delta and FP8 re-quantisation of h), and GEMM2 (down)
// writing fp32 rows for the weighted combine.
//
// Formats:
//   FP8  blockwise 128x128 e4m3 weights and per-token per-128-column e4m3
//        activations ("[Moe] Fix flashinfer_trtllm silently dropping
//        swiglu_limit clamped SwiGLU activation", sglang PR #39920,
//        "Modifications": DeepSeekFp8). The block scales make each 128-deep
//        slice of K its own dot product: its partial sum is scaled by
//        xs[row][kb] * ws[nb][kb] and added to the fp32 accumulator.
//   INT4 group-32 weights, byte = (odd k nibble << 4) | even k nibble,
//        w = (nibble - 8) * scale[n][k/32] ("sm100: Fused INT4 grouped +
//        SiLU Triton kernel", batchgen PR #239, commit text).
//   BF16 weights and activations.
// Epilogue: g' = min(g, L), u' = clamp(u, -L, L), h = g' sigmoid(alpha g')
// (u' + beta) (sglang PR #39920 "Modifications"; "fix(sm90): support
// parameterized SwiGLU in FP8 MegaMoE", DeepGEMM PR #445, "Summary"). The
// LoRA delta and the per-half global scales follow the true-units rule of
// "FlashInfer 0.6.18 SM100a+SM103a MoE-LoRA AOT" ("Changes since 1b699bf"):
// each half is scaled by its own global scale first, then the delta is added.
//
// Arithmetic: every format is expanded EXACTLY to a 16-bit MFMA type while
// the tile is written into LDS -- e4m3 -> bf16 (4 significant bits fit the 8
// of bf16), int4 -> fp16 ((nibble - 8) * bf16 scale has at most 11
// significant bits; 0x6400 | nibble is the fp16 1024 + nibble, minus 1032
// gives nibble - 8), bf16 activations -> fp16 for the int4 path -- and
// multiplied on v_mfma_f32_16x16x32_{bf16,f16}, whose accumulation of such
// products is exact. The FP8 MFMA is not used: on gfx950 it accumulates each
// dot product at reduced internal precision (measured about 2e-5 of
// sum |products|), which is enough to flip the e4m3 re-quantisation of h.
//
// Tiling: a workgroup of 8 waves owns BM sorted rows of one expert and 256
// weight rows in two halves of 128 ("lo", "hi"): for GEMM1 lo = gate rows
// n0..n0+127 and hi = the matching up rows I+n0..I+n0+127, so one tile yields
// 128 complete h columns (the FP8 re-quantisation group); for GEMM2 lo/hi are
// output columns n0..n0+255. Wave (wm, wn) computes rows wm*BM/2.. of columns
// wn*32..wn*32+31 of both halves, so gate and up values of one h element sit
// in the same lane. K advances 64 per stage: global -> registers (two stages
// in flight) -> exact expansion -> LDS (double buffered, one barrier per
// stage). LDS rows are 128 bytes; their 16-byte chunks are XOR-swizzled with
// (row / 2) mod 8 so the 16 rows read by one ds_read_b128 phase hit distinct
// banks. Workgroups are persistent: each computes the tile count from the
// expert offsets on the device and walks its XCD's contiguous share of the
// tiles, so the N-tiles of one expert (which share the gathered activation
// rows) stay in one XCD's L2.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace moe {

enum { FMT_BF16 = 0, FMT_FP8 = 1, FMT_INT4 = 2 };

constexpr int kThreads = 512;
constexpr int kMaxGroups = 1024;
constexpr int KS = 64;               // K elements per pipeline stage

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

// 8 e4m3fn codes (two dwords, k order) -> 8 bf16 (four dwords), exact: the
// hardware converts to fp32 and every e4m3 value has at most 4 significant
// bits, so the upper half of the fp32 is the bf16 value.
__device__ __forceinline__ i32x4 e4m3x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, false);
  f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, true);
  f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, false);
  f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, true);
  i32x4 o;
  o[0] = (int)__builtin_amdgcn_perm(__float_as_uint(a[1]), __float_as_uint(a[0]), 0x07060302u);
  o[1] = (int)__builtin_amdgcn_perm(__float_as_uint(b[1]), __float_as_uint(b[0]), 0x07060302u);
  o[2] = (int)__builtin_amdgcn_perm(__float_as_uint(c[1]), __float_as_uint(c[0]), 0x07060302u);
  o[3] = (int)__builtin_amdgcn_perm(__float_as_uint(d[1]), __float_as_uint(d[0]), 0x07060302u);
  return o;
}

// 8 bf16 -> 8 fp16 (exact for |v| in [2^-14, 65504])
__device__ __forceinline__ i32x4 bf16x8_to_f16x8(i32x4 v) {
  i32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t w = (uint32_t)v[i];
    _Float16 lo = (_Float16)bf16_bits_to_f32(w & 0xFFFFu);
    _Float16 hi = (_Float16)bf16_bits_to_f32(w >> 16);
    o[i] = (int)((uint32_t)__builtin_bit_cast(uint16_t, lo) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16));
  }
  return o;
}

// 8 packed nibbles (k = 0..7, low nibble first) -> 8 fp16 (nibble - 8) * s
__device__ __forceinline__ i32x4 int4x8_to_f16x8(uint32_t w, f16x2 sc2) {
  uint32_t lo = w & 0x0F0F0F0Fu;          // even-k nibbles, byte i = pair i
  uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;   // odd-k nibbles
  i32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t pr = ((lo >> (8 * i)) & 0xFFu) | (((hi >> (8 * i)) & 0xFFu) << 16);
    pr |= 0x64006400u;                    // (1024 + n_even, 1024 + n_odd)
    f16x2 v = __builtin_bit_cast(f16x2, pr);
    v = (v - (f16x2){(_Float16)1032.0f, (_Float16)1032.0f}) * sc2;
    o[i] = (int)__builtin_bit_cast(uint32_t, v);
  }
  return o;
}

struct GemmParams {
  // A side
  const uint8_t* a;          // x (GEMM1: gathered by token) or h (GEMM2)
  const float* as;           // FP8 per-row scales [rows][K/128]
  long a_ld;                 // bytes per A row
  const int* sorted_pair;    // GEMM1: sorted row -> pair id
  long T;
  int top_k;
  // B side
  const uint8_t* w;          // [G][N][K] codes (bytes; INT4 packed)
  const void* wsc;           // FP8 fp32 [G][N/128][K/128]; INT4 bf16 [G][N][K/32]
  int N, K, G;
  const int* offsets;
  int I;
  // GEMM1 epilogue
  const float* gscale;
  float alpha, beta, limit;
  const float* z;
  const uint16_t* lora_B;
  int lora_rank, lora_groups;
  float lora_scale;
  uint8_t* h;                // GEMM1 out: e4m3 [p_cap][I] or bf16 [p_cap][I]
  float* hs;
  // GEMM2 out
  float* y;                  // [p_cap][N]
};

template <int FMT, int BM>
struct Geo {
  // per 64-K stage, in 16-byte global chunks
  static constexpr int A_SRC = (FMT == FMT_FP8) ? 64 : 128;       // bytes per A row
  static constexpr int A_CH = BM * A_SRC / 16;
  static constexpr int A_PT = (A_CH + kThreads - 1) / kThreads;   // loads per thread
  static constexpr int B_SRC = (FMT == FMT_FP8) ? 64 : (FMT == FMT_INT4 ? 32 : 128);
  static constexpr int B_CH = 256 * B_SRC / 16;
  static constexpr int B_PT = B_CH / kThreads;
  static constexpr int A_LDS = BM * 128;                          // 16-bit tile bytes
  static constexpr int B_LDS = 256 * 128;
  static constexpr int STAGE = A_LDS + B_LDS;
  static constexpr int TOTAL = 2 * STAGE;
};

template <int FMT, int BM>
struct Regs {
  i32x4 a[Geo<FMT, BM>::A_PT];
  i32x4 b[Geo<FMT, BM>::B_PT];
  uint32_t sc;    // INT4: this thread's bf16 group scale
  float xs;       // FP8: row scale of the stage's 128-K block
};

template <int FMT, int BM, bool G1>
__global__ __launch_bounds__(kThreads) void moe_gemm_kernel(GemmParams P) {
  using Gm = Geo<FMT, BM>;
  constexpr int MS = BM / 32;            // 16-row subtiles per wave
  constexpr bool SCALED = (FMT == FMT_FP8);
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int s_cum[kMaxGroups + 1];
  __shared__ int s_wsum[8];
  __shared__ float s_xs[2][BM];          // FP8 row scales, by 128-K block parity

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int lr = lane & 15, lg = lane >> 4;
  const int G = P.G, K = P.K;
  const int NT = G1 ? (P.I >> 7) : ((P.N + 255) >> 8);
  const int NS = K / KS;
  const int nkb = K >> 7;

  // ---- M-tile prefix over groups (once per workgroup) ---------------------
  {
    int c0 = 0, c1 = 0;
    const int g0 = 2 * tid, g1 = 2 * tid + 1;
    if (g0 < G) c0 = (P.offsets[g0 + 1] - P.offsets[g0] + BM - 1) / BM;
    if (g1 < G) c1 = (P.offsets[g1 + 1] - P.offsets[g1] + BM - 1) / BM;
    int v = c0 + c1, incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    int base = 0;
    for (int i = 0; i < wave; ++i) base += s_wsum[i];
    int excl = base + incl - v;
    if (g0 < G) s_cum[g0] = excl;
    if (g1 < G) s_cum[g1] = excl + c0;
    if (tid == 0) {
      int tot = 0;
      for (int i = 0; i < 8; ++i) tot += s_wsum[i];
      s_cum[G] = tot;
    }
    __syncthreads();
  }
  const int total = s_cum[G] * NT;
  // XCD x (= blockIdx % 8) owns logical tiles [x*chunk, (x+1)*chunk)
  const int xcd = blockIdx.x & 7, nper = gridDim.x >> 3, slot = blockIdx.x >> 3;
  const int chunk = (total + 7) >> 3;
  const int t_end = min(total, (xcd + 1) * chunk);

  for (int lt = xcd * chunk + slot; lt < t_end; lt += nper) {
    const int mt = lt / NT, nt = lt - mt * NT;
    int glo = 0, ghi = G - 1;                 // group: last g with s_cum[g] <= mt
    while (glo < ghi) {
      int mid = (glo + ghi + 1) >> 1;
      if (s_cum[mid] <= mt) glo = mid; else ghi = mid - 1;
    }
    const int g = glo;
    const int row0 = P.offsets[g] + (mt - s_cum[g]) * BM;   // first sorted row
    const int m = min(BM, P.offsets[g + 1] - row0);

    int n_lo, n_hi;
    if (G1) {
      n_lo = nt * 128;
      n_hi = P.I + nt * 128;
    } else {
      n_lo = nt * 256;
      n_hi = (n_lo + 128 < P.N) ? n_lo + 128 : n_lo;       // ragged last tile
    }
    const long wrow = (FMT == FMT_INT4) ? K / 2 : (long)K * (FMT == FMT_FP8 ? 1 : 2);
    const uint8_t* wg = P.w + (long)g * P.N * wrow;

    // ---- per-thread global sources for this tile -------------------------
    const uint8_t* ap[Gm::A_PT];
    int a_row[Gm::A_PT], a_ch[Gm::A_PT];
    bool a_on[Gm::A_PT];
#pragma unroll
    for (int i = 0; i < Gm::A_PT; ++i) {
      int c = tid + i * kThreads;
      a_on[i] = (Gm::A_CH % kThreads == 0) || c < Gm::A_CH;
      c = min(c, Gm::A_CH - 1);     // surplus threads load a duplicate, store nothing
      int row = c / (Gm::A_SRC / 16), ch = c % (Gm::A_SRC / 16);
      a_row[i] = row; a_ch[i] = ch;
      int r = row0 + (row < m ? row : 0);
      long src = r;
      if (G1) {
        int p = P.sorted_pair[r];
        long npr = P.T * (long)P.top_k;
        src = (p < npr) ? (long)(p / P.top_k) : (long)(p - npr);
      }
      ap[i] = P.a + src * P.a_ld + ch * 16;
    }
    const float* xsp = nullptr;     // FP8: row (tid mod BM)'s activation scales
    if (SCALED) {
      const int tr = tid & (BM - 1);
      int r = row0 + (tr < m ? tr : 0);
      long src = r;
      if (G1) {
        int p = P.sorted_pair[r];
        long npr = P.T * (long)P.top_k;
        src = (p < npr) ? (long)(p / P.top_k) : (long)(p - npr);
      }
      xsp = P.as + src * nkb;
    }
    const uint8_t* bp[Gm::B_PT];
    int b_row[Gm::B_PT], b_ch[Gm::B_PT];
#pragma unroll
    for (int i = 0; i < Gm::B_PT; ++i) {
      int c = tid + i * kThreads;
      int row = c / (Gm::B_SRC / 16), ch = c % (Gm::B_SRC / 16);
      b_row[i] = row; b_ch[i] = ch;
      int n = (row < 128) ? n_lo + row : n_hi + (row - 128);
      bp[i] = wg + (long)n * wrow + ch * 16;
    }
    const uint16_t* scp = nullptr;   // INT4: bf16 scale row of this thread's B chunk
    if (FMT == FMT_INT4) {
      int row = b_row[0];
      int n = (row < 128) ? n_lo + row : n_hi + (row - 128);
      scp = (const uint16_t*)P.wsc + ((long)g * P.N + n) * (K / 32) + b_ch[0];
    }

    // Loads are unconditional (past the last stage they re-read it) so the
    // compiler's wait counts stay static and two stages remain in flight.
    auto gload = [&](Regs<FMT, BM>& R, int s) {
      s = min(s, NS - 1);
      const long adv = (long)s * Gm::A_SRC;
#pragma unroll
      for (int i = 0; i < Gm::A_PT; ++i) R.a[i] = *(const i32x4*)(ap[i] + adv);
      const long bdv = (long)s * Gm::B_SRC;
#pragma unroll
      for (int i = 0; i < Gm::B_PT; ++i) R.b[i] = *(const i32x4*)(bp[i] + bdv);
      if (FMT == FMT_INT4) R.sc = scp[2 * s];
      if (SCALED) R.xs = xsp[s >> 1];
    };
    auto sstore = [&](const Regs<FMT, BM>& R, int s, auto par) {
      constexpr int PAR = decltype(par)::value;
      if (s >= NS) return;
      uint8_t* sa = smem + PAR * Gm::STAGE;
      uint8_t* sb = sa + Gm::A_LDS;
#pragma unroll
      for (int i = 0; i < Gm::A_PT; ++i) {
        if (!a_on[i]) continue;
        const int row = a_row[i];
        if constexpr (FMT == FMT_FP8) {       // 16 codes -> logical chunks 2ch, 2ch+1
          i32x4 v = R.a[i];
          *(i32x4*)(sa + row * 128 + swz(row, 2 * a_ch[i]) * 16) =
              e4m3x8_to_bf16x8((uint32_t)v[0], (uint32_t)v[1]);
          *(i32x4*)(sa + row * 128 + swz(row, 2 * a_ch[i] + 1) * 16) =
              e4m3x8_to_bf16x8((uint32_t)v[2], (uint32_t)v[3]);
        } else if constexpr (FMT == FMT_INT4) {
          *(i32x4*)(sa + row * 128 + swz(row, a_ch[i]) * 16) = bf16x8_to_f16x8(R.a[i]);
        } else {
          *(i32x4*)(sa + row * 128 + swz(row, a_ch[i]) * 16) = R.a[i];
        }
      }
#pragma unroll
      for (int i = 0; i < Gm::B_PT; ++i) {
        const int row = b_row[i];
        if constexpr (FMT == FMT_FP8) {
          i32x4 v = R.b[i];
          *(i32x4*)(sb + row * 128 + swz(row, 2 * b_ch[i]) * 16) =
              e4m3x8_to_bf16x8((uint32_t)v[0], (uint32_t)v[1]);
          *(i32x4*)(sb + row * 128 + swz(row, 2 * b_ch[i] + 1) * 16) =
              e4m3x8_to_bf16x8((uint32_t)v[2], (uint32_t)v[3]);
        } else if constexpr (FMT == FMT_INT4) {   // 32 nibbles -> chunks 4ch..4ch+3
          _Float16 sh = (_Float16)bf16_bits_to_f32(R.sc);
          f16x2 s2 = (f16x2){sh, sh};
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *(i32x4*)(sb + row * 128 + swz(row, 4 * b_ch[i] + q) * 16) =
                int4x8_to_f16x8((uint32_t)R.b[i][q], s2);
        } else {
          *(i32x4*)(sb + row * 128 + swz(row, b_ch[i]) * 16) = R.b[i];
        }
      }
      if (SCALED && PAR == 0 && tid < BM) s_xs[(s >> 1) & 1][tid] = R.xs;
    };

    // ---- accumulators -----------------------------------------------------
    f32x4 acc[MS][4], part[MS][4];
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
        part[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
      }
    const int rbase = wm * (BM / 2);
    const float* wscale = SCALED ? (const float*)P.wsc + (long)g * (P.N >> 7) * nkb : nullptr;
    const int nb_lo = n_lo >> 7, nb_hi = n_hi >> 7;

    auto compute = [&](int s, auto par) {
      constexpr int PAR = decltype(par)::value;   // == s & 1
      if (s >= NS) return;
      const uint8_t* sa = smem + PAR * Gm::STAGE;
      const uint8_t* sb = sa + Gm::A_LDS;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        i32x4 af[MS];
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) {
          int row = rbase + ms * 16 + lr;
          af[ms] = *(const i32x4*)(sa + row * 128 + swz(row, kk * 4 + lg) * 16);
        }
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) {
          int row = (ns < 2 ? 0 : 128) + wn * 32 + (ns & 1) * 16 + lr;
          i32x4 bv = *(const i32x4*)(sb + row * 128 + swz(row, kk * 4 + lg) * 16);
#pragma unroll
          for (int ms = 0; ms < MS; ++ms) {
            f32x4& d = SCALED ? part[ms][ns] : acc[ms][ns];
            // an FP8 scale block starts from zero (even stage, first K slice)
            const f32x4 c = (SCALED && PAR == 0 && kk == 0) ? (f32x4){0.f, 0.f, 0.f, 0.f} : d;
            if constexpr (FMT == FMT_INT4)
              d = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, af[ms]),
                                                         __builtin_bit_cast(f16x8, bv), c, 0, 0, 0);
            else
              d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af[ms]),
                                                          __builtin_bit_cast(bf16x8, bv), c, 0, 0, 0);
          }
        }
      }
      if (SCALED && PAR == 1) {    // end of a 128-deep scale block
        const int kb = s >> 1;
        const float ws_lo = wscale[nb_lo * nkb + kb];
        const float ws_hi = wscale[nb_hi * nkb + kb];
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) {
          f32x4 xr = *(const f32x4*)(&s_xs[kb & 1][rbase + ms * 16 + 4 * lg]);
#pragma unroll
          for (int ns = 0; ns < 4; ++ns) {
            const float wsv = ns < 2 ? ws_lo : ws_hi;
#pragma unroll
            for (int r = 0; r < 4; ++r)
              acc[ms][ns][r] = fmaf(part[ms][ns][r], xr[r] * wsv, acc[ms][ns][r]);
          }
        }
      }
    };

    // ---- pipelined K loop: two stages in flight ---------------------------
    // stage t lives in register set t % 3 and LDS buffer t % 2; unrolled by
    // six so both are compile-time.
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    Regs<FMT, BM> r0, r1, r2;
    gload(r0, 0);
    gload(r1, 1);
    sstore(r0, 0, P0{});
    __syncthreads();
    for (int s = 0; s < NS; s += 6) {
      gload(r2, s + 2); compute(s, P0{});     sstore(r1, s + 1, P1{}); __syncthreads();
      gload(r0, s + 3); compute(s + 1, P1{}); sstore(r2, s + 2, P0{}); __syncthreads();
      gload(r1, s + 4); compute(s + 2, P0{}); sstore(r0, s + 3, P1{}); __syncthreads();
      gload(r2, s + 5); compute(s + 3, P1{}); sstore(r1, s + 4, P0{}); __syncthreads();
      gload(r0, s + 6); compute(s + 4, P0{}); sstore(r2, s + 5, P1{}); __syncthreads();
      gload(r1, s + 7); compute(s + 5, P1{}); sstore(r0, s + 6, P0{}); __syncthreads();
    }

    // ======================= epilogues =====================================
    if constexpr (!G1) {
#pragma unroll
      for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) {
          int col = (ns < 2 ? n_lo : n_hi) + wn * 32 + (ns & 1) * 16 + lr;
          bool colok = (ns < 2) || (n_hi != n_lo);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            int tr = rbase + ms * 16 + 4 * lg + r;
            if (tr < m && colok) P.y[(long)(row0 + tr) * P.N + col] = acc[ms][ns][r];
          }
        }
    } else {
      // gate = ns 0,1 ; up = ns 2,3 (same h columns)
      float gsg = 1.0f, gsu = 1.0f;
      if (P.gscale) { gsg = P.gscale[2 * g]; gsu = P.gscale[2 * g + 1]; }
#pragma unroll
      for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            acc[ms][j][r] *= gsg;
            acc[ms][j + 2][r] *= gsu;
          }
      if (P.z && g < P.lora_groups) {
        // delta[row][n] = s * sum_q z[row][q] * B[g][n][q]; z staged as [q][BM]
        float* sz = (float*)smem;
        const int R = P.lora_rank;
        for (int i = tid; i < R * BM; i += kThreads) {
          int q = i / BM, tr = i - q * BM;
          int rr = row0 + (tr < m ? tr : 0);
          sz[q * BM + tr] = P.z[(long)rr * R + q];
        }
        __syncthreads();
        const uint16_t* Bg = P.lora_B + (long)g * 2 * P.I * R;
        for (int q = 0; q < R; ++q) {
          float bgv[2], buv[2];
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            int c = wn * 32 + j * 16 + lr;
            bgv[j] = P.lora_scale * bf16_bits_to_f32(Bg[(long)(n_lo + c) * R + q]);
            buv[j] = P.lora_scale * bf16_bits_to_f32(Bg[(long)(n_hi + c) * R + q]);
          }
#pragma unroll
          for (int ms = 0; ms < MS; ++ms) {
            f32x4 zq = *(const f32x4*)(sz + q * BM + rbase + ms * 16 + 4 * lg);
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                acc[ms][j][r] = fmaf(zq[r], bgv[j], acc[ms][j][r]);
                acc[ms][j + 2][r] = fmaf(zq[r], buv[j], acc[ms][j + 2][r]);
              }
          }
        }
        __syncthreads();
      }
      float hv[MS][2][4];
      const float L = P.limit, al = P.alpha, be = P.beta;
#pragma unroll
      for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float gg = fminf(acc[ms][j][r], L);
            float uu = fminf(fmaxf(acc[ms][j + 2][r], -L), L);
            float sg = 1.0f / (1.0f + expf(-al * gg));
            hv[ms][j][r] = gg * sg * (uu + be);
          }
      if constexpr (FMT == FMT_FP8) {
        uint8_t* sh = smem;                              // [BM][128] codes
        float* s_amax = (float*)(smem + BM * 128);       // [4][BM]
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float a = max16(fmaxf(fabsf(hv[ms][0][r]), fabsf(hv[ms][1][r])));
            if (lr == 0) s_amax[wn * BM + rbase + ms * 16 + 4 * lg + r] = a;
          }
        __syncthreads();
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            int tr = rbase + ms * 16 + 4 * lg + r;
            float a = fmaxf(fmaxf(s_amax[tr], s_amax[BM + tr]),
                            fmaxf(s_amax[2 * BM + tr], s_amax[3 * BM + tr]));
            float sc = a > 0.0f ? a / 448.0f : 1.0f;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              int c = wn * 32 + j * 16 + lr;
              sh[tr * 128 + c] = (uint8_t)f32_to_e4m3(hv[ms][j][r] / sc);
            }
            if (wn == 0 && lr == 0 && tr < m) P.hs[(long)(row0 + tr) * (P.I >> 7) + nt] = sc;
          }
        __syncthreads();
        for (int c = tid; c < BM * 8; c += kThreads) {
          int tr = c >> 3, ch = c & 7;
          if (tr < m)
            *(i32x4*)(P.h + (long)(row0 + tr) * P.I + nt * 128 + ch * 16) =
                *(const i32x4*)(sh + tr * 128 + ch * 16);
        }
      } else {
        uint16_t* sh16 = (uint16_t*)smem;               // [BM][128] bf16
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            int tr = rbase + ms * 16 + 4 * lg + r;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              int c = wn * 32 + j * 16 + lr;
              sh16[tr * 128 + c] = (uint16_t)f32_to_bf16_bits(hv[ms][j][r]);
            }
          }
        __syncthreads();
        uint16_t* hout = (uint16_t*)P.h;
        for (int c = tid; c < BM * 16; c += kThreads) {
          int tr = c >> 4, ch = c & 15;
          if (tr < m)
            *(i32x4*)(hout + (long)(row0 + tr) * P.I + nt * 128 + ch * 8) =
                *(const i32x4*)(sh16 + tr * 128 + ch * 8);
        }
      }
    }
    __syncthreads();     // LDS is reused by the next tile
  }
}

static int num_cus() {
  static int n = 0;
  if (n == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        v > 0)
      n = v;
    else
      n = 256;
  }
  return n;
}

template <int FMT, int BM, bool G1>
static hipError_t run(const GemmParams& P, long p_cap, int NT, hipStream_t s) {
  constexpr int shm = Geo<FMT, BM>::TOTAL;
  static int per_cu = 0;   // resident workgroups per CU, per instantiation
  if (per_cu == 0) {
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&moe_gemm_kernel<FMT, BM, G1>),
        hipFuncAttributeMaxDynamicSharedMemorySize, shm);
    if (e != hipSuccess) return e;
    int nb = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &nb, reinterpret_cast<const void*>(&moe_gemm_kernel<FMT, BM, G1>), kThreads, shm);
    if (e != hipSuccess) return e;
    per_cu = nb > 0 ? nb : 1;
  }
  long max_tiles = ((p_cap + BM - 1) / BM + P.G) * (long)NT;
  long nwg = std::min<long>(max_tiles, (long)num_cus() * per_cu);
  nwg = (nwg + 7) & ~7L;
  if (nwg == 0) return hipSuccess;
  moe_gemm_kernel<FMT, BM, G1><<<dim3((unsigned)nwg), dim3(kThreads), shm, s>>>(P);
  return hipGetLastError();
}

template <int BM, bool G1>
static hipError_t run_fmt(int fmt, const GemmParams& P, long p_cap, int NT, hipStream_t s) {
  if (fmt == FMT_FP8) return run<FMT_FP8, BM, G1>(P, p_cap, NT, s);
  if (fmt == FMT_INT4) return run<FMT_INT4, BM, G1>(P, p_cap, NT, s);
  return run<FMT_BF16, BM, G1>(P, p_cap, NT, s);
}

template <bool G1>
static hipError_t dispatch(int fmt, const GemmParams& P, long p_cap, int NT, long rows_hint,
                           hipStream_t s) {
  // rows per expert on average decides the M tile
  if (rows_hint <= 32) return run_fmt<32, G1>(fmt, P, p_cap, NT, s);
  if (rows_hint <= 64) return run_fmt<64, G1>(fmt, P, p_cap, NT, s);
  return run_fmt<128, G1>(fmt, P, p_cap, NT, s);
}

hipError_t launch_gemm1(const Gemm1Args& a, hipStream_t s) {
  GemmParams P{};
  P.a = (const uint8_t*)a.x;
  P.as = a.xs;
  P.a_ld = (long)a.H * (a.fmt == FMT_FP8 ? 1 : 2);
  P.sorted_pair = a.sorted_pair;
  P.T = a.T;
  P.top_k = a.top_k;
  P.w = (const uint8_t*)a.wq;
  P.wsc = a.ws;
  P.N = 2 * a.I;
  P.K = a.H;
  P.G = a.G;
  P.offsets = a.offsets;
  P.I = a.I;
  P.gscale = a.gscale;
  P.alpha = a.alpha; P.beta = a.beta; P.limit = a.limit;
  P.z = a.z;
  P.lora_B = (const uint16_t*)a.lora_B;
  P.lora_rank = a.lora_rank;
  P.lora_groups = a.lora_groups;
  P.lora_scale = a.lora_scale;
  P.h = (uint8_t*)a.h;
  P.hs = a.hs;
  long hint = a.G > 0 ? a.p_cap / a.G : a.p_cap;
  return dispatch<true>(a.fmt, P, a.p_cap, a.I / 128, hint, s);
}

hipError_t launch_gemm2(const Gemm2Args& a, hipStream_t s) {
  GemmParams P{};
  P.a = (const uint8_t*)a.h;
  P.as = a.hs;
  P.a_ld = (long)a.I * (a.fmt == FMT_FP8 ? 1 : 2);
  P.w = (const uint8_t*)a.wq;
  P.wsc = a.ws;
  P.N = a.H;
  P.K = a.I;
  P.G = a.G;
  P.offsets = a.offsets;
  P.I = a.I;
  P.y = a.y;
  long hint = a.G > 0 ? a.p_cap / a.G : a.p_cap;
  return dispatch<false>(a.fmt, P, a.p_cap, (a.H + 255) / 256, hint, s);
}

}  // namespace moe
