// Grouped expert GEMMs on CDNA4 MFMA: GEMM1 over the fused [gate | up]
// weight with the parameterized-SwiGLU epilogue (plus optional per-half
// global scales, LoRA delta and FP8 re-quantisation of h), and GEMM2 (down)
// writing fp32 rows for the weighted combine.
//
// Formats:
//   FP8  blockwise 128x128 e4m3 weights and per-token per-128-column e4m3
//        activations ("[Moe] Fix flashinfer_trtllm silently dropping
//        swiglu_limit clamped SwiGLU activation", sglang PR #39920,
//        "Modifications": DeepSeekFp8). One 128-deep K step is exactly one
//        scale block, so each v_mfma_f32_16x16x128_f8f6f4 result is a block
//        partial sum that is scaled by xs[row][kb] * ws[nb][kb] and added.
//   INT4 group-32 weights, byte = (odd k nibble << 4) | even k nibble,
//        w = (nibble - 8) * scale[n][k/32] ("sm100: Fused INT4 grouped +
//        SiLU Triton kernel", batchgen PR #239, commit text). Nibbles are
//        unpacked in registers into fp16: 0x6400 | nibble is 1024 + nibble,
//        minus 1032 gives nibble - 8, times the bf16 scale. Both steps are
//        exact in fp16 (at most 11 significant bits), so the weights enter
//        v_mfma_f32_16x16x32_f16 without rounding; bf16 activations are
//        converted to fp16 on their way into LDS.
//   BF16 weights and activations on v_mfma_f32_16x16x32_bf16.
// Epilogue: g' = min(g, L), u' = clamp(u, -L, L), h = g' sigmoid(alpha g')
// (u' + beta) (sglang PR #39920 "Modifications"; "fix(sm90): support
// parameterized SwiGLU in FP8 MegaMoE", DeepGEMM PR #445, "Summary"). The
// LoRA delta and the per-half global scales follow the true-units rule of
// "FlashInfer 0.6.18 SM100a+SM103a MoE-LoRA AOT" ("Changes since 1b699bf"):
// each half is scaled by its own global scale first, then the delta is added.
//
// Tiling: a workgroup of 8 waves owns BM sorted rows of one expert and 256
// weight rows in two halves of 128 ("lo", "hi"): for GEMM1 lo = gate rows
// n0..n0+127 and hi = the matching up rows I+n0..I+n0+127, so one tile yields
// 128 complete h columns (the FP8 re-quantisation group); for GEMM2 lo/hi are
// output columns n0..n0+255. Wave (wm, wn) computes rows wm*BM/2.. of
// columns wn*32..wn*32+31 of both halves, so gate and up values of the same
// h element sit in the same lane. A and B stream HBM -> registers -> LDS
// (double buffered, one barrier per K step) with 16-byte chunks XOR-swizzled
// by row to spread LDS banks. Workgroup ids are remapped so that consecutive
// tiles of one expert (which share the gathered activation rows) land on the
// same XCD and its L2.
#include "common.h"
#include "launch.h"

namespace moe {

enum { FMT_BF16 = 0, FMT_FP8 = 1, FMT_INT4 = 2 };

constexpr int kThreads = 512;
constexpr int kMaxGroups = 1024;

template <int FMT>
struct FmtTraits;
template <>
struct FmtTraits<FMT_FP8> {
  static constexpr int KSTEP = 128;   // elements per pipeline stage
  static constexpr int AESZ = 1;      // bytes per A element in global memory
  static constexpr int BROW = 128;    // LDS bytes per B row per stage
};
template <>
struct FmtTraits<FMT_BF16> {
  static constexpr int KSTEP = 64;
  static constexpr int AESZ = 2;
  static constexpr int BROW = 128;
};
template <>
struct FmtTraits<FMT_INT4> {
  static constexpr int KSTEP = 64;
  static constexpr int AESZ = 2;
  static constexpr int BROW = 48;     // 32 packed bytes, padded
};

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 7); }

__device__ __forceinline__ f32x4 mfma_fp8(const i32x8& a, const i32x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// 8 bf16 (as 4 dwords) -> 8 fp16, exact for |v| in [2^-14, 65504]
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

// 8 packed nibbles (k = 0..7 of one row, low nibble first) -> 8 fp16 values
// (nibble - 8) * scale, exact.
__device__ __forceinline__ f16x8 int4x8_to_f16x8(uint32_t w, f16x2 sc2) {
  uint32_t lo = w & 0x0F0F0F0Fu;          // k even nibbles in bytes 0..3
  uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;   // k odd nibbles
  f16x8 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t pr = ((lo >> (8 * i)) & 0xFFu) | (((hi >> (8 * i)) & 0xFFu) << 16);
    pr |= 0x64006400u;                     // (1024 + n_even, 1024 + n_odd)
    f16x2 v = __builtin_bit_cast(f16x2, pr);
    v = (v - (f16x2){(_Float16)1032.0f, (_Float16)1032.0f}) * sc2;
    out[2 * i] = v[0];
    out[2 * i + 1] = v[1];
  }
  return out;
}

// 8 e4m3fn codes (k order, little-endian in two dwords) -> 8 bf16, exact:
// the hardware converts to fp32 and every e4m3 value has at most 4
// significant bits, so the upper half of the fp32 is the bf16 value.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(uint32_t w0, uint32_t w1) {
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
  return __builtin_bit_cast(bf16x8, o);
}

struct GemmParams {
  // A side
  const uint8_t* a;          // x (GEMM1: gathered by token) or h (GEMM2)
  const float* as;           // FP8 per-row scales [rows][K/128]
  long a_ld;                 // bytes per A row
  int gather;                // 1: A row = token of sorted_pair
  const int* sorted_pair;
  long T;
  int top_k;
  // B side
  const uint8_t* w;          // [G][N][K] codes (bytes; INT4 packed)
  const void* wsc;           // FP8 fp32 [G][N/128][K/128]; INT4 bf16 [G][N][K/32]
  int N, K, G;
  long p_cap;
  const int* offsets;
  int gemm1;                 // 1: lo = gate n0.., hi = up I+n0..; 0: lo/hi = n0, n0+128
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
  float* y;                  // [p_cap][H]
};

template <int FMT, int BM>
struct Smem {
  static constexpr int KSTEP = FmtTraits<FMT>::KSTEP;
  static constexpr int A_BYTES = BM * 128;
  static constexpr int B_BYTES = 256 * FmtTraits<FMT>::BROW;
  static constexpr int BS_BYTES = (FMT == FMT_INT4) ? 256 * 4 : 0;
  static constexpr int AS_BYTES = (FMT == FMT_FP8) ? BM * 4 : 0;
  static constexpr int STAGE = A_BYTES + B_BYTES + BS_BYTES + AS_BYTES;
  static constexpr int TOTAL = 2 * STAGE;
};

template <int FMT, int BM, bool G1>
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(GemmParams P) {
  using Tr = FmtTraits<FMT>;
  using S = Smem<FMT, BM>;
  constexpr int KSTEP = Tr::KSTEP;
  constexpr int MS = BM / 32;            // 16-row subtiles per wave
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int s_cum[kMaxGroups + 1];
  __shared__ int s_wsum[8];
  __shared__ int s_tile[3];              // group, m0, m
  __shared__ long s_arow[BM];            // byte offset of each tile row's A data
  __shared__ long s_srow[BM];            // FP8: index of the row's scale row

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int G = P.G;
  const int NT = G1 ? (P.I >> 7) : ((P.N + 255) >> 8);

  // ---- tile id (XCD-aware: consecutive logical tiles share an XCD) -------
  const int nwg = gridDim.x;
  const int bid = blockIdx.x;
  const int lin = (bid & 7) * (nwg >> 3) + (bid >> 3);
  const int mt_global = lin / NT, nt = lin - mt_global * NT;

  // ---- M-tile prefix over groups ----------------------------------------
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
    if (g0 < G && mt_global >= s_cum[g0] && mt_global < s_cum[g0] + c0) {
      s_tile[0] = g0; s_tile[1] = (mt_global - s_cum[g0]) * BM;
    }
    if (g1 < G && mt_global >= s_cum[g1] && mt_global < s_cum[g1] + c1) {
      s_tile[0] = g1; s_tile[1] = (mt_global - s_cum[g1]) * BM;
    }
    __syncthreads();
  }
  if (mt_global >= s_cum[G]) return;     // uniform across the workgroup
  const int g = s_tile[0];
  const int m0 = s_tile[1];
  const int row0 = P.offsets[g] + m0;    // first sorted row of the tile
  const int m = min(BM, P.offsets[g + 1] - row0);

  // ---- A row addresses ----------------------------------------------------
  if (tid < BM) {
    int r = row0 + (tid < m ? tid : 0);
    long src;
    if (P.gather) {
      int p = P.sorted_pair[r];
      long npr = P.T * (long)P.top_k;
      src = (p < npr) ? (long)(p / P.top_k) : (long)(p - npr);
    } else {
      src = r;
    }
    s_arow[tid] = src * P.a_ld;
    s_srow[tid] = src;
  }

  // ---- B (weight) rows ----------------------------------------------------
  const int K = P.K;
  const long wrow_bytes = (FMT == FMT_INT4) ? K / 2 : (long)K * (FMT == FMT_FP8 ? 1 : 2);
  int n_lo, n_hi;
  if (G1) {
    n_lo = nt * 128;
    n_hi = P.I + nt * 128;
  } else {
    n_lo = nt * 256;
    n_hi = (n_lo + 128 < P.N) ? n_lo + 128 : n_lo;   // ragged last tile
  }
  const uint8_t* wg = P.w + (long)g * P.N * wrow_bytes;
  __syncthreads();

  const int nk = K / KSTEP;
  const int nkb128 = K >> 7;

  // ---- global -> register staging ----------------------------------------
  constexpr int A_CHUNKS = BM * 8;                       // 16-byte chunks
  constexpr int A_PER_T = (A_CHUNKS + kThreads - 1) / kThreads;
  constexpr int B_CHUNKS = (FMT == FMT_INT4) ? 256 * 2 : 256 * 8;
  constexpr int B_PER_T = B_CHUNKS / kThreads;
  i32x4 ra[A_PER_T], rb[B_PER_T];
  uint32_t rbs = 0;
  float ras = 0.0f;

  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      int c = tid + i * kThreads;
      if (c < A_CHUNKS) {
        int row = c >> 3, ch = c & 7;
        const uint8_t* src = P.a + s_arow[row] + (long)kt * KSTEP * Tr::AESZ + ch * 16;
        ra[i] = *(const i32x4*)src;
      }
    }
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) {
      int c = tid + i * kThreads;
      int row, ch;
      if (FMT == FMT_INT4) { row = c >> 1; ch = c & 1; }
      else { row = c >> 3; ch = c & 7; }
      int n = (row < 128) ? n_lo + row : n_hi + (row - 128);
      long off = (long)n * wrow_bytes;
      if (FMT == FMT_INT4) off += (long)kt * (KSTEP / 2) + ch * 16;
      else off += (long)kt * KSTEP * (FMT == FMT_FP8 ? 1 : 2) + ch * 16;
      rb[i] = *(const i32x4*)(wg + off);
    }
    if (FMT == FMT_INT4 && tid < 256) {
      int row = tid;
      int n = (row < 128) ? n_lo + row : n_hi + (row - 128);
      const uint16_t* sc = (const uint16_t*)P.wsc + ((long)g * P.N + n) * (K / 32) + kt * 2;
      rbs = *(const uint32_t*)sc;
    }
    if (FMT == FMT_FP8 && tid < BM) ras = P.as[s_srow[tid] * nkb128 + kt];
  };
  auto sstore = [&](int buf) {
    uint8_t* st = smem + buf * S::STAGE;
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      int c = tid + i * kThreads;
      if (c < A_CHUNKS) {
        int row = c >> 3, ch = c & 7;
        i32x4 v = ra[i];
        if (FMT == FMT_INT4) v = bf16x8_to_f16x8(v);
        *(i32x4*)(st + row * 128 + swz(row, ch) * 16) = v;
      }
    }
    uint8_t* sb = st + S::A_BYTES;
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) {
      int c = tid + i * kThreads;
      if (FMT == FMT_INT4) {
        int row = c >> 1, ch = c & 1;
        *(i32x4*)(sb + row * Tr::BROW + ch * 16) = rb[i];
      } else {
        int row = c >> 3, ch = c & 7;
        *(i32x4*)(sb + row * 128 + swz(row, ch) * 16) = rb[i];
      }
    }
    if (FMT == FMT_INT4 && tid < 256) *(uint32_t*)(sb + S::B_BYTES + tid * 4) = rbs;
    if (FMT == FMT_FP8 && tid < BM) *(float*)(sb + S::B_BYTES + tid * 4) = ras;
  };

  // ---- accumulators ---------------------------------------------------------
  f32x4 acc[MS][4];
#pragma unroll
  for (int i = 0; i < MS; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const int rbase = wm * (BM / 2);          // first tile row of this wave
  const int lr = lane & 15, lg = lane >> 4;
  // FP8 block-scale rows (fp32 [N/128][K/128] per group)
  const float* wscale = (FMT == FMT_FP8) ? (const float*)P.wsc + (long)g * (P.N >> 7) * nkb128 : nullptr;
  const int nb_lo = n_lo >> 7, nb_hi = n_hi >> 7;

  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const uint8_t* st = smem + buf * S::STAGE;
    const uint8_t* sb = st + S::A_BYTES;
    if constexpr (FMT == FMT_FP8 && G1) {
      // GEMM1: the h re-quantisation decision needs fp32-exact sums, and the
      // FP8 MFMA accumulates each dot product at reduced internal precision
      // (measured ~2e-5 of sum |products| on gfx950), so the e4m3 codes are
      // expanded exactly to bf16 and multiplied on the BF16 MFMA, whose
      // accumulation of these products is exact. One 128-deep block = four
      // 32-deep MFMAs into a partial accumulator, then scaled once.
      const float* sas = (const float*)(sb + S::B_BYTES);
      f32x4 xsr[MS];
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) xsr[ms] = *(const f32x4*)(sas + rbase + ms * 16 + 4 * lg);
      const float ws_lo = wscale[nb_lo * nkb128 + kt];
      const float ws_hi = wscale[nb_hi * nkb128 + kt];
      f32x4 part[MS][4];
#pragma unroll
      for (int i = 0; i < MS; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) part[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const int chunk = 2 * kc + (lg >> 1), sub = 8 * (lg & 1);
        bf16x8 af[MS];
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) {
          int row = rbase + ms * 16 + lr;
          uint2 v = *(const uint2*)(st + row * 128 + swz(row, chunk) * 16 + sub);
          af[ms] = e4m3x8_to_bf16x8(v.x, v.y);
        }
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) {
          int row = (ns < 2 ? 0 : 128) + wn * 32 + (ns & 1) * 16 + lr;
          uint2 v = *(const uint2*)(sb + row * 128 + swz(row, chunk) * 16 + sub);
          bf16x8 b = e4m3x8_to_bf16x8(v.x, v.y);
#pragma unroll
          for (int ms = 0; ms < MS; ++ms)
            part[ms][ns] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ms], b, part[ms][ns], 0, 0, 0);
        }
      }
#pragma unroll
      for (int ns = 0; ns < 4; ++ns) {
        const float wsv = ns < 2 ? ws_lo : ws_hi;
#pragma unroll
        for (int ms = 0; ms < MS; ++ms)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[ms][ns][r] = fmaf(part[ms][ns][r], xsr[ms][r] * wsv, acc[ms][ns][r]);
      }
    } else if constexpr (FMT == FMT_FP8) {
      i32x8 af[MS];
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) {
        int row = rbase + ms * 16 + lr;
        i32x4 x0 = *(const i32x4*)(st + row * 128 + swz(row, 2 * lg) * 16);
        i32x4 x1 = *(const i32x4*)(st + row * 128 + swz(row, 2 * lg + 1) * 16);
        af[ms] = (i32x8){x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      }
      const float* sas = (const float*)(sb + S::B_BYTES);
      f32x4 xsr[MS];
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) xsr[ms] = *(const f32x4*)(sas + rbase + ms * 16 + 4 * lg);
      const float ws_lo = wscale[nb_lo * nkb128 + kt];
      const float ws_hi = wscale[nb_hi * nkb128 + kt];
#pragma unroll
      for (int ns = 0; ns < 4; ++ns) {
        int row = (ns < 2 ? 0 : 128) + wn * 32 + (ns & 1) * 16 + lr;
        i32x4 y0 = *(const i32x4*)(sb + row * 128 + swz(row, 2 * lg) * 16);
        i32x4 y1 = *(const i32x4*)(sb + row * 128 + swz(row, 2 * lg + 1) * 16);
        i32x8 bf = (i32x8){y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
        const float wsv = ns < 2 ? ws_lo : ws_hi;
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) {
          f32x4 p = mfma_fp8(af[ms], bf, (f32x4){0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[ms][ns][r] = fmaf(p[r], xsr[ms][r] * wsv, acc[ms][ns][r]);
        }
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        i32x4 af[MS];
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) {
          int row = rbase + ms * 16 + lr;
          af[ms] = *(const i32x4*)(st + row * 128 + swz(row, kk * 4 + lg) * 16);
        }
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) {
          int row = (ns < 2 ? 0 : 128) + wn * 32 + (ns & 1) * 16 + lr;
          if constexpr (FMT == FMT_BF16) {
            i32x4 bv = *(const i32x4*)(sb + row * 128 + swz(row, kk * 4 + lg) * 16);
            bf16x8 b = __builtin_bit_cast(bf16x8, bv);
#pragma unroll
            for (int ms = 0; ms < MS; ++ms)
              acc[ms][ns] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(bf16x8, af[ms]), b, acc[ms][ns], 0, 0, 0);
          } else {
            uint32_t wv = *(const uint32_t*)(sb + row * Tr::BROW + kk * 16 + 4 * lg);
            uint32_t sv = *(const uint32_t*)(sb + S::B_BYTES + row * 4);
            uint32_t sbits = kk ? (sv >> 16) : (sv & 0xFFFFu);
            _Float16 sh = (_Float16)bf16_bits_to_f32(sbits);
            f16x8 b = int4x8_to_f16x8(wv, (f16x2){sh, sh});
#pragma unroll
            for (int ms = 0; ms < MS; ++ms)
              acc[ms][ns] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                  __builtin_bit_cast(f16x8, af[ms]), b, acc[ms][ns], 0, 0, 0);
          }
        }
      }
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // ======================= epilogues =======================================
  if constexpr (!G1) {
    // GEMM2: fp32 rows y[row][col]
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

  // GEMM1: gate = ns 0,1 ; up = ns 2,3 (same h columns)
  float gsg = 1.0f, gsu = 1.0f;
  if (P.gscale) { gsg = P.gscale[2 * g]; gsu = P.gscale[2 * g + 1]; }
  float hv[MS][2][4];
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
    // delta[row][n] = s * sum_q z[row][q] * B[g][n][q], gate n = n_lo + c,
    // up n = n_hi + c; z staged in LDS as [q][BM]
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

  // h tile staged in LDS, then written as whole rows
  uint8_t* sh = smem;
  if constexpr (FMT == FMT_FP8) {
    float* s_amax = (float*)(smem + BM * 128);   // [4][BM]
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
        float s = a > 0.0f ? a / 448.0f : 1.0f;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          int c = wn * 32 + j * 16 + lr;
          sh[tr * 128 + c] = (uint8_t)f32_to_e4m3(hv[ms][j][r] / s);
        }
        if (wn == 0 && lr == 0 && tr < m) P.hs[(long)(row0 + tr) * (P.I >> 7) + nt] = s;
      }
    __syncthreads();
    // 128 bytes per row: 8 chunks
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
  }  // GEMM1 epilogue
}

template <int FMT, int BM, bool G1>
static hipError_t run(const GemmParams& P, int NT, hipStream_t s) {
  long max_mt = (P.p_cap + BM - 1) / BM + P.G;
  long nwg = max_mt * NT;
  nwg = (nwg + 7) & ~7L;
  if (nwg == 0) return hipSuccess;
  constexpr int shm = Smem<FMT, BM>::TOTAL;
  static bool attr_set = false;   // per instantiation, first launch
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&grouped_gemm_kernel<FMT, BM, G1>),
        hipFuncAttributeMaxDynamicSharedMemorySize, shm);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  grouped_gemm_kernel<FMT, BM, G1><<<dim3((unsigned)nwg), dim3(kThreads), shm, s>>>(P);
  return hipGetLastError();
}

template <int BM, bool G1>
static hipError_t run_fmt(int fmt, const GemmParams& P, int NT, hipStream_t s) {
  if (fmt == FMT_FP8) return run<FMT_FP8, BM, G1>(P, NT, s);
  if (fmt == FMT_INT4) return run<FMT_INT4, BM, G1>(P, NT, s);
  return run<FMT_BF16, BM, G1>(P, NT, s);
}

template <bool G1>
static hipError_t dispatch(int fmt, const GemmParams& P, int NT, long rows_hint, hipStream_t s) {
  // rows per expert on average decides the M tile
  if (rows_hint <= 32) return run_fmt<32, G1>(fmt, P, NT, s);
  if (rows_hint <= 64) return run_fmt<64, G1>(fmt, P, NT, s);
  return run_fmt<128, G1>(fmt, P, NT, s);
}

hipError_t launch_gemm1(const Gemm1Args& a, hipStream_t s) {
  GemmParams P{};
  P.a = (const uint8_t*)a.x;
  P.as = a.xs;
  P.a_ld = (long)a.H * (a.fmt == FMT_FP8 ? 1 : 2);
  P.gather = 1;
  P.sorted_pair = a.sorted_pair;
  P.T = a.T;
  P.top_k = a.top_k;
  P.w = (const uint8_t*)a.wq;
  P.wsc = a.ws;
  P.N = 2 * a.I;
  P.K = a.H;
  P.G = a.G;
  P.p_cap = a.p_cap;
  P.offsets = a.offsets;
  P.gemm1 = 1;
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
  return dispatch<true>(a.fmt, P, a.I / 128, hint, s);
}

hipError_t launch_gemm2(const Gemm2Args& a, hipStream_t s) {
  GemmParams P{};
  P.a = (const uint8_t*)a.h;
  P.as = a.hs;
  P.a_ld = (long)a.I * (a.fmt == FMT_FP8 ? 1 : 2);
  P.gather = 0;
  P.w = (const uint8_t*)a.wq;
  P.wsc = a.ws;
  P.N = a.H;
  P.K = a.I;
  P.G = a.G;
  P.p_cap = a.p_cap;
  P.offsets = a.offsets;
  P.gemm1 = 0;
  P.I = a.I;
  P.y = a.y;
  long hint = a.G > 0 ? a.p_cap / a.G : a.p_cap;
  return dispatch<false>(a.fmt, P, (a.H + 255) / 256, hint, s);
}

}  // namespace moe
