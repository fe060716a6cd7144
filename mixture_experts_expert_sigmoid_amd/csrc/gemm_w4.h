// Grouped GEMM for 4-bit expert weights: GEMM1 over [gate | up] with the
// parameterized SwiGLU epilogue writing bf16 h, and GEMM2 (down) writing
// fp32 rows for the weighted combine. One kernel family, templated on the
// weight format WF:
//
//   INT4 group-32 ("sm100: Fused INT4 grouped + SiLU Triton kernel",
//   batchgen PR #239, commit text): w[n][k] = (nibble - 8) * scale[n][k / 32]
//   with a bf16 scale;
//   NVFP4 (the weight format of the MoE-LoRA release, "FlashInfer 0.6.18
//   SM100a+SM103a MoE-LoRA AOT" release notes, "Changes since 1b699bf"):
//   w[n][k] = e2m1(code) * e4m3(scale[n][k / 16]) * global scale, the global
//   scale per expert and (W13) per half;
//   MXFP4: w[n][k] = e2m1(code) * 2^(scale[n][k / 32] - 127).
// Byte j of a weight row holds k = 2j in its low nibble and k = 2j + 1 in
// its high nibble; activations are bf16, accumulation fp32.
//
// Arithmetic: each nibble is expanded in registers to an exact f16 value
// and the products with f16 activations are formed on
// v_mfma_f32_16x16x32_f16, accumulated in fp32 across the whole K; no
// per-block scaling step is needed (the block scale is inside the operand).
//   INT4: an AND-OR with 0x6400 places a nibble n in the mantissa of
//   1024 + n (or 1024 + 16 n for the second nibble of a byte), one f16
//   subtraction leaves n - 8 (or 16 (n - 8)) exactly, and one f16
//   multiplication by the scale (or scale / 16) is exact because n - 8 has
//   at most 3 significant bits and a bf16 scale 8: the product fits f16's
//   11 for |scale| in [2^-13, 2^13) (scale / 16 stays on f16's 2^-24 grid,
//   8 |scale| below its 65504).
//   FP4: the three magnitude bits of a code go to f16 bits 11..9 and its
//   sign to bit 15, which is exactly e2m1 * 2^-14 (the e2m1 subnormal 0.5
//   lands on the f16 subnormal 2^-15); one f16 multiplication by the block
//   scale (NVFP4: e4m3 * 2^7, read from the code's bits as e4m3 * 2^-8 and
//   multiplied by 2^15; MXFP4: 2^(e - 113)) is exact, since e2m1 * e4m3
//   has at most 6 significant bits and every product lies in f16's range
//   on a grid of 2^-24 or coarser (MXFP4: for exponents 104..128). The
//   NVFP4 accumulator is multiplied by 2^7 (and W2's by its global scale)
//   after the K loop; W13's global scales are applied in the epilogue.
//   Scales outside those ranges (INT4 and MXFP4 as stated, NVFP4's NaN
//   codes) and bf16 activations beyond f16's 65504 are checked as they are
//   used and reported in the error word; the kernels then still run (with
//   MXFP4 exponents clamped to 99..128), but those outputs are not valid.
//
// K order: the expansion of one dword (k0..k7 of a 32-K group) yields the
// f16 values in the order k0, k4, k1, k5, k2, k6, k3, k7; the activations
// are laid out with the same permutation of each 8 (by the f16 conversion
// pass for GEMM1, while staging for GEMM2), so the dot products are
// unchanged.
//
// Work split as in the FP8 kernel: 8 waves own BM rows of one expert and
// 256 weight rows in two halves (GEMM1: 128 gate + the matching 128 up
// rows; GEMM2: 256 output columns); wave w computes all BM rows of columns
// 16w..16w+15 of both halves, weights go HBM -> registers (two 128-K blocks
// in flight, 16 bytes per row and lane per block) and are expanded there;
// the f16 activation block is staged in LDS (a ring of four stages).
#pragma once
#include "act16_dev.h"
#include "gemm_common.h"

namespace moe {

// Activation blocks in a ring of four LDS stages, staged two blocks ahead,
// with a barrier after every second block (as in the FP8 kernel)
constexpr int kW4Stages = 4;

template <int BM>
struct I4Geo {
  static constexpr int MS = BM / 16;              // 16-row subtiles
  static constexpr int A_BYTES = BM * 256;        // one K block, f16
  static constexpr int A_CH = BM * 16;            // 16-byte chunks
  static constexpr int A_PT = (A_CH + kThreads - 1) / kThreads;
  static constexpr int STAGE = A_BYTES;
  static constexpr int LDS = kW4Stages * STAGE;
};

// f16 A rows are 256 bytes; chunk c of row r is stored at c ^ (r & 0b1011),
// conflict-free for the fragment reads and the row-wise stores (the FP8
// kernel's bf16 layout)
__device__ __forceinline__ int i4_swz(int row, int c) { return c ^ (row & 11); }

__device__ __forceinline__ f16x2 h2_bits(uint32_t u) { return __builtin_bit_cast(f16x2, u); }

// (a & m) | c in one v_and_or_b32 (m uniform: one scalar operand per VOP3)
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(m), "v"(c));
  return r;
}

// one dword of nibbles (k0..k7, low nibble first) -> the 8 exact f16 values
// (n - 8) * s in the order k0, k4, k1, k5, k2, k6, k3, k7; s2 = (s, s),
// s16 = (s / 16, s / 16)
__device__ __forceinline__ f16x8 int4x8_f16(uint32_t w, f16x2 s2, f16x2 s16) {
  const uint32_t w8 = w >> 8;
  const f16x2 b1032 = h2_bits(0x64086408u), b1152 = h2_bits(0x64806480u);   // 1032, 1152
  const f16x2 a = (h2_bits(and_or(w, 0x000F000Fu, 0x64006400u)) - b1032) * s2;
  const f16x2 b = (h2_bits(and_or(w, 0x00F000F0u, 0x64006400u)) - b1152) * s16;
  const f16x2 c = (h2_bits(and_or(w8, 0x000F000Fu, 0x64006400u)) - b1032) * s2;
  const f16x2 d = (h2_bits(and_or(w8, 0x00F000F0u, 0x64006400u)) - b1152) * s16;
  return (f16x8){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// one dword of e2m1 codes (k0..k7, low nibble first) -> the 8 exact f16
// values e2m1 * 2^-14 * s in the order k0, k4, k1, k5, k2, k6, k3, k7: for
// the codes of k_j and k_j+4 (bits 4j..4j+3 and 4j+16..4j+19) the magnitude
// bits move to 11..9 (and 27..25) and the sign bit to 15 (and 31)
__device__ __forceinline__ f16x8 fp4x8_f16(uint32_t w, f16x2 s) {
  const uint32_t M = 0x0E000E00u, S = 0x80008000u;
  const f16x2 a = h2_bits(and_or(w << 9, M, (w << 12) & S)) * s;
  const f16x2 b = h2_bits(and_or(w << 5, M, (w << 8) & S)) * s;
  const f16x2 c = h2_bits(and_or(w << 1, M, (w << 4) & S)) * s;
  const f16x2 d = h2_bits(and_or(w >> 3, M, w & S)) * s;
  return (f16x8){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Per-format pieces. A lane's 16 weight bytes per row and 128-K block hold
// K 32 lg .. 32 lg + 31 of the block (block sb): INT4 and MXFP4 have one
// scale for them (index 4 sb + lg of the row's K / 32), NVFP4 two (indices
// 8 sb + 2 lg and + 1 of the row's K / 16, read as one 16-bit word).
template <int WF>
struct W4 {
  // expansion VALU instructions per dword, for the scheduler hints
  static constexpr int kValuPerItem = WF == FMT_INT4 ? 15 : 21;
  // the accumulator's factor after the K loop (NVFP4 scales carry 2^7)
  static constexpr float kPost = WF == FMT_NVFP4 ? 128.0f : 1.0f;
  // scale bytes per weight row (INT4: K / 32 bf16; NVFP4: K / 16 e4m3;
  // MXFP4: K / 32 e8m0) and per 128-K block
  static constexpr int kRowDiv = WF == FMT_MXFP4 ? 32 : 16;
  static constexpr int kBlockBytes = WF == FMT_MXFP4 ? 4 : 8;
  // the first scale byte of lane group lg in row n of group g
  __device__ static const uint8_t* lane_ptr(const GemmParams& P, int g, long n, int lg) {
    return (const uint8_t*)P.wsc + ((long)g * P.N + n) * (P.K / kRowDiv) +
           lg * (kBlockBytes / 4);
  }
  // the lane's scale word of block sb (one bf16, two e4m3 or one e8m0)
  __device__ static uint32_t load(const uint8_t* p, int sb) {
    if constexpr (WF == FMT_MXFP4) return p[kBlockBytes * sb];
    else return *(const uint16_t*)(p + kBlockBytes * sb);
  }
  // operand scales: x for the first 16 K of the lane's 32, y for the second
  // (INT4: x = s, y = s / 16 for both halves, see int4x8_f16)
  __device__ static void regs(uint32_t sw, f16x2& x, f16x2& y) {
    if constexpr (WF == FMT_INT4) {
      const _Float16 sh = (_Float16)bf16_bits_to_f32(sw);
      x = (f16x2){sh, sh};
      y = x * (f16x2){(_Float16)0.0625f, (_Float16)0.0625f};
    } else if constexpr (WF == FMT_NVFP4) {
      // e4m3 code c as f16 bits (c & 0x7F) << 7 with its sign at bit 15 is
      // e4m3(c) * 2^-8 (normal and subnormal codes alike); times 2^15
      const f16x2 k = (f16x2){(_Float16)32768.0f, (_Float16)32768.0f};
      const uint32_t lo = ((sw & 0x7Fu) << 7) | ((sw & 0x80u) << 8);
      const uint32_t hi = ((sw & 0x7F00u) >> 1) | (sw & 0x8000u);
      x = h2_bits(lo | (lo << 16)) * k;
      y = h2_bits(hi | (hi << 16)) * k;
    } else {
      // 2^(e - 113) as f16 bits (e - 98) << 10; exponents outside 99..128
      // are clamped (the format's exact range here is 104..128)
      const uint32_t e = min(max(sw, 99u), 128u);
      const uint32_t b = (e - 98u) << 10;
      x = h2_bits(b | (b << 16));
      y = x;
    }
  }
  // a scale word whose products would not expand exactly to f16: INT4 a
  // bf16 |s| outside [2^-13, 2^13) other than zero, NVFP4 a NaN e4m3 code,
  // MXFP4 an exponent outside 104..128
  __device__ static bool scale_bad(uint32_t sw) {
    if constexpr (WF == FMT_INT4) {
      const uint32_t a = sw & 0x7FFFu;
      return a != 0u && (a < 0x3900u || a >= 0x4600u);
    } else if constexpr (WF == FMT_NVFP4) {
      return (sw & 0x7Fu) == 0x7Fu || (sw & 0x7F00u) == 0x7F00u;
    } else {
      return sw - 104u > 24u;
    }
  }
  __device__ static f16x8 expand(uint32_t w, f16x2 x, f16x2 y, bool second) {
    if constexpr (WF == FMT_INT4) return int4x8_f16(w, x, y);
    else return fp4x8_f16(w, second ? y : x);
  }
};

// Accumulator layout: acc[ms][ns][r] is activation row 16 ms + (lane % 16)
// and weight column (ns ? hi : lo) + 16 wave + 4 (lane / 16) + r.
template <int BM, bool G1, bool LORA>
__device__ __forceinline__ void w4_epilogue(const GemmParams& P, const Tile& t,
                                              f32x4 (&acc)[BM / 16][2], uint8_t* smem) {
  constexpr int MS = BM / 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int c0 = 16 * wave + 4 * lg;
  const int g = t.g, row0 = t.row0, m = t.m;
  if constexpr (!G1) {
    const bool hi_ok = t.n_hi != t.n_lo;
    if constexpr (LORA)
      if (P.z && g < P.lora_groups) lora_delta_tile<BM>(P, t, acc, smem, hi_ok);   // down LoRA
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
      const int tr = 16 * ms + lr;
      store_y16(P, row0 + tr, t.n_lo + c0, acc[ms][0], tr < m);
      if (hi_ok) store_y16(P, row0 + tr, t.n_hi + c0, acc[ms][1], tr < m);
    }
  } else {
    if (P.gscale) {
      const float gsg = P.gscale[2 * g], gsu = P.gscale[2 * g + 1];
#pragma unroll
      for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          acc[ms][0][r] *= gsg;
          acc[ms][1][r] *= gsu;
        }
    }
    if constexpr (LORA)
      if (P.z && g < P.lora_groups) lora_delta_tile<BM>(P, t, acc, smem, true);
    const float L = P.limit, al = P.alpha, be = P.beta;
    uint16_t* h = (uint16_t*)P.h;
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
      const int tr = 16 * ms + lr;
      uint32_t hb[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float gg = fminf(acc[ms][0][r], L);
        const float uu = fminf(fmaxf(acc[ms][1][r], -L), L);
        const float sg = __builtin_amdgcn_rcpf(1.0f + expf(-al * gg));
        hb[r] = f32_to_bf16_bits(gg * sg * (uu + be));
      }
      if (tr < m)         // 4 consecutive h columns
        *(uint2*)(h + (long)(row0 + tr) * P.I + t.nt * 128 + c0) =
            (uint2){hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16)};
    }
  }
}

// One tile of BM rows over K blocks [k0, k1) (see the FP8 kernel for the
// pipeline); PART: fp32 sums to partial slot `slot` (split-K).
template <int WF, int BM, bool G1, bool PART, bool LORA>
__device__ __forceinline__ void w4_tile(const GemmParams& P, const Tile& tl, uint8_t* smem,
                                          int k0, int k1, int slot = 0) {
  using Gm = I4Geo<BM>;
  constexpr int MS = Gm::MS;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int K = P.K;
  const int g = tl.g, row0 = tl.row0, m = tl.m;

  // ---- sources at K block 0 ----------------------------------------------
  // A: 256 bytes (128 f16 or bf16) per row and block, 16 chunks of 16
  const uint8_t* ap[Gm::A_PT];
  int a_st[Gm::A_PT];
#pragma unroll
  for (int i = 0; i < Gm::A_PT; ++i) {
    const int cc = min(tid + i * kThreads, Gm::A_CH - 1);
    const int row = cc >> 4, ch = cc & 15;
    ap[i] = P.a + a_source_row<G1>(P, row0 + (row < m ? row : 0)) * P.a_ld + ch * 16;
    a_st[i] = row * 256 + 16 * i4_swz(row, ch);
  }
  // weights: K / 2 bytes per row, 64 per block; this lane's 16 bytes hold
  // K 32 lg .. 32 lg + 31 of the block
  using F = W4<WF>;
  const long wrow = K >> 1;
  const uint8_t* wg = P.w + (long)g * P.N * wrow;
  const long nl = tl.n_lo + 16 * wave + lr, nh = tl.n_hi + 16 * wave + lr;
  const uint8_t* bp0 = wg + nl * wrow + 16 * lg;
  const uint8_t* bp1 = wg + nh * wrow + 16 * lg;
  const uint8_t* sp0 = F::lane_ptr(P, g, nl, lg);
  const uint8_t* sp1 = F::lane_ptr(P, g, nh, lg);

  i32x4 ra[Gm::A_PT];
  // range problems met by the wave (ballot masks, uniform): scales, h
  uint64_t bad_s = 0, bad_h = 0;
  auto gload_a = [&](int s) {            // past the last block: re-read it
    const long adv = (long)min(s, k1 - 1) * 256;
#pragma unroll
    for (int i = 0; i < Gm::A_PT; ++i) ra[i] = *(const i32x4*)(ap[i] + adv);
  };
  auto store_a = [&](int buf) {
    uint8_t* st = smem + buf * Gm::STAGE;
#pragma unroll
    for (int i = 0; i < Gm::A_PT; ++i) {
      if (Gm::A_CH % kThreads == 0 || tid + i * kThreads < Gm::A_CH) {
        if constexpr (G1)                // already f16 in the K order above
          *(i32x4*)(st + a_st[i]) = ra[i];
        else {                           // h: bf16 -> f16, reordered
          *(f16x8*)(st + a_st[i]) = bf16x8_f16p(ra[i]);
          bad_h |= __builtin_amdgcn_ballot_w64(bf16x8_f16_overflow(ra[i]));
        }
      }
    }
  };
  struct WB {
    i32x4 q[2];                          // lo, hi rows
    uint32_t s[2];                       // their scale words
  };
  auto gload_b = [&](WB& b, int s) {   // past the last block: re-read it
    const int sb = min(s, k1 - 1);
    b.q[0] = *(const i32x4*)(bp0 + (long)sb * 64);
    b.q[1] = *(const i32x4*)(bp1 + (long)sb * 64);
    b.s[0] = F::load(sp0, sb);
    b.s[1] = F::load(sp1, sb);
  };

  f32x4 acc[MS][2];
#pragma unroll
  for (int i = 0; i < MS; ++i) {
    acc[i][0] = (f32x4){0.f, 0.f, 0.f, 0.f};
    acc[i][1] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }

  // The weight expansion is pipelined: each block is done in two K halves
  // (32-deep steps j = 0, 1, then j = 2, 3); the MFMAs of the first half run
  // while the second half's weights are expanded, and those of the second
  // half while the next block's first half is expanded, the conversions
  // spread over the subtiles between the MFMAs.
  f16x8 bwA[2][2], bwB[2][2];            // [ns][j] of the first / second half
  auto scale_regs = [&](const WB& b, f16x2 (&sx)[2], f16x2 (&sy)[2]) {
    bad_s |= __builtin_amdgcn_ballot_w64(F::scale_bad(b.s[0]) || F::scale_bad(b.s[1]));
#pragma unroll
    for (int ns = 0; ns < 2; ++ns) F::regs(b.s[ns], sx[ns], sy[ns]);
  };
  auto block = [&](int s, int buf, WB& rc, WB& rn) {
#pragma unroll
    for (int i = 0; i < 2; ++i) asm volatile("" : "+v"(rc.q[i]), "+v"(rn.q[i]));
    f16x2 s2[2], s16[2], s2n[2], s16n[2];
    scale_regs(rc, s2, s16);
    scale_regs(rn, s2n, s16n);
    gload_a(s + 2);
    const uint8_t* sa = smem + buf * Gm::STAGE;
    // A fragment of step t = (half h, subtile ms): chunks 4 lg + 2 h, + 1
    auto lds_h = [&](int t, f16x8 (&af)[2]) {
      const int h = t / MS, row = 16 * (t % MS) + lr;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        af[jj] = *(const f16x8*)(sa + row * 256 + 16 * i4_swz(row, 4 * lg + 2 * h + jj));
    };
    f16x8 fr[2][2];
    lds_h(0, fr[0]);
#pragma unroll
    for (int t = 0; t < 2 * MS; ++t) {
      const int h = t / MS, ms = t % MS;
      if (t + 1 < 2 * MS) lds_h(t + 1, fr[(t + 1) & 1]);
      if (t == MS) gload_b(rc, s + 2);   // this block's raw weights are expanded
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        acc[ms][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(h ? bwB[0][jj] : bwA[0][jj],
                                                           fr[t & 1][jj], acc[ms][0], 0, 0, 0);
        acc[ms][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(h ? bwB[1][jj] : bwA[1][jj],
                                                           fr[t & 1][jj], acc[ms][1], 0, 0, 0);
      }
      // expansion items (ns, jj) of this step: item i goes to subtile i*MS/4
      int nitem = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i * MS / 4 == ms) {
          const int ns = i >> 1, jj = i & 1;
          if (h == 0)
            bwB[ns][jj] = F::expand((uint32_t)rc.q[ns][2 + jj], s2[ns], s16[ns], true);
          else
            bwA[ns][jj] = F::expand((uint32_t)rn.q[ns][jj], s2n[ns], s16n[ns], false);
          ++nitem;
        }
      }
      if (t + 1 < 2 * MS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // DS read
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                      // MFMA
        if (q < 3) {                                                          // VALU
          if (nitem == 1) __builtin_amdgcn_sched_group_barrier(0x002, F::kValuPerItem / 3, 0);
          if (nitem == 2) __builtin_amdgcn_sched_group_barrier(0x002, 2 * F::kValuPerItem / 3, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    store_a((buf + 2) & (kW4Stages - 1));   // block s + 2
  };

  WB rb0, rb1;
  gload_b(rb0, k0);
  gload_b(rb1, k0 + 1);
  gload_a(k0);
  store_a(0);
  gload_a(k0 + 1);
  store_a(1);
  {                                      // first half of block k0
    f16x2 s2[2], s16[2];
    scale_regs(rb0, s2, s16);
#pragma unroll
    for (int ns = 0; ns < 2; ++ns)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        bwA[ns][jj] = F::expand((uint32_t)rb0.q[ns][jj], s2[ns], s16[ns], false);
  }
  __syncthreads();
  // block i = s - k0 reads stage i % 4 (staged in block i - 2) and stages
  // block i + 2 into the stage of block i - 2; the barrier after each pair
  // orders both (see the FP8 kernel)
  int s = k0;
  for (; s + 2 <= k1; s += 2) {
    const int i = s - k0;
    block(s, i & 3, rb0, rb1);
    block(s + 1, (i + 1) & 3, rb1, rb0);
    __syncthreads();
  }
  if (s < k1) {
    block(s, (s - k0) & 3, rb0, rb1);
    __syncthreads();
  }
  if ((bad_s | bad_h) && P.err && lane == 0)
    atomicOr(P.err, (bad_s ? MOE_DEVERR_BIT_W4_SCALE : 0) | (bad_h ? MOE_DEVERR_BIT_F16_RANGE : 0));
  if constexpr (WF != FMT_INT4) {
    // NVFP4's 2^7 and, for W2, the expert's global scale (before the LoRA
    // delta, which is in true units)
    float f = F::kPost;
    if constexpr (!G1)
      if (P.gscale) f *= P.gscale[g];
    if (f != 1.0f) {
#pragma unroll
      for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          acc[ms][0][r] *= f;
          acc[ms][1][r] *= f;
        }
    }
  }
  if constexpr (PART) {
    const int c0 = 16 * wave + 4 * lg;
    const bool hi_ok = G1 || tl.n_hi != tl.n_lo;
    // GEMM2's down-LoRA delta goes into the tile's first partial slot once
    if constexpr (!G1 && LORA)
      if (slot == 0 && P.z && tl.g < P.lora_groups)
        lora_delta_tile<BM>(P, tl, acc, smem, hi_ok);
    float* base = P.part + ((long)slot * P.p_rows + row0) * P.N;
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
      const int tr = 16 * ms + lr;
      if (tr < m) {
        *(f32x4*)(base + (long)tr * P.N + tl.n_lo + c0) = acc[ms][0];
        if (hi_ok) *(f32x4*)(base + (long)tr * P.N + tl.n_hi + c0) = acc[ms][1];
      }
    }
  } else {
    w4_epilogue<BM, G1, LORA>(P, tl, acc, smem);
    __syncthreads();       // LDS is reused by the next tile
  }
}

template <int WF, int TBM, bool G1, bool LORA>
__device__ __forceinline__ void w4_plain_tiles(const GemmParams& P, uint8_t* smem,
                                                 const int* s_cum) {
  const int NT = G1 ? (P.I >> 7) : ((P.N + 255) >> 8);
  const int NS = P.K >> 7;
  const int total = s_cum[P.G] * NT;
  const int xcd = blockIdx.x & 7, nper = gridDim.x >> 3, slot = blockIdx.x >> 3;
  const int chunk = (total + 7) >> 3;
  const int t_end = min(total, (xcd + 1) * chunk);
  for (int lt = xcd * chunk + slot; lt < t_end; lt += nper) {
    Tile tl = decode_tile<TBM, G1>(P, lt, NT, s_cum);
    tl.g = __builtin_amdgcn_readfirstlane(tl.g);
    tl.row0 = __builtin_amdgcn_readfirstlane(tl.row0);
    tl.m = __builtin_amdgcn_readfirstlane(tl.m);
    tl.nt = __builtin_amdgcn_readfirstlane(tl.nt);
    tl.n_lo = __builtin_amdgcn_readfirstlane(tl.n_lo);
    tl.n_hi = __builtin_amdgcn_readfirstlane(tl.n_hi);
    if constexpr (TBM >= 128) {
      if (tl.m > 64) { w4_tile<WF, 128, G1, false, LORA>(P, tl, smem, 0, NS); continue; }
    }
    if constexpr (TBM >= 64) {
      if (tl.m > 32) { w4_tile<WF, 64, G1, false, LORA>(P, tl, smem, 0, NS); continue; }
    }
    w4_tile<WF, 32, G1, false, LORA>(P, tl, smem, 0, NS);
  }
}

template <int WF, int TBM, bool G1, bool LORA>
__global__ __launch_bounds__(kThreads) void moe_gemm_w4_kernel(GemmParams P) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int s_cum[kMaxGroups + 1];
  __shared__ int s_wsum[8];
  // SK_DEVICE launch: return if the split-K kernel takes this GEMM
  if (P.sk_mode == SK_DEVICE &&
      sk_rule(tiles32(P.offsets, P.G, s_cum) * (G1 ? (P.I >> 7) : ((P.N + 255) >> 8)),
              P.K >> 7))
    return;
  tile_prefix<TBM>(P.offsets, P.G, s_cum, s_wsum);
  w4_plain_tiles<WF, TBM, G1, LORA>(P, smem, s_cum);
}

// Split-K (stream-K) variant, schedule as in the FP8 kernel
template <int WF, bool G1, bool LORA>
__global__ __launch_bounds__(kThreads) void moe_gemm_w4_sk_kernel(GemmParams P) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int s_cum[kMaxGroups + 1];
  __shared__ int s_wsum[8];
  const int G = P.G;
  const int NT = G1 ? (P.I >> 7) : ((P.N + 255) >> 8);
  const int NS = P.K >> 7;
  tile_prefix<kSkBM>(P.offsets, G, s_cum, s_wsum);
  if (P.sk_mode == SK_DEVICE && !sk_rule((long)s_cum[G] * NT, NS)) {
    // whole tiles here, as the plain kernel's 32-row class would run them
    // (GEMM1 of INT4 and MXFP4; NVFP4's split-K kernel would lose its
    // second workgroup per CU to the extra registers, so its plain kernel
    // is launched beside it and takes this case)
    if constexpr (G1 && WF != FMT_NVFP4) w4_plain_tiles<WF, kSkBM, G1, LORA>(P, smem, s_cum);
    return;
  }
  const long U = (long)s_cum[G] * NT * NS;
  const int W = sk_workgroups((long)s_cum[G] * NT, NS, gridDim.x);
  const int b = blockIdx.x;
  if (b >= W) return;
  const long u1 = (long)(b + 1) * U / W;
  for (long u = (long)b * U / W; u < u1;) {
    const int t = (int)(u / NS);
    const int k0 = (int)(u - (long)t * NS);
    const int k1 = (int)std::min<long>(NS, k0 + (u1 - u));
    Tile tl = decode_tile<kSkBM, G1>(P, t, NT, s_cum);
    tl.g = __builtin_amdgcn_readfirstlane(tl.g);
    tl.row0 = __builtin_amdgcn_readfirstlane(tl.row0);
    tl.m = __builtin_amdgcn_readfirstlane(tl.m);
    tl.nt = __builtin_amdgcn_readfirstlane(tl.nt);
    tl.n_lo = __builtin_amdgcn_readfirstlane(tl.n_lo);
    tl.n_hi = __builtin_amdgcn_readfirstlane(tl.n_hi);
    const int slot = b - sk_owner((long)t * NS, U, W);
    w4_tile<WF, kSkBM, G1, true, LORA>(P, tl, smem, k0, k1, slot);
    u += k1 - k0;
  }
}

template <int WF, int TBM, bool G1, bool LORA>
static hipError_t run_w4(const GemmParams& P, long p_cap, int NT, hipStream_t s) {
  constexpr int shm = LORA ? std::max(I4Geo<TBM>::LDS, kLoraLds) : I4Geo<TBM>::LDS;
  static int per_cu = 0;
  if (per_cu == 0) {
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&moe_gemm_w4_kernel<WF, TBM, G1, LORA>),
        hipFuncAttributeMaxDynamicSharedMemorySize, shm);
    if (e != hipSuccess) return e;
    int nb = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &nb, reinterpret_cast<const void*>(&moe_gemm_w4_kernel<WF, TBM, G1, LORA>), kThreads, shm);
    if (e != hipSuccess) return e;
    per_cu = nb > 0 ? nb : 1;
  }
  long max_tiles = ((p_cap + TBM - 1) / TBM + P.G) * (long)NT;
  long nwg = std::min<long>(max_tiles, (long)num_cus() * per_cu);
  nwg = (nwg + 7) & ~7L;
  if (nwg == 0) return hipSuccess;
  GemmParams Q = P;
  Q.lds_bytes = shm;
  moe_gemm_w4_kernel<WF, TBM, G1, LORA><<<dim3((unsigned)nwg), dim3(kThreads), shm, s>>>(Q);
  return hipGetLastError();
}

template <int WF, bool G1, bool LORA>
static hipError_t run_w4_sk(const GemmParams& P, long p_cap, hipStream_t s, int* sk_grid) {
  constexpr int shm = LORA ? std::max(I4Geo<kSkBM>::LDS, kLoraLds) : I4Geo<kSkBM>::LDS;
  static int per_cu = 0;
  if (per_cu == 0) {
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&moe_gemm_w4_sk_kernel<WF, G1, LORA>),
        hipFuncAttributeMaxDynamicSharedMemorySize, shm);
    if (e != hipSuccess) return e;
    int nb = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &nb, reinterpret_cast<const void*>(&moe_gemm_w4_sk_kernel<WF, G1, LORA>), kThreads, shm);
    if (e != hipSuccess) return e;
    per_cu = nb > 0 ? nb : 1;
  }
  // a multiple of 8: the whole-tile walk of an SK_DEVICE launch splits
  // the grid over the 8 XCDs
  const int grid = std::max(8, (num_cus() * per_cu) & ~7);
  *sk_grid = grid;
  if (p_cap == 0) return hipSuccess;
  GemmParams Q = P;
  Q.lds_bytes = shm;
  moe_gemm_w4_sk_kernel<WF, G1, LORA><<<dim3((unsigned)grid), dim3(kThreads), shm, s>>>(Q);
  return hipGetLastError();
}

template <int WF, bool G1, bool LORA>
static hipError_t run_w4_tbm(const GemmParams& P, long p_cap, int NT, hipStream_t s) {
  const long hint = P.G > 0 ? p_cap / P.G : p_cap;
  if (hint <= 32) return run_w4<WF, 32, G1, LORA>(P, p_cap, NT, s);
  if (hint <= 64) return run_w4<WF, 64, G1, LORA>(P, p_cap, NT, s);
  return run_w4<WF, 128, G1, LORA>(P, p_cap, NT, s);
}

template <int WF, bool LORA>
static hipError_t launch_w4(const GemmParams& P, bool g1, long p_cap, int NT, hipStream_t s,
                            int* sk_grid) {
  if (P.part)
    return g1 ? run_w4_sk<WF, true, LORA>(P, p_cap, s, sk_grid)
              : run_w4_sk<WF, false, LORA>(P, p_cap, s, sk_grid);
  return g1 ? run_w4_tbm<WF, true, LORA>(P, p_cap, NT, s)
            : run_w4_tbm<WF, false, LORA>(P, p_cap, NT, s);
}

// layers with a LoRA run the instantiations that carry the delta
template <int WF>
static hipError_t launch_w4_fmt(const GemmParams& P, bool g1, long p_cap, int NT, hipStream_t s,
                                int* sk_grid) {
  return P.z ? launch_w4<WF, true>(P, g1, p_cap, NT, s, sk_grid)
             : launch_w4<WF, false>(P, g1, p_cap, NT, s, sk_grid);
}

}  // namespace moe
