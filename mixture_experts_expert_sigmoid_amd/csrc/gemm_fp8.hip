// Grouped GEMM for blockwise-FP8 experts: GEMM1 over [gate | up] with the
// SwiGLU epilogue and e4m3 re-quantisation of h, and GEMM2 (down) writing
// fp32 rows for the weighted combine.
//
// Scales: "DeepSeekFp8" blockwise 128x128 weight scales and per-token
// per-128-column activation scales ("[Moe] Fix flashinfer_trtllm silently
// dropping swiglu_limit clamped SwiGLU activation", sglang PR #39920,
// "Modifications"). Each 128-deep slice of K is its own dot product, whose
// sum is multiplied by xs[row][kb] * ws[nb][kb]. A K step of this kernel is
// exactly one such block: for every 16x16 output subtile four 32-deep bf16
// MFMAs (GEMM1) or one 128-deep FP8 MFMA (GEMM2) sum the block into a
// short-lived partial that is scaled into the fp32 accumulator, so no
// per-block accumulators live across steps.
//
// Arithmetic, GEMM1: the e4m3 codes are expanded exactly to bf16 (hardware
// v_cvt_scalef32_pk_bf16_fp8 with scale 1; every e4m3 value has at most 4
// significant bits) and multiplied on v_mfma_f32_16x16x32_bf16, whose
// accumulation of such products is exact. The FP8 MFMA is not used there:
// on gfx950 it accumulates at reduced internal precision (measured about
// 2e-5 of sum |products|), enough to flip many e4m3 re-quantisation
// decisions of h. GEMM2's fp32 output only feeds the weighted combine, so
// it runs on v_mfma_f32_16x16x128_f8f6f4 straight from the codes: one
// instruction per 16x16 subtile and scale block, no conversions, half the
// LDS bytes (measured output error 2e-4..5e-4 of RMS(out), against about
// 1e-6 for the exact path).
//
// Work split: a workgroup of 8 waves owns BM sorted rows of one expert and
// 256 weight rows in two halves ("lo", "hi"). GEMM1: lo = gate rows
// nt*128.., hi = the matching up rows I + nt*128.., so one tile yields 128
// complete h columns, the FP8 re-quantisation group; GEMM2: lo/hi = output
// columns nt*256.. and nt*256 + 128.. (the decode-sized GEMM2 without LoRA
// runs 4-wave workgroups of half that width, see moe_gemm_fp8_kernel).
// Wave w computes all BM rows of columns 16w..16w+15 of both halves: gate
// and up of one h element meet in one lane, and every weight byte is used
// by exactly one wave, so weights stream from HBM straight into registers
// (two K blocks in flight) and never pass through LDS (GEMM1 expands them
// there once per block). The activation block is staged in LDS (a ring of
// four stages, below) together with its rows' activation scales --
// expanded to bf16 once per workgroup for GEMM1, as raw codes for GEMM2 --
// and read by every wave. The weights are the MFMA's first operand, so a
// lane's partials belong to one activation row and four consecutive weight
// columns: the block scale of a partial is one product xs[row] * ws[half]
// per lane and subtile, and the epilogue writes whole dwords of codes
// (GEMM1) or 16-byte fp32 runs (GEMM2).
//
// K order inside a block: lane (r = l % 16, q = l / 16) feeds the MFMA with
// elements 32q .. 32q + 31 of its row (bf16: 8 of them per 32-deep MFMA,
// step j taking 32q + 8j ..), on both operands -- any permutation of K
// shared by A and B leaves the dot product unchanged and this one gives
// every lane 32 contiguous weight bytes per row.
#include "gemm_common.h"

namespace moe {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Activation blocks live in a ring of kF8Stages LDS stages: block i of a
// tile is staged during block i - 2 and read in block i, and the workgroup
// meets at a barrier after every second block. Between barriers the waves
// drift apart (the two waves of a SIMD share its matrix core, and the one
// with the lower issue priority falls behind); the ring keeps the stage a
// fast wave writes two blocks ahead distinct from the two a slow wave may
// still read.
constexpr int kF8Stages = 4;

// F8: the activation block stays e4m3 (128-byte rows) for the FP8 MFMA;
// otherwise it is expanded to bf16 (256-byte rows)
template <int BM, bool F8, int NTH = kThreads>
struct F8Geo {
  static constexpr int MS = BM / 16;                       // 16-row subtiles
  static constexpr int A_BYTES = BM * (F8 ? 128 : 256);    // one K block
  static constexpr int A_CH = BM * 8;                      // 16-byte code chunks
  static constexpr int A_PT = (A_CH + NTH - 1) / NTH;
  static constexpr int X_BYTES = BM * 4;                   // row scales, [16][MS]
  static constexpr int STAGE = A_BYTES + X_BYTES;
  static constexpr int LDS = kF8Stages * STAGE;
};

// bf16 A rows are 256 bytes = 16 chunks of 16; chunk c of row r is stored
// at c ^ (r & 0b1011). gfx950 serves a ds_read_b128 / ds_write_b128 in four
// passes of 16 lanes -- the lanes that share lane bit 5 and the parity of
// lane bits 2..4 -- over 64 four-byte banks (fitted to bank-conflict counter
// readings of eight address patterns); under that rule this XOR makes both
// the 16-row fragment reads and the row-wise chunk stores conflict-free,
// where the plain c ^ (r & 15) costs two passes per read.
__device__ __forceinline__ int swz16(int row, int c) { return c ^ (row & 11); }

// e4m3 A rows are 128 bytes = 8 chunks of 16; chunk c of row r is stored at
// c ^ swz8(r). A fragment read (lanes r = 0..15 of a pass reading chunks 2q,
// 2q + 1 of rows 16 ms + r) and the row-wise chunk stores are both
// conflict-free under the four-pass rule above.
__device__ __forceinline__ int swz8(int row) { return ((row >> 1) & 1) | ((row >> 1) & 4); }

// 8 e4m3fn codes (two dwords, byte order) -> 8 bf16, exact
__device__ __forceinline__ bf16x8 e4m3x8_bf16(uint32_t w0, uint32_t w1) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  return (bf16x8){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Accumulator layout (weights are the MFMA's first operand): acc[ms][ns][r]
// is activation row 16 ms + (lane % 16) and weight column
// (ns ? hi : lo) + 16 wave + 4 (lane / 16) + r.
template <int BM, bool G1, bool LORA>
__device__ __forceinline__ void fp8_epilogue(const GemmParams& P, const Tile& t,
                                             f32x4 (&acc)[BM / 16][2], uint8_t* smem) {
  constexpr int MS = BM / 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int c0 = 16 * wave + 4 * lg;            // first of the lane's 4 columns
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
    float gsg = 1.0f, gsu = 1.0f;
    if (P.gscale) { gsg = P.gscale[2 * g]; gsu = P.gscale[2 * g + 1]; }
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        acc[ms][0][r] *= gsg;
        acc[ms][1][r] *= gsu;
      }
    if constexpr (LORA)
      if (P.z && g < P.lora_groups) lora_delta_tile<BM>(P, t, acc, smem, true);
    float hv[MS][4];
    const float L = P.limit, al = P.alpha, be = P.beta;
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float gg = fminf(acc[ms][0][r], L);
        const float uu = fminf(fmaxf(acc[ms][1][r], -L), L);
        const float sg = __builtin_amdgcn_rcpf(1.0f + expf(-al * gg));
        hv[ms][r] = gg * sg * (uu + be);
      }
    if (LORA && P.h_lora) {   // the down-LoRA input: h before the re-quantisation, bf16
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) {
        const int tr = 16 * ms + lr;
        if (tr < m)
          *(uint2*)(P.h_lora + (long)(row0 + tr) * P.I + t.nt * 128 + c0) =
              (uint2){f32_to_bf16_bits(hv[ms][0]) | (f32_to_bf16_bits(hv[ms][1]) << 16),
                      f32_to_bf16_bits(hv[ms][2]) | (f32_to_bf16_bits(hv[ms][3]) << 16)};
      }
    }
    // e4m3 re-quantisation per row and 128 columns: s = amax / 448, codes
    // round-to-nearest-even of h * (1 / s). Row amax: the lane's 4 columns,
    // the 4 lanes of the row (lane / 16), then the 8 waves through LDS.
    constexpr int kStg = 144;                         // staging row stride
    uint8_t* sh = smem;                               // [BM][kStg] codes
    float* s_amax = (float*)(smem + BM * kStg);       // [BM][8]
    float* s_inv = s_amax + 8 * BM;                   // [BM]
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
      float a = fmaxf(fmaxf(fabsf(hv[ms][0]), fabsf(hv[ms][1])),
                      fmaxf(fabsf(hv[ms][2]), fabsf(hv[ms][3])));
      a = max_across_rows(a);
      if (lg == 0) s_amax[(16 * ms + lr) * 8 + wave] = a;
    }
    __syncthreads();
    if (tid < BM) {
      const f32x4 a0 = *(const f32x4*)(s_amax + tid * 8);
      const f32x4 a1 = *(const f32x4*)(s_amax + tid * 8 + 4);
      const float a = fmaxf(fmaxf(fmaxf(a0[0], a0[1]), fmaxf(a0[2], a0[3])),
                            fmaxf(fmaxf(a1[0], a1[1]), fmaxf(a1[2], a1[3])));
      const float sc = a > 0.0f ? a / 448.0f : 1.0f;
      s_inv[tid] = 1.0f / sc;
      if (tid < m) P.hs[(long)(row0 + tid) * (P.I >> 7) + t.nt] = sc;
    }
    __syncthreads();
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
      const int tr = 16 * ms + lr;
      const float inv = s_inv[tr];
      float q[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)   // |q| <= 448 up to rounding; clamp, then RNE
        q[r] = __builtin_amdgcn_fmed3f(hv[ms][r] * inv, -448.0f, 448.0f);
      int v = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
      v = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], v, true);
      *(int*)(sh + tr * kStg + c0) = v;               // 4 consecutive columns
    }
    __syncthreads();
    for (int i = tid; i < BM * 8; i += kThreads) {
      const int tr = i >> 3, ch = i & 7;
      if (tr < m)
        *(i32x4*)(P.h + (long)(row0 + tr) * P.I + t.nt * 128 + ch * 16) =
            *(const i32x4*)(sh + tr * kStg + ch * 16);
    }
  }
}

// One tile of BM rows (BM = 32, 64 or 128; the rows at and after tl.m are
// padding) over K blocks [k0, k1): staging, K loop and epilogue. Called by
// the whole workgroup. DEEP: the A fragments are read from LDS two subtiles
// ahead (three register sets), the first two before the weight expansion;
// it pays where registers allow (kernels whose largest row class is 64 or
// less) and spills in the 128-row class. PART: the block-scaled fp32 sums
// go to partial slot `slot` instead of the epilogue (stream-K).
template <int BM, bool G1, bool DEEP, bool PART, bool LORA, int NTH = kThreads>
__device__ __forceinline__ void fp8_tile(const GemmParams& P, const Tile& tl, uint8_t* smem,
                                         int k0, int k1, int slot = 0) {
  static_assert(NTH == kThreads || (!G1 && !LORA && !PART), "4-wave tiles: plain GEMM2 only");
  // GEMM2 runs on the FP8 MFMA: its fp32 output feeds only the weighted
  // combine, where the FP8 MFMA's reduced-precision accumulation stays far
  // inside the output tolerance; GEMM1 keeps the exact bf16 path because its
  // output is re-quantised to e4m3.
  constexpr bool F8 = !G1;
  using Gm = F8Geo<BM, F8, NTH>;
  constexpr int MS = Gm::MS;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int K = P.K;
  const int NS = K >> 7;                      // K blocks of 128 (scale stride)
  const int g = tl.g, row0 = tl.row0, m = tl.m;

  // ---- this thread's sources at K block 0 (+128 bytes per block) --------
  const uint8_t* ap[Gm::A_PT];
  int a_st[Gm::A_PT];
#pragma unroll
  for (int i = 0; i < Gm::A_PT; ++i) {
    const int cc = min(tid + i * NTH, Gm::A_CH - 1);
    const int row = cc >> 3, ch = cc & 7;
    ap[i] = P.a + a_source_row<G1>(P, row0 + (row < m ? row : 0)) * P.a_ld + ch * 16;
    a_st[i] = F8 ? row * 128 + 16 * (ch ^ swz8(row)) : row * 256;
  }
  const float* xsp = P.as;               // row tid's activation scales
  if (tid < BM) xsp = P.as + a_source_row<G1>(P, row0 + (tid < m ? tid : 0)) * NS;
  const uint8_t* wg = P.w + (long)g * P.N * K;
  const uint8_t* bp0 = wg + (long)(tl.n_lo + 16 * wave + lr) * K + 32 * lg;
  const uint8_t* bp1 = wg + (long)(tl.n_hi + 16 * wave + lr) * K + 32 * lg;
  const float* wsl = (const float*)P.wsc + ((long)g * (P.N >> 7) + (tl.n_lo >> 7)) * NS;
  const float* wsh = (const float*)P.wsc + ((long)g * (P.N >> 7) + (tl.n_hi >> 7)) * NS;

  i32x4 ra[Gm::A_PT];
  float rxs = 0.0f;
  float wl_n = 0.0f, wh_n = 0.0f;       // weight block scales, one block ahead
  auto gload_a = [&](int s) {           // past the last block: re-read it
    const int sc = min(s, k1 - 1);
    const long adv = (long)sc * 128;
#pragma unroll
    for (int i = 0; i < Gm::A_PT; ++i) ra[i] = *(const i32x4*)(ap[i] + adv);
    if (tid < BM) rxs = xsp[sc];
  };
  auto gload_ws = [&](int s) {
    const int sc = min(s, k1 - 1);
    wl_n = wsl[sc];
    wh_n = wsh[sc];
  };
  // expand the codes to bf16 into LDS buffer buf; row scales as [16][MS]
  // so that each lane reads its rows' scales (rows lr, lr + 16, ...) at once
  auto store_a = [&](int buf) {
    uint8_t* st = smem + buf * Gm::STAGE;
#pragma unroll
    for (int i = 0; i < Gm::A_PT; ++i) {
      if (Gm::A_CH % NTH == 0 || tid + i * NTH < Gm::A_CH) {
        const int cc = tid + i * NTH, row = cc >> 3, ch = cc & 7;
        const i32x4 v = ra[i];
        if constexpr (F8) {
          *(i32x4*)(st + a_st[i]) = v;
        } else {
          *(bf16x8*)(st + a_st[i] + 16 * swz16(row, 2 * ch)) =
              e4m3x8_bf16((uint32_t)v[0], (uint32_t)v[1]);
          *(bf16x8*)(st + a_st[i] + 16 * swz16(row, 2 * ch + 1)) =
              e4m3x8_bf16((uint32_t)v[2], (uint32_t)v[3]);
        }
      }
    }
    if (tid < BM) ((float*)(st + Gm::A_BYTES))[(tid & 15) * MS + (tid >> 4)] = rxs;
  };
  auto gload_b = [&](i32x4 (&rb)[4], int s) {
    const long adv = (long)min(s, k1 - 1) * 128;
    rb[0] = *(const i32x4*)(bp0 + adv);
    rb[1] = *(const i32x4*)(bp0 + adv + 16);
    rb[2] = *(const i32x4*)(bp1 + adv);
    rb[3] = *(const i32x4*)(bp1 + adv + 16);
  };

  f32x4 acc[MS][2];
#pragma unroll
  for (int i = 0; i < MS; ++i) {
    acc[i][0] = (f32x4){0.f, 0.f, 0.f, 0.f};
    acc[i][1] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }

  // One K block: expand this block's weights, prefetch (A one block ahead,
  // B two blocks ahead into the registers just freed), then MFMA + scale.
  auto block = [&](int s, int buf, i32x4 (&rb)[4]) {
    const uint8_t* sa = smem + buf * Gm::STAGE;
    // A fragment of subtile ms: bf16 path 4 x 8 elements (K 32 lg + 8 j ..),
    // FP8 path the 32 codes K 32 lg .. 32 lg + 31 (as the weights)
    struct Frag {
      bf16x8 h[4];
      i32x8 q;
    };
    auto lds_a = [&](int ms, Frag& af) {
      const int row = 16 * ms + lr;
      if constexpr (F8) {
        const i32x4 u = *(const i32x4*)(sa + row * 128 + 16 * ((2 * lg) ^ swz8(row)));
        const i32x4 v = *(const i32x4*)(sa + row * 128 + 16 * ((2 * lg + 1) ^ swz8(row)));
        af.q = (i32x8){u[0], u[1], u[2], u[3], v[0], v[1], v[2], v[3]};
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          af.h[j] = *(const bf16x8*)(sa + row * 256 + 16 * swz16(row, 4 * lg + j));
      }
    };
    constexpr int D = DEEP ? 2 : 1;     // LDS prefetch distance, subtiles
    Frag fr[D + 1];
    if constexpr (DEEP) {
      lds_a(0, fr[0]);
      if (MS > 1) lds_a(1, fr[1]);
    }
    // pin this block's weight registers here so their expansion is not
    // hoisted into the previous block (it would double the live registers)
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(rb[i]));
    bf16x8 bw[2][4];     // bf16 path: the 32 codes of each row, expanded
    i32x8 bw8[2];        // FP8 path: the same codes as one MFMA operand
    if constexpr (F8) {
#pragma unroll
      for (int ns = 0; ns < 2; ++ns) {
        const i32x4 u = rb[2 * ns], v = rb[2 * ns + 1];
        bw8[ns] = (i32x8){u[0], u[1], u[2], u[3], v[0], v[1], v[2], v[3]};
      }
    } else {
#pragma unroll
      for (int ns = 0; ns < 2; ++ns)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const i32x4 v = rb[2 * ns + h];
          bw[ns][2 * h] = e4m3x8_bf16((uint32_t)v[0], (uint32_t)v[1]);
          bw[ns][2 * h + 1] = e4m3x8_bf16((uint32_t)v[2], (uint32_t)v[3]);
        }
    }
    // block s's weight scales arrived with its activations; reading them
    // here would expose a global-load latency per block on small tiles
    const float wl = wl_n, wh = wh_n;
    gload_ws(s + 1);
    gload_a(s + 2);
    gload_b(rb, s + 2);
    // this lane's activation scales for rows lr + 16 ms
    float xs[MS];
    {
      const float* sx = (const float*)(sa + Gm::A_BYTES) + lr * MS;
      if constexpr (MS % 4 == 0) {
#pragma unroll
        for (int i = 0; i < MS; i += 4) {
          const f32x4 v = *(const f32x4*)(sx + i);
          xs[i] = v[0]; xs[i + 1] = v[1]; xs[i + 2] = v[2]; xs[i + 3] = v[3];
        }
      } else if constexpr (MS % 2 == 0) {   // rows of MS floats: 8-byte aligned
#pragma unroll
        for (int i = 0; i < MS; i += 2) {
          const float2 v = *(const float2*)(sx + i);
          xs[i] = v.x; xs[i + 1] = v.y;
        }
      } else {
#pragma unroll
        for (int i = 0; i < MS; ++i) xs[i] = sx[i];
      }
    }
    // software pipeline over the 16-row subtiles: while the MFMAs of
    // subtile ms run, the A fragments of ms + 1 are in flight and ms - 1
    // is scaled into the accumulator. The scheduling fences keep the live
    // registers to that working set.
    auto scale_into = [&](int ms, const f32x4& p0, const f32x4& p1) {
      const float cl = xs[ms] * wl, ch = xs[ms] * wh;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        acc[ms][0][r] = fmaf(p0[r], cl, acc[ms][0][r]);
        acc[ms][1][r] = fmaf(p1[r], ch, acc[ms][1][r]);
      }
      asm volatile("" : "+v"(acc[ms][0]), "+v"(acc[ms][1]));   // keep in place
    };
    // weights as the first MFMA operand: p[r] = weight column 4 lg + r of
    // the wave's 16, activation row lr
    auto sub = [&](const Frag& af, f32x4& p0, f32x4& p1) {
      p0 = (f32x4){0.f, 0.f, 0.f, 0.f};
      p1 = p0;
      if constexpr (F8) {   // e4m3 x e4m3, unscaled (scale operands 0)
        p0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bw8[0], af.q, p0, 0, 0, 0, 0, 0, 0);
        p1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bw8[1], af.q, p1, 0, 0, 0, 0, 0, 0);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          p0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bw[0][j], af.h[j], p0, 0, 0, 0);
          p1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bw[1][j], af.h[j], p1, 0, 0, 0);
        }
      }
    };
    // D + 1 fragment sets and two partial sets rotate over the (unrolled)
    // subtiles, so the pipeline needs no register copies
    f32x4 pp[2][2];
    if constexpr (!DEEP) lds_a(0, fr[0]);
    // order inside a region: the prefetch reads first, then the MFMAs
    // with the scaling arithmetic spread between them
    auto pattern = [&](bool reads) {
      if constexpr (F8) {
        if (reads) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0); // DS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);            // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);            // VALU
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
      } else {
        if (reads) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0); // DS read
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // MFMA
          if (i < 5) __builtin_amdgcn_sched_group_barrier(0x002, 2, 0); // VALU
        }
      }
    };
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
      if (ms + D < MS) lds_a(ms + D, fr[(ms + D) % (D + 1)]);
      sub(fr[ms % (D + 1)], pp[ms & 1][0], pp[ms & 1][1]);
      if (ms > 0) scale_into(ms - 1, pp[(ms - 1) & 1][0], pp[(ms - 1) & 1][1]);
      pattern(ms + D < MS);
      __builtin_amdgcn_sched_barrier(0);
    }
    scale_into(MS - 1, pp[(MS - 1) & 1][0], pp[(MS - 1) & 1][1]);
    store_a((buf + 2) & (kF8Stages - 1));   // block s + 2
  };

  i32x4 rb0[4], rb1[4];
  gload_b(rb0, k0);
  gload_b(rb1, k0 + 1);
  gload_ws(k0);
  gload_a(k0);
  store_a(0);
  gload_a(k0 + 1);
  store_a(1);
  __syncthreads();
  // block i = s - k0 reads stage i % 4 (staged in block i - 2) and stages
  // block i + 2 into stage (i + 2) % 4, which held block i - 2; both were
  // completed by every wave before the barrier that closed the pair
  // i - 2, i - 1 (or the prologue's)
  int s = k0;
  for (; s + 2 <= k1; s += 2) {
    const int i = s - k0;
    block(s, i & 3, rb0);
    block(s + 1, (i + 1) & 3, rb1);
    __syncthreads();
  }
  if (s < k1) {            // odd block count
    block(s, (s - k0) & 3, rb0);
    __syncthreads();
  }
  if constexpr (PART) {
    // acc[ms][ns][r]: row 16 ms + lr, column (ns ? hi : lo) + 16 wave + 4 lg + r
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
    fp8_epilogue<BM, G1, LORA>(P, tl, acc, smem);
    __syncthreads();       // LDS is reused by the next tile
  }
}

// Tiles are scheduled with up to TBM rows of one expert; each runs the code
// of the smallest row class (32 / 64 / 128, at most TBM) that holds its
// valid rows, so a lightly loaded expert does not pay for TBM rows of MFMA
// work.
// The tiles (TBM-row scheduling, s_cum its prefix) walked by persistent
// workgroups: XCD x (= blockIdx % 8) owns logical tiles [x*chunk,
// (x+1)*chunk), so the N-tiles of one expert share an L2.
template <int TBM, bool G1, bool LORA, int NTH>
__device__ __forceinline__ void plain_tiles(const GemmParams& P, uint8_t* smem,
                                            const int* s_cum) {
  constexpr int W2 = NTH / 2;                // GEMM2 tile columns: 16 per wave and half
  const int NT = G1 ? (P.I >> 7) : ((P.N + W2 - 1) / W2);
  const int NS = P.K >> 7;
  const int total = s_cum[P.G] * NT;
  const int xcd = blockIdx.x & 7, nper = gridDim.x >> 3, slot = blockIdx.x >> 3;
  const int chunk = (total + 7) >> 3;
  const int t_end = min(total, (xcd + 1) * chunk);
  for (int lt = xcd * chunk + slot; lt < t_end; lt += nper) {
    Tile tl = decode_tile<TBM, G1>(P, lt, NT, s_cum, W2);
    tl.g = __builtin_amdgcn_readfirstlane(tl.g);
    tl.row0 = __builtin_amdgcn_readfirstlane(tl.row0);
    tl.m = __builtin_amdgcn_readfirstlane(tl.m);
    tl.nt = __builtin_amdgcn_readfirstlane(tl.nt);
    tl.n_lo = __builtin_amdgcn_readfirstlane(tl.n_lo);
    tl.n_hi = __builtin_amdgcn_readfirstlane(tl.n_hi);
    if constexpr (TBM >= 160) {
      if (tl.m > 128) {
        fp8_tile<160, G1, false, false, LORA, NTH>(P, tl, smem, 0, NS);
        continue;
      }
    }
    if constexpr (TBM >= 128) {
      if (tl.m > 64) {
        fp8_tile<128, G1, false, false, LORA, NTH>(P, tl, smem, 0, NS);
        continue;
      }
    }
    if constexpr (TBM >= 64) {
      if (tl.m > 32) {
        fp8_tile<64, G1, G1 && TBM <= 64, false, LORA, NTH>(P, tl, smem, 0, NS);
        continue;
      }
    }
    fp8_tile<32, G1, G1 && TBM <= 64, false, LORA, NTH>(P, tl, smem, 0, NS);
  }
}

// LORA: the kernel carries the LoRA delta (and the bf16 down-LoRA input of
// GEMM1); layers without LoRA run the instantiation without that code.
// NTH: 512 threads (8 waves), or 256 (4 waves, 128-column GEMM2 tiles) for
// the plain GEMM2 without LoRA at decode sizes (32-row tiles): twice the
// tiles, so that a few experts' tiles still spread over the whole GPU, with
// more workgroups per CU and independent barriers. (With 128-row tiles the
// 256-column tiles are faster: half the activation reads.)
template <int TBM, bool G1, bool LORA, int NTH>
__global__ __launch_bounds__(NTH) void moe_gemm_fp8_kernel(GemmParams P) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];   // 2 stages
  __shared__ int s_cum[kMaxGroups + 1];
  __shared__ int s_wsum[8];
  tile_prefix<TBM>(P.offsets, P.G, s_cum, s_wsum);
  plain_tiles<TBM, G1, LORA, NTH>(P, smem, s_cum);
}

// Split-K (stream-K) kernel over 32-row tiles (see gemm_common.h):
// workgroup b runs the K-block segments of its unit range and leaves fp32
// partial sums in slot b - (first workgroup of the tile).
template <bool G1, bool LORA>
__global__ __launch_bounds__(kThreads) void moe_gemm_fp8_sk_kernel(GemmParams P) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int s_cum[kMaxGroups + 1];
  __shared__ int s_wsum[8];
  const int G = P.G;
  const int NT = G1 ? (P.I >> 7) : ((P.N + 255) >> 8);
  const int NS = P.K >> 7;
  tile_prefix<kSkBM>(P.offsets, G, s_cum, s_wsum);
  // SK_DEVICE: the rule on the real tile count picked whole tiles; run them
  // here as the plain kernel would (its 32-row class: the host sends only
  // batches of at most 16 rows per group this way), so no second launch
  if (P.sk_mode == SK_DEVICE && !sk_rule((long)s_cum[G] * NT, NS)) {
    plain_tiles<kSkBM, G1, LORA, kThreads>(P, smem, s_cum);
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
    fp8_tile<kSkBM, G1, G1, true, LORA>(P, tl, smem, k0, k1, slot);
    u += k1 - k0;
  }
}

template <int TBM, bool G1, bool LORA>
static hipError_t run_fp8(const GemmParams& P, long p_cap, int NT, hipStream_t s) {
  constexpr int NTH = (!G1 && !LORA && TBM <= 32) ? 256 : kThreads;
  if (NTH != kThreads) NT = (P.N + NTH / 2 - 1) / (NTH / 2);
  constexpr int shm = LORA ? std::max(F8Geo<TBM, !G1>::LDS, kLoraLds) : F8Geo<TBM, !G1, NTH>::LDS;
  static int per_cu = 0;   // resident workgroups per CU, per instantiation
  if (per_cu == 0) {
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&moe_gemm_fp8_kernel<TBM, G1, LORA, NTH>),
        hipFuncAttributeMaxDynamicSharedMemorySize, shm);
    if (e != hipSuccess) return e;
    int nb = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &nb, reinterpret_cast<const void*>(&moe_gemm_fp8_kernel<TBM, G1, LORA, NTH>), NTH, shm);
    if (e != hipSuccess) return e;
    per_cu = nb > 0 ? nb : 1;
  }
  long max_tiles = ((p_cap + TBM - 1) / TBM + P.G) * (long)NT;
  long nwg = std::min<long>(max_tiles, (long)num_cus() * per_cu);
  nwg = (nwg + 7) & ~7L;
  if (nwg == 0) return hipSuccess;
  GemmParams Q = P;
  Q.lds_bytes = shm;
  moe_gemm_fp8_kernel<TBM, G1, LORA, NTH><<<dim3((unsigned)nwg), dim3(NTH), shm, s>>>(Q);
  return hipGetLastError();
}

template <bool G1, bool LORA>
static hipError_t run_fp8_sk(const GemmParams& P, long p_cap, int NT, hipStream_t s,
                             int* sk_grid) {
  constexpr int shm = LORA ? std::max(F8Geo<kSkBM, !G1>::LDS, kLoraLds) : F8Geo<kSkBM, !G1>::LDS;
  static int per_cu = 0;
  if (per_cu == 0) {
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&moe_gemm_fp8_sk_kernel<G1, LORA>),
        hipFuncAttributeMaxDynamicSharedMemorySize, shm);
    if (e != hipSuccess) return e;
    int nb = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &nb, reinterpret_cast<const void*>(&moe_gemm_fp8_sk_kernel<G1, LORA>), kThreads, shm);
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
  moe_gemm_fp8_sk_kernel<G1, LORA><<<dim3((unsigned)grid), dim3(kThreads), shm, s>>>(Q);
  return hipGetLastError();
}

template <bool G1, bool LORA>
static hipError_t run_fp8_tbm(const GemmParams& P, long p_cap, int NT, hipStream_t s) {
  // the largest row class worth scheduling: rows per group on average
  const long hint = P.G > 0 ? p_cap / P.G : p_cap;
  if (hint <= 32) return run_fp8<32, G1, LORA>(P, p_cap, NT, s);
  if (hint <= 64) return run_fp8<64, G1, LORA>(P, p_cap, NT, s);
  // GEMM2 without LoRA also has a 160-row class: a group of 129..160 rows
  // (common when groups average ~115 rows) streams its weights once instead
  // of twice, and a large group needs a fifth fewer M-tiles. GEMM1's bf16
  // activation ring has no room for it.
  if constexpr (!G1 && !LORA) return run_fp8<160, G1, LORA>(P, p_cap, NT, s);
  return run_fp8<128, G1, LORA>(P, p_cap, NT, s);
}

template <bool LORA>
static hipError_t launch_fp8(const GemmParams& P, bool g1, long p_cap, int NT, hipStream_t s,
                             int* sk_grid) {
  if (P.part)
    return g1 ? run_fp8_sk<true, LORA>(P, p_cap, NT, s, sk_grid)
              : run_fp8_sk<false, LORA>(P, p_cap, NT, s, sk_grid);
  return g1 ? run_fp8_tbm<true, LORA>(P, p_cap, NT, s) : run_fp8_tbm<false, LORA>(P, p_cap, NT, s);
}

hipError_t launch_gemm_fp8(const GemmParams& P, bool g1, long p_cap, int NT, hipStream_t s,
                           int* sk_grid) {
  return (P.z || P.h_lora) ? launch_fp8<true>(P, g1, p_cap, NT, s, sk_grid)
                           : launch_fp8<false>(P, g1, p_cap, NT, s, sk_grid);
}

}  // namespace moe
