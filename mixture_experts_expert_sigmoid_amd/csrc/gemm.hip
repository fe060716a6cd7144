// Grouped expert GEMMs on CDNA4 MFMA for BF16 layers: GEMM1 over the fused
// [gate | up] weight with the parameterized-SwiGLU epilogue (plus optional
// per-half global scales and LoRA delta), and GEMM2 (down) writing fp32 rows
// for the weighted combine. Blockwise-FP8 layers use the kernels of
// gemm_fp8.hip, 4-bit layers (INT4, NVFP4, MXFP4) those of gemm_w4.h; this
// file also holds the host dispatch for every format.
//
// Epilogue: g' = min(g, L), u' = clamp(u, -L, L), h = g' sigmoid(alpha g')
// (u' + beta) ("[Moe] Fix flashinfer_trtllm silently dropping swiglu_limit
// clamped SwiGLU activation", sglang PR #39920, "Modifications"; "fix(sm90):
// support parameterized SwiGLU in FP8 MegaMoE", DeepGEMM PR #445,
// "Summary"). The LoRA delta and the per-half global scales follow the
// true-units rule of "FlashInfer 0.6.18 SM100a+SM103a MoE-LoRA AOT"
// ("Changes since 1b699bf"): each half is scaled by its own global scale
// first, then the delta is added. Products run on v_mfma_f32_16x16x32_bf16.
//
// Tiling: a workgroup of 8 waves owns BM sorted rows of one expert and 256
// weight rows in two halves of 128 ("lo", "hi"): for GEMM1 lo = gate rows
// n0..n0+127 and hi = the matching up rows I+n0..I+n0+127, so one tile yields
// 128 complete h columns; for GEMM2 lo/hi are output columns n0..n0+255.
// Wave (wm, wn) computes rows wm*BM/2.. of columns wn*32..wn*32+31 of both
// halves, so gate and up values of one h element sit in the same lane. K
// advances 64 per stage: global -> registers (two stages in flight) -> LDS
// (double buffered, one barrier per stage). LDS rows are 128 bytes; their
// 16-byte chunks are XOR-swizzled with (row / 2) mod 8 so the 16 rows read
// by one ds_read_b128 are free of bank conflicts.
// Workgroups are persistent: each computes the tile count from the expert
// offsets on the device and walks its XCD's contiguous share of the tiles,
// so the N-tiles of one expert (which share the gathered activation rows)
// stay in one XCD's L2.
#include "gemm_common.h"

namespace moe {

template <int BM>
struct Geo {
  // per 64-K stage, in 16-byte global chunks
  static constexpr int A_SRC = 128;                               // bytes per A row
  static constexpr int A_CH = BM * A_SRC / 16;
  static constexpr int A_PT = (A_CH + kThreads - 1) / kThreads;   // loads per thread
  static constexpr int B_SRC = 128;
  static constexpr int B_CH = 256 * B_SRC / 16;
  static constexpr int B_PT = B_CH / kThreads;
  static constexpr int A_LDS = BM * 128;                          // 16-bit tile bytes
  static constexpr int B_LDS = 256 * 128;
  static constexpr int STAGE = A_LDS + B_LDS;
  static constexpr int TOTAL = 2 * STAGE;
};

template <int BM>
struct Regs {
  i32x4 a[Geo<BM>::A_PT];
  i32x4 b[Geo<BM>::B_PT];
};

template <int BM, bool G1>
__global__ __launch_bounds__(kThreads) void moe_gemm_kernel(GemmParams P) {
  using Gm = Geo<BM>;
  constexpr int MS = BM / 32;            // 16-row subtiles per wave
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int s_cum[kMaxGroups + 1];
  __shared__ int s_wsum[8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int lr = lane & 15, lg = lane >> 4;
  const int G = P.G, K = P.K;
  const int NT = G1 ? (P.I >> 7) : ((P.N + 255) >> 8);
  const int NS = K / KS;

  tile_prefix<BM>(P.offsets, G, s_cum, s_wsum);
  const int total = s_cum[G] * NT;
  // XCD x (= blockIdx % 8) owns logical tiles [x*chunk, (x+1)*chunk)
  const int xcd = blockIdx.x & 7, nper = gridDim.x >> 3, slot = blockIdx.x >> 3;
  const int chunk = (total + 7) >> 3;
  const int t_end = min(total, (xcd + 1) * chunk);

  for (int lt = xcd * chunk + slot; lt < t_end; lt += nper) {
    const Tile tl = decode_tile<BM, G1>(P, lt, NT, s_cum);
    const int g = tl.g, row0 = tl.row0, m = tl.m, n_lo = tl.n_lo, n_hi = tl.n_hi;
    const long wrow = (long)K * 2;
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
      const long src = a_source_row<G1>(P, row0 + (row < m ? row : 0));
      ap[i] = P.a + src * P.a_ld + ch * 16;
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

    // Loads are unconditional (past the last stage they re-read it) so the
    // compiler's wait counts stay static and two stages remain in flight.
    auto gload = [&](Regs<BM>& R, int s) {
      s = min(s, NS - 1);
      const long adv = (long)s * Gm::A_SRC;
#pragma unroll
      for (int i = 0; i < Gm::A_PT; ++i) R.a[i] = *(const i32x4*)(ap[i] + adv);
      const long bdv = (long)s * Gm::B_SRC;
#pragma unroll
      for (int i = 0; i < Gm::B_PT; ++i) R.b[i] = *(const i32x4*)(bp[i] + bdv);
    };
    auto sstore = [&](const Regs<BM>& R, int s, auto par, auto guard) {
      constexpr int PAR = decltype(par)::value;
      if (decltype(guard)::value && s >= NS) return;
      uint8_t* sa = smem + PAR * Gm::STAGE;
      uint8_t* sb = sa + Gm::A_LDS;
#pragma unroll
      for (int i = 0; i < Gm::A_PT; ++i) {
        // surplus threads (a_on false) store the same bytes as the thread
        // they duplicated: harmless, and it keeps the stage branch-free
        const int row = a_row[i];
        *(i32x4*)(sa + row * 128 + swz(row, a_ch[i]) * 16) = R.a[i];
      }
#pragma unroll
      for (int i = 0; i < Gm::B_PT; ++i) {
        const int row = b_row[i];
        *(i32x4*)(sb + row * 128 + swz(row, b_ch[i]) * 16) = R.b[i];
      }
    };

    // ---- accumulators -----------------------------------------------------
    f32x4 acc[MS][4];
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
      }
    const int rbase = wm * (BM / 2);

    auto compute = [&](int s, auto par, auto guard) {
      constexpr int PAR = decltype(par)::value;   // == s & 1
      if (decltype(guard)::value && s >= NS) return;
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
            f32x4& d = acc[ms][ns];
            const f32x4 c = d;
            d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af[ms]),
                                                        __builtin_bit_cast(bf16x8, bv), c, 0, 0, 0);
          }
        }
      }
    };

    // ---- pipelined K loop: two stages in flight ---------------------------
    // stage t lives in register set t % 3 and LDS buffer t % 2; unrolled by
    // six so both are compile-time.
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using GY = std::true_type;    // guarded: skips stages past the end
    using GN = std::false_type;
    Regs<BM> r0, r1, r2;
    gload(r0, 0);
    gload(r1, 1);
    sstore(r0, 0, P0{}, GY{});
    __syncthreads();
    int s = 0;
    // full groups of six stages, branch-free
    for (; s + 6 <= NS; s += 6) {
      gload(r2, s + 2); compute(s, P0{}, GN{});     sstore(r1, s + 1, P1{}, GY{});
      __syncthreads();
      gload(r0, s + 3); compute(s + 1, P1{}, GN{}); sstore(r2, s + 2, P0{}, GY{});
      __syncthreads();
      gload(r1, s + 4); compute(s + 2, P0{}, GN{}); sstore(r0, s + 3, P1{}, GY{});
      __syncthreads();
      gload(r2, s + 5); compute(s + 3, P1{}, GN{}); sstore(r1, s + 4, P0{}, GY{});
      __syncthreads();
      gload(r0, s + 6); compute(s + 4, P0{}, GN{}); sstore(r2, s + 5, P1{}, GY{});
      __syncthreads();
      gload(r1, s + 7); compute(s + 5, P1{}, GN{}); sstore(r0, s + 6, P0{}, GY{});
      __syncthreads();
    }
    if (s < NS) {                 // remaining 1..5 stages (s % 6 == 0 here)
      gload(r2, s + 2); compute(s, P0{}, GY{});     sstore(r1, s + 1, P1{}, GY{}); __syncthreads();
      gload(r0, s + 3); compute(s + 1, P1{}, GY{}); sstore(r2, s + 2, P0{}, GY{}); __syncthreads();
      gload(r1, s + 4); compute(s + 2, P0{}, GY{}); sstore(r0, s + 3, P1{}, GY{}); __syncthreads();
      gload(r2, s + 5); compute(s + 3, P1{}, GY{}); sstore(r1, s + 4, P0{}, GY{}); __syncthreads();
      gload(r0, s + 6); compute(s + 4, P0{}, GY{}); sstore(r2, s + 5, P1{}, GY{}); __syncthreads();
    }

    tile_epilogue<BM, G1>(P, tl, acc, smem);
    __syncthreads();     // LDS is reused by the next tile
  }
}

int num_cus() {
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

template <int BM, bool G1>
static hipError_t run(const GemmParams& P, long p_cap, int NT, hipStream_t s) {
  constexpr int shm = Geo<BM>::TOTAL;
  static int per_cu = 0;   // resident workgroups per CU, per instantiation
  if (per_cu == 0) {
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&moe_gemm_kernel<BM, G1>),
        hipFuncAttributeMaxDynamicSharedMemorySize, shm);
    if (e != hipSuccess) return e;
    int nb = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &nb, reinterpret_cast<const void*>(&moe_gemm_kernel<BM, G1>), kThreads, shm);
    if (e != hipSuccess) return e;
    per_cu = nb > 0 ? nb : 1;
  }
  long max_tiles = ((p_cap + BM - 1) / BM + P.G) * (long)NT;
  long nwg = std::min<long>(max_tiles, (long)num_cus() * per_cu);
  nwg = (nwg + 7) & ~7L;
  if (nwg == 0) return hipSuccess;
  moe_gemm_kernel<BM, G1><<<dim3((unsigned)nwg), dim3(kThreads), shm, s>>>(P);
  return hipGetLastError();
}

// BF16 layers: rows per expert on average decide the M tile
template <bool G1>
static hipError_t dispatch(const GemmParams& P, long p_cap, int NT, long rows_hint,
                           hipStream_t s) {
  if (rows_hint <= 32) return run<32, G1>(P, p_cap, NT, s);
  if (rows_hint <= 64) return run<64, G1>(P, p_cap, NT, s);
  return run<128, G1>(P, p_cap, NT, s);
}

hipError_t launch_gemm1(const Gemm1Args& a, hipStream_t s) {
  GemmParams P{};
  P.a = (const uint8_t*)a.x;
  P.as = (const float*)a.xs;
  const bool mx = a.fmt == FMT_MXFP4_A8;
  P.a_ld = (long)a.H * (a.fmt == FMT_FP8 || mx ? 1 : 2);   // bytes per activation row
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
  P.n_adapters = a.n_adapters;
  P.zad = a.zad;
  P.h = (uint8_t*)a.h;
  P.hs = a.hs;
  P.h_lora = (uint16_t*)a.h_lora;
  P.err = a.err;
  long hint = a.G > 0 ? a.p_cap / a.G : a.p_cap;
  if (a.fmt != FMT_BF16) {
    const bool fp8 = a.fmt == FMT_FP8;
    hipError_t e = hipSuccess;
    if (!fp8 && !mx) {             // f16 activations in the 4-bit kernel's K order
      if (!a.x16_ready) e = launch_act_f16p(a.x, a.T, a.H, a.x16, a.err, s);
      if (e != hipSuccess) return e;
      P.a = (const uint8_t*)a.x16;
    }
    auto run = [&](int* grid) {
      return fp8 ? launch_gemm_fp8(P, true, a.p_cap, a.I / 128, s, grid)
             : mx ? launch_gemm1_mx(P, a.p_cap, a.I / 128, s, grid)
                  : launch_gemm_w4(a.fmt, P, true, a.p_cap, a.I / 128, s, grid);
    };
    const int mode = a.part ? splitk_mode(a.fmt, a.p_cap, a.G, a.I / 128, a.H / 128, true)
                            : SK_PLAIN;
    P.sk_mode = mode;
    // SK_DEVICE: the split-K kernel alone decides on the device and runs
    // whole tiles itself when split-K does not pay, except for NVFP4 and a
    // W4A8 layer with LoRA, whose split-K kernels would lose occupancy to
    // the whole-tile code: there the plain kernel is launched too and
    // returns at once if the split-K kernel takes the GEMM
    const bool whole = fp8 || (mx ? !P.z : a.fmt != FMT_NVFP4);
    if (mode == SK_PLAIN || (mode == SK_DEVICE && !whole)) {
      e = run(nullptr);
      if (e != hipSuccess || mode == SK_PLAIN) return e;
    }
    P.part = a.part;
    P.p_rows = a.p_cap;
    int grid = 0;
    e = run(&grid);
    return e == hipSuccess ? launch_gemm1_sk_epilogue(P, grid, fp8, s) : e;
  }
  return dispatch<true>(P, a.p_cap, a.I / 128, hint, s);
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
  P.gscale = a.gscale;
  P.y = a.y;
  P.z = a.z;
  P.lora_B = (const uint16_t*)a.lora_B;
  P.lora_rank = a.lora_rank;
  P.lora_groups = a.z ? a.lora_groups : 0;
  P.lora_scale = a.lora_scale;
  P.n_adapters = a.n_adapters;
  P.zad = a.zad;
  P.err = a.err;
  long hint = a.G > 0 ? a.p_cap / a.G : a.p_cap;
  *a.sk_grid = 0;
  *a.sk_mode = SK_PLAIN;
  const int NT = (a.H + 255) / 256;
  if (a.fmt != FMT_BF16) {
    const bool fp8 = a.fmt == FMT_FP8;
    auto run = [&](int* grid) {
      return fp8 ? launch_gemm_fp8(P, false, a.p_cap, NT, s, grid)
                 : launch_gemm_w4(a.fmt, P, false, a.p_cap, NT, s, grid);
    };
    const int mode = splitk_mode(a.fmt, a.p_cap, a.G, NT, a.I / 128, false);
    P.sk_mode = mode;
    *a.sk_mode = mode;
    if (mode != SK_SPLIT) {
      P.y16 = (uint16_t*)a.y;      // int16 rows, then their scale exponents
      P.ye = (int8_t*)((char*)a.y + (size_t)a.p_cap * a.H * 2);
      hipError_t e = run(nullptr);
      if (e != hipSuccess || mode == SK_PLAIN) return e;
    }
    P.part = a.y;                  // the partial-sum slots (slot 0 = plain rows)
    P.p_rows = a.p_cap;
    return run(a.sk_grid);
  }
  return dispatch<false>(P, a.p_cap, NT, hint, s);
}

int splitk_mode(int fmt, long p_cap, int G, int NT, int NS, bool g1) {
  if (fmt == FMT_BF16 || p_cap <= 0) return SK_PLAIN;
  const long tiles = std::min<long>(p_cap, G + p_cap / kSkBM) * NT;
  if (sk_rule(tiles, NS)) return SK_SPLIT;
  return g1 && tiles <= kSkDeviceMaxTiles && p_cap <= 16L * G ? SK_DEVICE : SK_PLAIN;
}

}  // namespace moe
