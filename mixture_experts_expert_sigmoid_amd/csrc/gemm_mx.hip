// GEMM1 of the MXFP4 W4A8 layers on the block-scaled matrix cores: MXFP4
// expert weights (e2m1 codes, e8m0 scale per 32 K) times MXFP8 activations
// (e4m3 codes, e8m0 scale per 32 columns, quant.hip) on
// v_mfma_scale_f32_16x16x128_f8f6f4, then the parameterized SwiGLU epilogue
// of the 4-bit kernels (gemm_w4.h) writing bf16 h. The weights are the
// format of the MXFP4 layers; the pages name 4-bit expert weights ("FlashInfer
// 0.6.18 SM100a+SM103a MoE-LoRA AOT" release notes, "Changes since 1b699bf")
// and fix no activation format for them: MXFP8 is this library's choice,
// the form these instructions take.
//
// The instruction applies both operands' scales itself, so the fp32
// accumulator runs through the whole K with no per-block scaling step: one
// MFMA per 16x16 subtile and 128-deep K block. Its 128-deep sums are not
// fp32-accurate (measured on gfx950: within 2e-5 of the block's sum of
// |products|), so this GEMM is not bit-comparable to the W4A16 kernel; h
// is rounded to bf16 and GEMM2 runs the W4A16 MXFP4 kernel on it.
//
// Operand layout (found by one-hot probes on gfx950): for the fp4 source
// (the weights, first operand) lane group q = lane / 16 holds K 32q ..
// 32q + 31 of its row, low nibble first -- 16 contiguous bytes of a packed
// row; for the fp8 source (the activations) lane group q holds K 16q ..
// 16q + 15 in its first 16 bytes and K 64 + 16q .. 64 + 16q + 15 in its
// second 16; the scale of K block j (32 wide) of a row comes from lane
// group j's scale register on both sides (its low byte).
//
// Work split and pipeline as in the FP8 kernel (gemm_fp8.hip): 8 waves own
// BM sorted rows of one expert and 256 weight rows -- 128 gate rows nt*128..
// and the matching 128 up rows I + nt*128.. -- wave w computing columns
// 16w..16w+15 of both halves; weights stream HBM -> registers two blocks
// ahead (16 bytes and one scale byte per row and lane per block); the
// activation codes and their rows' scale words are staged in a ring of four
// LDS stages, two blocks ahead, with a barrier after every second block.
#include "gemm_w4.h"

namespace moe {

constexpr int kMxStages = 4;

template <int BM>
struct MxGeo {
  static constexpr int MS = BM / 16;              // 16-row subtiles
  static constexpr int A_BYTES = BM * 128;        // e4m3 codes of one K block
  static constexpr int A_CH = BM * 8;             // 16-byte chunks
  static constexpr int A_PT = (A_CH + kThreads - 1) / kThreads;
  static constexpr int X_BYTES = BM * 4;          // the rows' four e8m0 codes, [16][MS]
  static constexpr int STAGE = A_BYTES + X_BYTES;
  static constexpr int LDS = kMxStages * STAGE;
};

// e4m3 A rows are 128 bytes = 8 chunks of 16; chunk c of row r sits at
// swz(r, c) = c ^ ((r >> 1) & 7). Under gfx950's four-pass service of
// ds_read_b128 / ds_write_b128 (16 lanes a pass: those sharing lane bit 5
// and the parity of lane bits 2..4, over 64 four-byte banks) both the
// fragment reads (chunks q and q + 4 of rows 16 ms + 0..15) and the
// row-wise chunk stores are conflict-free.

template <int BM, bool PART, bool LORA>
__device__ __forceinline__ void mx_tile(const GemmParams& P, const Tile& tl, uint8_t* smem,
                                        int k0, int k1, int slot = 0) {
  using Gm = MxGeo<BM>;
  constexpr int MS = Gm::MS;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int K = P.K;
  const int KS32 = K >> 5;                    // scale codes per row
  const int g = tl.g, row0 = tl.row0, m = tl.m;

  // ---- sources at K block 0 ----------------------------------------------
  const uint8_t* ap[Gm::A_PT];
  int a_st[Gm::A_PT];
#pragma unroll
  for (int i = 0; i < Gm::A_PT; ++i) {
    const int cc = min(tid + i * kThreads, Gm::A_CH - 1);
    const int row = cc >> 3, ch = cc & 7;
    ap[i] = P.a + a_source_row<true>(P, row0 + (row < m ? row : 0)) * P.a_ld + ch * 16;
    a_st[i] = row * 128 + 16 * swz(row, ch);
  }
  // row tid's scale codes (four per block, one 32-bit word)
  const uint8_t* xsp = (const uint8_t*)P.as;
  if (tid < BM) xsp += a_source_row<true>(P, row0 + (tid < m ? tid : 0)) * KS32;
  const long wrow = K >> 1;
  const uint8_t* wg = P.w + (long)g * P.N * wrow;
  const long nl = tl.n_lo + 16 * wave + lr, nh = tl.n_hi + 16 * wave + lr;
  const uint8_t* bp0 = wg + nl * wrow + 16 * lg;
  const uint8_t* bp1 = wg + nh * wrow + 16 * lg;
  const uint8_t* sp0 = (const uint8_t*)P.wsc + ((long)g * P.N + nl) * KS32 + lg;
  const uint8_t* sp1 = (const uint8_t*)P.wsc + ((long)g * P.N + nh) * KS32 + lg;

  // Activation blocks travel global -> registers -> LDS. Two register sets
  // (by block parity) give each gathered row load two blocks of latency:
  // the set of block j is loaded at the end of block j - 4 and stored into
  // its LDS stage at the end of block j - 2.
  struct AR {
    i32x4 v[Gm::A_PT];
    uint32_t xs;
  };
  AR ra0, ra1;
  uint64_t bad_s = 0;                          // NaN weight scales met (ballot)
  auto gload_a = [&](AR& r, int s) {           // past the last block: re-read it
    const int sc = min(s, k1 - 1);
#pragma unroll
    for (int i = 0; i < Gm::A_PT; ++i) r.v[i] = *(const i32x4*)(ap[i] + (long)sc * 128);
    r.xs = tid < BM ? *(const uint32_t*)(xsp + 4 * sc) : 0u;
  };
  auto store_a = [&](const AR& r, int buf) {
    uint8_t* st = smem + buf * Gm::STAGE;
#pragma unroll
    for (int i = 0; i < Gm::A_PT; ++i)
      if (Gm::A_CH % kThreads == 0 || tid + i * kThreads < Gm::A_CH)
        *(i32x4*)(st + a_st[i]) = r.v[i];
    if (tid < BM) ((uint32_t*)(st + Gm::A_BYTES))[(tid & 15) * MS + (tid >> 4)] = r.xs;
  };
  struct WB {
    i32x4 q[2];                                // lo, hi rows: 32 codes each
    uint32_t s[2];                             // their e8m0 scale codes
  };
  auto gload_b = [&](WB& b, int s) {
    const int sb = min(s, k1 - 1);
    b.q[0] = *(const i32x4*)(bp0 + (long)sb * 64);
    b.q[1] = *(const i32x4*)(bp1 + (long)sb * 64);
    b.s[0] = sp0[4 * sb];
    b.s[1] = sp1[4 * sb];
  };

  f32x4 acc[MS][2];
#pragma unroll
  for (int i = 0; i < MS; ++i) {
    acc[i][0] = (f32x4){0.f, 0.f, 0.f, 0.f};
    acc[i][1] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }

  auto block = [&](int s, int buf, WB& rb, AR& ra) {
    const uint8_t* sa = smem + buf * Gm::STAGE;
#pragma unroll
    for (int i = 0; i < 2; ++i) asm volatile("" : "+v"(rb.q[i]));
    bad_s |= __builtin_amdgcn_ballot_w64(rb.s[0] == 0xFFu || rb.s[1] == 0xFFu);
    const i32x8 w0 = {rb.q[0][0], rb.q[0][1], rb.q[0][2], rb.q[0][3], 0, 0, 0, 0};
    const i32x8 w1 = {rb.q[1][0], rb.q[1][1], rb.q[1][2], rb.q[1][3], 0, 0, 0, 0};
    const int ws0 = (int)rb.s[0], ws1 = (int)rb.s[1];
    gload_b(rb, s + 2);
    // this lane's activation scale codes: byte lg of rows lr + 16 ms
    int xsc[MS];
    {
      const uint32_t* sx = (const uint32_t*)(sa + Gm::A_BYTES) + lr * MS;
      uint32_t wv[MS];
      if constexpr (MS >= 4) {
#pragma unroll
        for (int i = 0; i < MS; i += 4) {
          const i32x4 v = *(const i32x4*)(sx + i);
          wv[i] = v[0]; wv[i + 1] = v[1]; wv[i + 2] = v[2]; wv[i + 3] = v[3];
        }
      } else {
#pragma unroll
        for (int i = 0; i < MS; ++i) wv[i] = sx[i];
      }
#pragma unroll
      for (int i = 0; i < MS; ++i) xsc[i] = (int)((wv[i] >> (8 * lg)) & 0xFFu);
    }
    // fragment of subtile ms: chunks lg (K 16 lg ..) and lg + 4 (K 64 + 16 lg ..)
    auto lds_a = [&](int ms) {
      const int row = 16 * ms + lr;
      const i32x4 u = *(const i32x4*)(sa + row * 128 + 16 * swz(row, lg));
      const i32x4 v = *(const i32x4*)(sa + row * 128 + 16 * swz(row, lg + 4));
      return (i32x8){u[0], u[1], u[2], u[3], v[0], v[1], v[2], v[3]};
    };
    i32x8 fr[2];
    fr[0] = lds_a(0);
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
      if (ms + 1 < MS) fr[(ms + 1) & 1] = lds_a(ms + 1);
      // src0 fp4 (format 4), src1 fp8 e4m3 (format 0)
      acc[ms][0] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          w0, fr[ms & 1], acc[ms][0], 4, 0, 0, ws0, 0, xsc[ms]);
      acc[ms][1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          w1, fr[ms & 1], acc[ms][1], 4, 0, 0, ws1, 0, xsc[ms]);
      // pin the products here (a pure value would sink past the barrier) and
      // keep one subtile's fragment in flight: the live registers stay the
      // accumulators, two fragments and the next blocks' weights
      asm volatile("" : "+v"(acc[ms][0]), "+v"(acc[ms][1]));
      __builtin_amdgcn_sched_barrier(0);
    }
    store_a(ra, (buf + 2) & (kMxStages - 1));   // block s + 2 (loaded in block s - 2)
    gload_a(ra, s + 4);
  };

  WB rb0, rb1;
  gload_b(rb0, k0);
  gload_b(rb1, k0 + 1);
  gload_a(ra0, k0);
  gload_a(ra1, k0 + 1);
  store_a(ra0, 0);
  store_a(ra1, 1);
  gload_a(ra0, k0 + 2);
  gload_a(ra1, k0 + 3);
  __syncthreads();
  // block i = s - k0 reads stage i % 4 (staged in block i - 2) and stages
  // block i + 2 into the stage of block i - 2; the barrier after each pair
  // orders both (as in the FP8 kernel)
  int s = k0;
  for (; s + 2 <= k1; s += 2) {
    const int i = s - k0;
    block(s, i & 3, rb0, ra0);
    block(s + 1, (i + 1) & 3, rb1, ra1);
    __syncthreads();
  }
  if (s < k1) {
    block(s, (s - k0) & 3, rb0, ra0);
    __syncthreads();
  }
  if (bad_s && P.err && lane == 0) atomicOr(P.err, MOE_DEVERR_BIT_W4_SCALE);
  if constexpr (PART) {
    const int c0 = 16 * wave + 4 * lg;
    float* base = P.part + ((long)slot * P.p_rows + row0) * P.N;
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
      const int tr = 16 * ms + lr;
      if (tr < m) {
        *(f32x4*)(base + (long)tr * P.N + tl.n_lo + c0) = acc[ms][0];
        *(f32x4*)(base + (long)tr * P.N + tl.n_hi + c0) = acc[ms][1];
      }
    }
  } else {
    w4_epilogue<BM, true, LORA>(P, tl, acc, smem);
    __syncthreads();       // LDS is reused by the next tile
  }
}

// Whole tiles walked by persistent workgroups: XCD x (= blockIdx % 8) owns
// logical tiles [x*chunk, (x+1)*chunk)
template <int TBM, bool LORA>
__device__ __forceinline__ void mx_plain_tiles(const GemmParams& P, uint8_t* smem,
                                               const int* s_cum) {
  const int NT = P.I >> 7, NS = P.K >> 7;
  const int total = s_cum[P.G] * NT;
  const int xcd = blockIdx.x & 7, nper = gridDim.x >> 3, slot = blockIdx.x >> 3;
  const int chunk = (total + 7) >> 3;
  const int t_end = min(total, (xcd + 1) * chunk);
  for (int lt = xcd * chunk + slot; lt < t_end; lt += nper) {
    Tile tl = decode_tile<TBM, true>(P, lt, NT, s_cum);
    tl.g = __builtin_amdgcn_readfirstlane(tl.g);
    tl.row0 = __builtin_amdgcn_readfirstlane(tl.row0);
    tl.m = __builtin_amdgcn_readfirstlane(tl.m);
    tl.nt = __builtin_amdgcn_readfirstlane(tl.nt);
    tl.n_lo = __builtin_amdgcn_readfirstlane(tl.n_lo);
    tl.n_hi = __builtin_amdgcn_readfirstlane(tl.n_hi);
    if constexpr (TBM >= 128) {
      if (tl.m > 64) { mx_tile<128, false, LORA>(P, tl, smem, 0, NS); continue; }
    }
    if constexpr (TBM >= 64) {
      if (tl.m > 32) { mx_tile<64, false, LORA>(P, tl, smem, 0, NS); continue; }
    }
    mx_tile<32, false, LORA>(P, tl, smem, 0, NS);
  }
}

template <int TBM, bool LORA>
__global__ __launch_bounds__(kThreads) void moe_gemm_mx_kernel(GemmParams P) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int s_cum[kMaxGroups + 1];
  __shared__ int s_wsum[8];
  const int NT = P.I >> 7, NS = P.K >> 7;
  // SK_DEVICE launch (with LoRA only): return if the split-K kernel takes
  // this GEMM
  if (P.sk_mode == SK_DEVICE && sk_rule(tiles32(P.offsets, P.G, s_cum) * NT, NS)) return;
  tile_prefix<TBM>(P.offsets, P.G, s_cum, s_wsum);
  mx_plain_tiles<TBM, LORA>(P, smem, s_cum);
}

// Split-K (stream-K) variant for decode sizes, schedule as in the FP8 kernel
template <bool LORA>
__global__ __launch_bounds__(kThreads) void moe_gemm_mx_sk_kernel(GemmParams P) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int s_cum[kMaxGroups + 1];
  __shared__ int s_wsum[8];
  const int G = P.G;
  const int NT = P.I >> 7, NS = P.K >> 7;
  tile_prefix<kSkBM>(P.offsets, G, s_cum, s_wsum);
  if (P.sk_mode == SK_DEVICE && !sk_rule((long)s_cum[G] * NT, NS)) {
    // whole tiles here, as the plain kernel's 32-row class would run them
    // (without LoRA: with it the extra registers would cost the split-K
    // kernel its second workgroup per CU, and the plain kernel is launched
    // beside it)
    if constexpr (!LORA) mx_plain_tiles<kSkBM, LORA>(P, smem, s_cum);
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
    Tile tl = decode_tile<kSkBM, true>(P, t, NT, s_cum);
    tl.g = __builtin_amdgcn_readfirstlane(tl.g);
    tl.row0 = __builtin_amdgcn_readfirstlane(tl.row0);
    tl.m = __builtin_amdgcn_readfirstlane(tl.m);
    tl.nt = __builtin_amdgcn_readfirstlane(tl.nt);
    tl.n_lo = __builtin_amdgcn_readfirstlane(tl.n_lo);
    tl.n_hi = __builtin_amdgcn_readfirstlane(tl.n_hi);
    const int slot = b - sk_owner((long)t * NS, U, W);
    mx_tile<kSkBM, true, LORA>(P, tl, smem, k0, k1, slot);
    u += k1 - k0;
  }
}

template <int TBM, bool LORA>
static hipError_t run_mx(const GemmParams& P, long p_cap, int NT, hipStream_t s) {
  constexpr int shm = LORA ? std::max(MxGeo<TBM>::LDS, kLoraLds) : MxGeo<TBM>::LDS;
  static int per_cu = 0;
  if (per_cu == 0) {
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&moe_gemm_mx_kernel<TBM, LORA>),
        hipFuncAttributeMaxDynamicSharedMemorySize, shm);
    if (e != hipSuccess) return e;
    int nb = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &nb, reinterpret_cast<const void*>(&moe_gemm_mx_kernel<TBM, LORA>), kThreads, shm);
    if (e != hipSuccess) return e;
    per_cu = nb > 0 ? nb : 1;
  }
  long max_tiles = ((p_cap + TBM - 1) / TBM + P.G) * (long)NT;
  long nwg = std::min<long>(max_tiles, (long)num_cus() * per_cu);
  nwg = (nwg + 7) & ~7L;
  if (nwg == 0) return hipSuccess;
  GemmParams Q = P;
  Q.lds_bytes = shm;
  moe_gemm_mx_kernel<TBM, LORA><<<dim3((unsigned)nwg), dim3(kThreads), shm, s>>>(Q);
  return hipGetLastError();
}

template <bool LORA>
static hipError_t run_mx_sk(const GemmParams& P, long p_cap, hipStream_t s, int* sk_grid) {
  constexpr int shm = LORA ? std::max(MxGeo<kSkBM>::LDS, kLoraLds) : MxGeo<kSkBM>::LDS;
  static int per_cu = 0;
  if (per_cu == 0) {
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&moe_gemm_mx_sk_kernel<LORA>),
        hipFuncAttributeMaxDynamicSharedMemorySize, shm);
    if (e != hipSuccess) return e;
    int nb = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &nb, reinterpret_cast<const void*>(&moe_gemm_mx_sk_kernel<LORA>), kThreads, shm);
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
  moe_gemm_mx_sk_kernel<LORA><<<dim3((unsigned)grid), dim3(kThreads), shm, s>>>(Q);
  return hipGetLastError();
}

template <bool LORA>
static hipError_t launch_mx(const GemmParams& P, long p_cap, int NT, hipStream_t s,
                            int* sk_grid) {
  if (P.part) return run_mx_sk<LORA>(P, p_cap, s, sk_grid);
  const long hint = P.G > 0 ? p_cap / P.G : p_cap;
  if (hint <= 32) return run_mx<32, LORA>(P, p_cap, NT, s);
  if (hint <= 64) return run_mx<64, LORA>(P, p_cap, NT, s);
  return run_mx<128, LORA>(P, p_cap, NT, s);
}

hipError_t launch_gemm1_mx(const GemmParams& P, long p_cap, int NT, hipStream_t s,
                           int* sk_grid) {
  return P.z ? launch_mx<true>(P, p_cap, NT, s, sk_grid)
             : launch_mx<false>(P, p_cap, NT, s, sk_grid);
}

}  // namespace moe
