// Shared pieces of the grouped expert GEMM kernels: parameters, the
// device-side tile and split-K schedules, and the BF16 epilogue (the FP8 and
// 4-bit kernels have their own).
//
// Epilogue semantics: g' = min(g, L), u' = clamp(u, -L, L),
// h = g' sigmoid(alpha g') (u' + beta) ("[Moe] Fix flashinfer_trtllm silently
// dropping swiglu_limit clamped SwiGLU activation", sglang PR #39920,
// "Modifications"; "fix(sm90): support parameterized SwiGLU in FP8
// MegaMoE", DeepGEMM PR #445, "Summary"), after each half's own global scale
// and the LoRA delta in true units ("FlashInfer 0.6.18 SM100a+SM103a
// MoE-LoRA AOT" release notes, "Changes since 1b699bf"). BF16 and INT4
// layers round h to bf16.
#pragma once
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace moe {

// FMT_MXFP4_A8: MXFP4 weights with MXFP8 activations into GEMM1 (gemm_mx.hip);
// its GEMM2 is the MXFP4 kernel
enum { FMT_BF16 = 0, FMT_FP8 = 1, FMT_INT4 = 2, FMT_NVFP4 = 3, FMT_MXFP4 = 4, FMT_MXFP4_A8 = 5 };

constexpr int kThreads = 512;
constexpr int kMaxGroups = 1024;
constexpr int KS = 64;               // K elements per pipeline stage

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

struct GemmParams {
  // A side
  const uint8_t* a;          // x (GEMM1: gathered by token) or h (GEMM2)
  const float* as;           // FP8 per-row scales [rows][K/128]; MXFP4 W4A8: the
                             // e8m0 codes [rows][K/32] (bytes, read as such)
  long a_ld;                 // bytes per A row
  const int* sorted_pair;    // GEMM1: sorted row -> pair id
  long T;
  int top_k;
  // B side
  const uint8_t* w;          // [G][N][K] codes (bytes; INT4 packed)
  const void* wsc;           // FP8 fp32 [G][N/128][K/128]; INT4 bf16 [G][N][K/32];
                             // NVFP4 e4m3 [G][N][K/16]; MXFP4 e8m0 [G][N][K/32]
  int N, K, G;
  const int* offsets;
  int I;
  // global scales: GEMM1 [G][2] (gate, up) in the epilogue; GEMM2 (FP4
  // formats) [G] after the K loop
  const float* gscale;
  float alpha, beta, limit;
  // LoRA delta of this GEMM (GEMM1: on [gate | up]; GEMM2: on the down
  // projection): acc += lora_scale * z[row] . B[g][column], z fp32
  // [rows][rank], B bf16 [G][N][rank], groups g < lora_groups
  const float* z;
  const uint16_t* lora_B;
  int lora_rank, lora_groups;
  float lora_scale;
  // a batch of adapters: B is [n_adapters][lora_groups][N][rank] and row r
  // uses adapter zad[r] (-1: none, its z row is zero)
  int n_adapters;
  const int* zad;
  uint8_t* h;                // GEMM1 out: e4m3 [p_cap][I] or bf16 [p_cap][I]
  float* hs;
  uint16_t* h_lora;          // GEMM1 out (FP8 layers), nullable: bf16 [p_cap][I]
                             // SwiGLU output before the re-quantisation
  // GEMM2 out: fp32 rows [p_cap][N] (BF16 layers), or for the FP8 and 4-bit
  // kernels int16 rows y16 [p_cap][N] with one power-of-two scale exponent
  // per row and 16 columns, ye [p_cap][N / 16] (see store_y16)
  float* y;
  uint16_t* y16;
  int8_t* ye;
  // split-K (decode sizes): fp32 partial sums [kSkSlots][p_rows][N]
  float* part;
  long p_rows;
  int lds_bytes;             // the launch's dynamic LDS (the LoRA epilogue's room)
  int* err;                  // nullable: 4-bit range problems (MOE_DEVERR_BIT_*)
  int sk_mode;               // SK_DEVICE: decide plain / split-K on the device
};

// Dynamic LDS of the FP8 / 4-bit instantiations with LoRA code: room for a
// tile's z rows and the B blocks of 8 rank-16 adapters at once (see
// lora_delta_tile); those kernels run one workgroup per CU either way.
constexpr int kLoraLds = 80 * 1024;
constexpr int kLoraSlots = 16;           // most adapters staged per round


// ---------------------------------------------------------------------------
// device-side tile schedule: M-tiles of BM rows per group, NT column tiles
// ---------------------------------------------------------------------------

// Fills s_cum[0..G] with the exclusive prefix of ceil(rows_g / BM), called
// by the whole workgroup (a multiple of 64 threads, at least 256; s_wsum
// holds one int per wave); G <= kMaxGroups, each thread taking
// kMaxGroups / blockDim.x consecutive groups.
template <int BM>
__device__ __forceinline__ void tile_prefix(const int* offsets, int G, int* s_cum,
                                            int* s_wsum) {
  constexpr int QMAX = kMaxGroups / 256;     // workgroups of at least 256 threads
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = (kMaxGroups + (int)blockDim.x - 1) / (int)blockDim.x;   // groups per thread
  // the thread's q + 1 offsets, all loads issued before the first use
  // (indices past G re-read offsets[G])
  int o[QMAX + 1], tl[QMAX];
#pragma unroll
  for (int i = 0; i <= QMAX; ++i) o[i] = i <= q ? offsets[min(tid * q + i, G)] : 0;
  int v = 0;
#pragma unroll
  for (int i = 0; i < QMAX; ++i) {
    tl[i] = (i < q && tid * q + i < G) ? (o[i + 1] - o[i] + BM - 1) / BM : 0;
    v += tl[i];
  }
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int t = __shfl_up(incl, d, 64);
    if (lane >= d) incl += t;
  }
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  int run = incl - v;
  for (int i = 0; i < wave; ++i) run += s_wsum[i];
#pragma unroll
  for (int i = 0; i < QMAX; ++i)
    if (i < q && tid * q + i < G) {
      s_cum[tid * q + i] = run;
      run += tl[i];
    }
  if (tid == 0) {
    int tot = 0;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) tot += s_wsum[i];
    s_cum[G] = tot;
  }
  __syncthreads();
}

struct Tile {
  int g, row0, m, nt, n_lo, n_hi;
};

// ---------------------------------------------------------------------------
// stream-K schedule for decode sizes, where the tiles of a grouped GEMM are
// fewer than the CUs: the U = tiles * NS (tile, K block) units are cut into
// W equal contiguous ranges, one per workgroup; workgroup w owns units
// [w U / W, (w + 1) U / W). W is capped so that every range holds at least
// ceil(NS / (kSkSlots - 1)) units, which bounds the workgroups meeting one
// tile -- its partial-sum slots -- to kSkSlots. When the tiles already fill
// 80..100 % of the grid, W = tiles: one whole tile per workgroup, one slot.
// With more tiles than workgroups each range spans several whole tiles and
// at most two split ones, so the work is balanced to one K block. Partials
// are reduced in slot order by the consumer, so results do not depend on
// timing. Producer and consumers evaluate this from the same (tiles, NS,
// grid).
// ---------------------------------------------------------------------------
// the split-K rule on a tile count (tiles of kSkBM rows times NT): the
// host applies it to its shape-only bound, the kernels of an SK_DEVICE
// launch to the real count
__host__ __device__ inline bool sk_rule(long tiles, int NS) {
  if (tiles <= 0 || tiles > kSkMaxTiles) return false;
  const long waves = (tiles + kSkCUs - 1) / kSkCUs;
  return (waves * kSkCUs - tiles) * NS >= 8 * kSkCUs;
}

// sum over the G groups of ceil(rows / kSkBM), for the whole workgroup
// (blockDim.x threads, a multiple of 64; s_red holds 16 ints)
__device__ __forceinline__ long tiles32(const int* offsets, int G, int* s_red) {
  int v = 0;
  for (int g = threadIdx.x; g < G; g += blockDim.x)
    v += (offsets[g + 1] - offsets[g] + kSkBM - 1) / kSkBM;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = v;
  __syncthreads();
  long tot = 0;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) tot += s_red[i];
  __syncthreads();
  return tot;
}

__device__ __forceinline__ int sk_workgroups(long tiles, int NS, int grid) {
  if (tiles <= grid && tiles * 5 >= 4L * grid) return (int)tiles;
  const int lmin = (NS + kSkSlots - 2) / (kSkSlots - 1);
  const long w = tiles * NS / lmin;
  return (int)(w < 1 ? 1 : (w < grid ? w : grid));
}
// the workgroup whose range holds unit u
__device__ __forceinline__ int sk_owner(long u, long U, int W) {
  return (int)(((u + 1) * W - 1) / U);
}
// number of partial slots (consecutive workgroups) of the tile whose units
// start at uf
__device__ __forceinline__ int sk_nslots(long uf, int NS, long U, int W) {
  return sk_owner(uf + NS - 1, U, W) - sk_owner(uf, U, W) + 1;
}
// the group owning sorted row r: last g with s_off[g] <= r (LDS copy of
// the offsets; empty groups share their successor's offset)
__device__ __forceinline__ int group_of_row(const int* s_off, int G, int r) {
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_off[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Logical tile lt -> group, first sorted row, valid rows, column halves.
// GEMM1: lo = gate rows nt*128.., hi = up rows I + nt*128..;
// GEMM2: lo/hi = output columns nt*w2.. and nt*w2 + w2/2.. (hi = lo if
// ragged); w2 = 256 for 8-wave workgroups, 128 for 4-wave ones.
template <int BM, bool G1>
__device__ __forceinline__ Tile decode_tile(const GemmParams& P, int lt, int NT,
                                            const int* s_cum, int w2 = 256) {
  Tile t;
  const int mt = lt / NT;
  t.nt = lt - mt * NT;
  int glo = 0, ghi = P.G - 1;                 // last g with s_cum[g] <= mt
  while (glo < ghi) {
    int mid = (glo + ghi + 1) >> 1;
    if (s_cum[mid] <= mt) glo = mid; else ghi = mid - 1;
  }
  t.g = glo;
  t.row0 = P.offsets[t.g] + (mt - s_cum[t.g]) * BM;
  t.m = min(BM, P.offsets[t.g + 1] - t.row0);
  if (G1) {
    t.n_lo = t.nt * 128;
    t.n_hi = P.I + t.nt * 128;
  } else {
    t.n_lo = t.nt * w2;
    t.n_hi = (t.n_lo + w2 / 2 < P.N) ? t.n_lo + w2 / 2 : t.n_lo;
  }
  return t;
}

// Row index of the A operand for sorted row r: the token (GEMM1 gathers x)
// or r itself (GEMM2 reads h in sorted order).
template <bool G1>
__device__ __forceinline__ long a_source_row(const GemmParams& P, int r) {
  if (!G1) return r;
  int p = P.sorted_pair[r];
  long npr = P.T * (long)P.top_k;
  return (p < npr) ? (long)(p / P.top_k) : (long)(p - npr);
}

// LoRA delta on a tile of the FP8 / 4-bit kernels, whose weights are the
// MFMA's first operand: acc[ms][ns][r] is row 16 ms + lane % 16 of the tile
// and column (ns ? n_hi : n_lo) + 16 wave + 4 (lane / 16) + r.
//   acc += sum_q (lora_scale * z[row][q]) * B[a(row)][g][column][q]
// on the matrix cores: v_mfma_f32_16x16x16bf16_1k with the B rows as the
// first operand (lane: column 16 wave + lane % 16, ranks 4 (lane / 16) ..
// + 3) and z' = lora_scale * z as the second. z' is fp32; it enters as the
// exact sum of three bf16 terms (z1 = bf16(z'), z2 = bf16(z' - z1),
// z3 = z' - z1 - z2), so every product is exact and only the fp32
// accumulation rounds. Ranks are padded with zeros to 16 (or 32).
// The tile's distinct adapters (one when there is no batch of adapters)
// are listed in ascending order; their B blocks ([lo 128 | hi 128 columns]
// [ranks] bf16) are staged in LDS after the z' rows, as many per round as
// fit, and for each adapter the rows that use it take its product (the
// others multiply zeros, which leaves their accumulators unchanged). So a
// row's result depends only on its own adapter: a batch in which every
// token uses adapter a gives the one-adapter result bit for bit. Rows
// without an adapter (z = 0) are skipped. The hi half is read only when
// hi_ok (otherwise the lo columns are staged twice and the hi values never
// stored). Every thread of the workgroup calls it (barriers inside).
typedef short lora_s4 __attribute__((ext_vector_type(4)));

// three bf16 terms whose sum is the fp32 pair (x, y) exactly (normal range),
// packed two per dword: t[0] = (x1 | y1 << 16), t[1] = (x2 ...), t[2] = ...
__device__ __forceinline__ void split3_bf16(float x, float y, uint32_t (&t)[3]) {
  const uint32_t x1 = f32_to_bf16_bits(x), y1 = f32_to_bf16_bits(y);
  const float rx = x - __uint_as_float(x1 << 16), ry = y - __uint_as_float(y1 << 16);
  const uint32_t x2 = f32_to_bf16_bits(rx), y2 = f32_to_bf16_bits(ry);
  const float sx = rx - __uint_as_float(x2 << 16), sy = ry - __uint_as_float(y2 << 16);
  t[0] = x1 | (y1 << 16);
  t[1] = x2 | (y2 << 16);
  t[2] = f32_to_bf16_bits(sx) | (f32_to_bf16_bits(sy) << 16);
}

// GEMM2's rows for the weighted combine in half the bytes of fp32, as block
// floating point: each run of 16 columns of a row (the 4 lanes r, r + 16,
// r + 32, r + 48 hold 4 consecutive columns each) shares one power-of-two
// scale 2^e and every value is an int16 multiple of it. With m the run's
// largest finite magnitude, m in [2^(E-1), 2^E), e = E - 15 (at least -128),
// so q = round-to-nearest-even(v / 2^e) lies in [-32767, 32767] (|v| <= m <
// 2^(e+15); a value that rounds to 2^15 is clamped, one unit) and the error
// of every value is at most 2^e / 2 <= 2^-15 m (2^e when clamped). A value
// that is not finite is stored as -32768 and read back as NaN. The combine
// multiplies q by 2^e exactly. Called by all 64 lanes of the wave (the run
// maximum is a lane exchange); ok: this lane's row is valid.
__device__ __forceinline__ void store_y16(const GemmParams& P, long row, int col,
                                          const f32x4& v, bool ok) {
  float m = 0.0f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float a = fabsf(v[r]);
    m = fmaxf(m, a <= 3.402823466e38f ? a : 0.0f);
  }
  m = max_across_rows(m);
  const int e = max(__builtin_amdgcn_frexp_expf(m) - 15, -128);
  if (ok) {
    int q[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float t = __builtin_rintf(__builtin_amdgcn_ldexpf(v[r], -e));
      q[r] = fabsf(v[r]) <= 3.402823466e38f
                 ? (int)__builtin_amdgcn_fmed3f(t, -32767.0f, 32767.0f)
                 : -32768;
    }
    const uint2 w = {(uint32_t)(q[0] & 0xFFFF) | ((uint32_t)q[1] << 16),
                     (uint32_t)(q[2] & 0xFFFF) | ((uint32_t)q[3] << 16)};
    *(uint2*)(P.y16 + row * P.N + col) = w;
    if ((threadIdx.x & 48) == 0) P.ye[row * (P.N >> 4) + (col >> 4)] = (int8_t)e;
  }
}

template <int BM>
__device__ __forceinline__ void lora_delta_tile(const GemmParams& P, const Tile& t,
                                                f32x4 (&acc)[BM / 16][2], uint8_t* smem,
                                                bool hi_ok) {
  constexpr int MS = BM / 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int g = t.g, row0 = t.row0, m = t.m;
  const int R = P.lora_rank;
  const int Rp = R <= 16 ? 16 : 32;                  // padded ranks
  const bool batch = P.n_adapters > 1;
  const int nhi = hi_ok ? t.n_hi : t.n_lo;
  // LDS: z' [BM][Rp] fp32 | row -> list index [BM] | adapter list [BM] |
  // list length | B slots, each [lo | hi][128][Rp] bf16 + a 16-byte pad
  // that puts the same column of different slots in different banks
  float* sz = (float*)smem;
  int* s_idx = (int*)(sz + BM * Rp);
  int* s_list = s_idx + BM;
  int* s_n = s_list + BM;
  uint8_t* sb = (uint8_t*)(s_n + 4);
  const int blk = 128 * Rp * 2;                      // bytes of one 128-column block
  const int ss = 2 * blk + 16;
  // LoRA launches give kLoraLds bytes: at least 3 slots at 32 ranks and
  // BM = 128 (the floor of 1 only keeps the round loop finite)
  const int slots = max(1, min(kLoraSlots, (P.lds_bytes - (int)(sb - smem)) / ss));
  for (int i = tid; i < BM * Rp; i += kThreads) {
    const int tr = i / Rp, q = i - tr * Rp;
    sz[i] = (q < R && tr < m) ? P.lora_scale * P.z[(long)(row0 + tr) * R + q] : 0.0f;
  }
  if (wave == 0) {
    // distinct adapters of the tile's rows, ascending (one wave minimum each)
    constexpr int RPL = (BM + 63) / 64;              // rows per lane
    int ad[RPL], ix[RPL];
#pragma unroll
    for (int j = 0; j < RPL; ++j) {
      const int tr = lane + 64 * j;
      ad[j] = tr < m ? (batch ? P.zad[row0 + tr] : 0) : -1;
      ix[j] = -1;
    }
    int n = 0;
    while (true) {
      int cand = 0x7FFFFFFF;
#pragma unroll
      for (int j = 0; j < RPL; ++j)
        if (ad[j] >= 0 && ix[j] < 0) cand = min(cand, ad[j]);
      cand = wave_min_i32(cand);
      if (cand == 0x7FFFFFFF) break;
#pragma unroll
      for (int j = 0; j < RPL; ++j)
        if (ad[j] == cand) ix[j] = n;
      if (lane == 0) s_list[n] = cand;
      ++n;
    }
#pragma unroll
    for (int j = 0; j < RPL; ++j) {
      const int tr = lane + 64 * j;
      if (tr < BM) s_idx[tr] = ix[j];
    }
    if (lane == 0) s_n[0] = n;
  }
  __syncthreads();
  const int n = s_n[0];
  for (int base = 0; base < n; base += slots) {
    const int cnt = min(slots, n - base);
    // stage the B blocks of adapters base .. base + cnt - 1
    if (R == Rp) {
      // 16-byte chunks in rounds of 8 per thread, each round's loads
      // issued before its LDS stores
      const int per = 2 * blk / 16;                  // chunks per slot
      const int total = cnt * per;
      for (int c0 = 0; c0 < total; c0 += 8 * kThreads) {
        i32x4 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int c = min(c0 + tid + i * kThreads, total - 1);
          const int j = c / per, rem = c - j * per;
          const int half = rem >= per / 2, off = rem - half * (per / 2);
          const uint16_t* src = P.lora_B +
              ((long)s_list[base + j] * P.lora_groups + g) * P.N * R + (long)(half ? nhi : t.n_lo) * R;
          v[i] = *(const i32x4*)((const uint8_t*)src + 16 * off);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int c = c0 + tid + i * kThreads;
          if (c < total) {
            const int j = c / per, rem = c - j * per;
            const int half = rem >= per / 2, off = rem - half * (per / 2);
            *(i32x4*)(sb + j * ss + half * blk + 16 * off) = v[i];
          }
        }
      }
    } else {                                         // ranks padded with zeros
      const int per = 2 * 128 * Rp;                  // elements per slot
      for (int c = tid; c < cnt * per; c += kThreads) {
        const int j = c / per, rem = c - j * per;
        const int col = rem / Rp, q = rem - col * Rp;
        const int half = col >= 128, cc = col - 128 * half;
        uint16_t v = 0;
        if (q < R)
          v = P.lora_B[((long)s_list[base + j] * P.lora_groups + g) * P.N * R +
                       (long)((half ? nhi : t.n_lo) + cc) * R + q];
        *(uint16_t*)(sb + j * ss + half * blk + (cc * Rp + q) * 2) = v;
      }
    }
    __syncthreads();
    const int colb = (16 * wave + lr) * Rp * 2;      // the lane's B column
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
      const int row = 16 * ms + lr;
      const int k = s_idx[row] - base;               // the row's slot this round
      for (int ks = 0; ks < Rp; ks += 16) {
        const f32x4 zv = *(const f32x4*)(sz + row * Rp + ks + 4 * lg);
        uint32_t za[3], zb[3];
        split3_bf16(zv[0], zv[1], za);
        split3_bf16(zv[2], zv[3], zb);
        for (int j = 0; j < cnt; ++j) {
          if (!__ballot(k == j)) continue;           // no row of this subtile uses it
          const uint8_t* bj = sb + j * ss + colb + (ks + 4 * lg) * 2;
          const lora_s4 blo = *(const lora_s4*)bj;
          const lora_s4 bhi = *(const lora_s4*)(bj + blk);
          const bool take = k == j;
#pragma unroll
          for (int u = 0; u < 3; ++u) {
            const uint2 zz = take ? make_uint2(za[u], zb[u]) : make_uint2(0u, 0u);
            const lora_s4 zo = __builtin_bit_cast(lora_s4, zz);
            acc[ms][0] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(blo, zo, acc[ms][0], 0, 0, 0);
            acc[ms][1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(bhi, zo, acc[ms][1], 0, 0, 0);
          }
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// epilogues. acc[ms][ns] holds rows rbase + 16 ms + 4 (lane/16) + r and
// column (ns < 2 ? lo : hi) + wn*32 + (ns & 1)*16 + lane%16.
// smem: at least max(BM*128*2, R*BM*4, BM*128 + 16*BM) bytes, free to reuse.
// ---------------------------------------------------------------------------
template <int BM, bool G1>
__device__ __forceinline__ void tile_epilogue(const GemmParams& P, const Tile& t,
                                              f32x4 (&acc)[BM / 32][4], uint8_t* smem) {
  constexpr int MS = BM / 32;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int lr = lane & 15, lg = lane >> 4;
  const int rbase = wm * (BM / 2);
  const int g = t.g, row0 = t.row0, m = t.m, nt = t.nt;
  const bool hi_ok = G1 || t.n_hi != t.n_lo;
  if constexpr (G1) {
    // gate = ns 0,1 ; up = ns 2,3 (same h columns): global scales first
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
    const int nhi = hi_ok ? t.n_hi : t.n_lo;      // an absent hi half is never stored
    if (P.n_adapters <= 1) {
      const uint16_t* Bg = P.lora_B + (long)g * P.N * R;
      for (int q = 0; q < R; ++q) {
        float bgv[2], buv[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          int c = wn * 32 + j * 16 + lr;
          bgv[j] = P.lora_scale * bf16_bits_to_f32(Bg[(long)(t.n_lo + c) * R + q]);
          buv[j] = P.lora_scale * bf16_bits_to_f32(Bg[(long)(nhi + c) * R + q]);
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
    } else {
      // a batch of adapters: each row's B (rows without one have z = 0)
#pragma unroll
      for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tr = rbase + ms * 16 + 4 * lg + r;
          const int a = max(P.zad[row0 + (tr < m ? tr : 0)], 0);
          const uint16_t* Bg = P.lora_B + ((long)a * P.lora_groups + g) * P.N * R;
          for (int q = 0; q < R; ++q) {
            const float zq = sz[q * BM + tr];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              int c = wn * 32 + j * 16 + lr;
              acc[ms][j][r] = fmaf(zq, P.lora_scale * bf16_bits_to_f32(
                                           Bg[(long)(t.n_lo + c) * R + q]), acc[ms][j][r]);
              acc[ms][j + 2][r] = fmaf(zq, P.lora_scale * bf16_bits_to_f32(
                                               Bg[(long)(nhi + c) * R + q]), acc[ms][j + 2][r]);
            }
          }
        }
    }
    __syncthreads();
  }
  if constexpr (!G1) {
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
      for (int ns = 0; ns < 4; ++ns) {
        int col = (ns < 2 ? t.n_lo : t.n_hi) + wn * 32 + (ns & 1) * 16 + lr;
        bool colok = (ns < 2) || hi_ok;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          int tr = rbase + ms * 16 + 4 * lg + r;
          if (tr < m && colok) P.y[(long)(row0 + tr) * P.N + col] = acc[ms][ns][r];
        }
      }
    return;
  } else {
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
    {
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
}

int num_cus();

// Blockwise-FP8 grouped GEMM (gemm_fp8.hip). With P.part set it runs the
// stream-K schedule and leaves partial sums for sk_grid workgroups; the
// consumer (launch_gemm1_sk_epilogue, or the combine) reduces them.
hipError_t launch_gemm_fp8(const GemmParams& P, bool g1, long p_cap, int NT, hipStream_t s,
                           int* sk_grid = nullptr);
// GEMM1 epilogue after split-K (sk_epilogue.hip); fp8h: e4m3 h + scales
// (FP8 layers), else bf16 h (4-bit layers)
hipError_t launch_gemm1_sk_epilogue(const GemmParams& P, int sk_grid, bool fp8h, hipStream_t s);

// 4-bit grouped GEMMs (gemm_w4.h: INT4, NVFP4, MXFP4), same conventions;
// GEMM1 reads f16 activations prepared by launch_act_f16p.
hipError_t launch_gemm_w4(int fmt, const GemmParams& P, bool g1, long p_cap, int NT,
                          hipStream_t s, int* sk_grid = nullptr);
hipError_t launch_gemm_int4(const GemmParams& P, bool g1, long p_cap, int NT, hipStream_t s,
                            int* sk_grid);
hipError_t launch_gemm_nvfp4(const GemmParams& P, bool g1, long p_cap, int NT, hipStream_t s,
                             int* sk_grid);
hipError_t launch_gemm_mxfp4(const GemmParams& P, bool g1, long p_cap, int NT, hipStream_t s,
                             int* sk_grid);
// GEMM1 of the MXFP4 W4A8 layers on the block-scaled matrix cores
// (gemm_mx.hip): A = MXFP8 codes, P.as their e8m0 codes; bf16 h
hipError_t launch_gemm1_mx(const GemmParams& P, long p_cap, int NT, hipStream_t s,
                           int* sk_grid);
// err (nullable): MOE_DEVERR_BIT_F16_RANGE is ORed in for a value beyond f16
hipError_t launch_act_f16p(const void* x, long T, int H, void* out, int* err, hipStream_t s);

}  // namespace moe
