// Router GEMM fused with the sigmoid-gate epilogue, with an optional
// selection bias and the packed (id << 16 | bf16 weight) output.
//
// "Enable and fuse the Inkling MoE gate epilogue on Intel XPU" (sglang PR
// #36385): the 258-column gate GEMM that feeds the epilogue, ranking by
// iterative masked-max passes ("3. Performance"), weights as
// exp(lp - logsumexp(lp)) with lp = logsigmoid(x) ("2. Correctness"); the
// router-epilogue commit message: the ranking key is sigmoid(logits) + bias
// with the bias covering the routed columns only, the winner carries its
// RAW logit out of the top-k loop, sink columns join only the normaliser,
// the global scale multiplies the weights, and the packed form is read back
// with & 0xFFFF.
//
// GEMM: logits[t][c] = sum_h x[t][h] Wg[c][h] with bf16 operands on
// v_mfma_f32_16x16x32_bf16 and fp32 accumulation. A workgroup of 4 waves
// owns 32 tokens (two 16-token subtiles) and every logit column; wave w owns
// the 16-column subtiles w, w + 4, w + 8, ... of both token subtiles, so each
// router-weight element is read by exactly one wave, straight from memory
// into registers as the MFMA's first operand (a lane's four accumulators are
// then four consecutive columns of one token), while the 32 token rows are
// shared by the four waves through the L1 cache. Two K steps of 32 are in
// flight. With enough tokens for the whole GPU (one launch) the workgroup
// puts its 32 x C logits in LDS and runs the epilogue itself; with few
// tokens the K range is split over workgroups that write fp32 partial sums,
// and a second kernel adds them in split order and runs the same epilogue.
//
// Epilogue: with a selection bias the ranking keys sigmoid(logit) + bias
// (fp64-evaluated sigmoid, see sigmoid_key) are computed first by the whole
// workgroup into LDS, one key per thread and pass; then one 16-lane group
// per token row (one DPP row: max, min and sum over the group take four
// steps). Lane l of a group holds columns l, l + 16, ...; each of the k
// passes takes the group maximum of the lanes' best untaken keys, then the
// lowest column holding it, so equal keys go to the lower column; the owner
// lane marks it taken and publishes the raw logit. Then lane j < k holds
// slot j, lanes k .. k + S - 1 the sinks, and the renormalisation is a group
// max and a group sum.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kGBM = 32;          // tokens per GEMM workgroup
constexpr int kGRows = 4;         // rows per reduce + epilogue workgroup
constexpr int kGMaxSplits = 32;   // K splits at most
constexpr int kGThreads = 256;    // 4 waves
constexpr int kGDepth = 4;        // K steps of the GEMM ring (3 in flight)

struct GateP {
  const uint8_t* x;     // bf16 [T][H]
  const uint8_t* wg;    // bf16 [NC][H]
  long T;
  int H, NC, n_routed, n_sink, k;
  int NS;               // 16-column subtiles, ceil(NC / 16)
  int steps;            // K steps of 32 per split
  int S;                // splits
  const float* bias;    // [n_routed] or NULL
  float scale;
  float* part;          // [S][T][16 NS] partial logits (S > 1)
  float* logits;        // [T][NC] or NULL
  int* ids;
  float* w;
  float* sw;
  int* packed;          // [T][k] or NULL
};

// ---------------------------------------------------------------- GEMM --
// acc[j][ts] holds columns 16 (4 j + wave) + 4 (lane / 16) + r, r = 0..3, of
// token t0 + 16 ts + lane % 16 over the split's K range.
template <int NQ>
__device__ __forceinline__ void gate_gemm(const GateP& P, f32x4 (&acc)[NQ][2],
                                          long t0, int split) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const long rowb = (long)P.H * 2;
  const int st0 = split * P.steps;
  const int nst = min(P.steps, P.H / 32 - st0);
  const long kb = ((long)st0 * 32 + 8 * lg) * 2;
  const uint8_t* xa[2];
#pragma unroll
  for (int ts = 0; ts < 2; ++ts) {
    const long row = min(t0 + 16 * ts + lr, P.T - 1);   // rows past T: discarded
    xa[ts] = P.x + row * rowb + kb;
  }
  const uint8_t* wa[NQ];
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int col = min(16 * (4 * j + wave) + lr, P.NC - 1);   // padding: discarded
    wa[j] = P.wg + (long)col * rowb + kb;
  }
#pragma unroll
  for (int j = 0; j < NQ; ++j)
#pragma unroll
    for (int ts = 0; ts < 2; ++ts) acc[j][ts] = (f32x4){0.f, 0.f, 0.f, 0.f};
  // this wave's column subtiles: 4 j + wave < NS for j < nq (wave-uniform)
  const int nq = (P.NS - wave + 3) >> 2;

  struct Fr { i32x4 a[NQ]; i32x4 b[2]; };
  // loads are unconditional (past the end they re-read the last step) so the
  // wait counts stay static: kGDepth steps in flight, a step's registers
  // reloaded as soon as its MFMAs have issued
  auto load = [&](Fr& f, int st) {
    const long off = (long)min(st, nst - 1) * 64;
#pragma unroll
    for (int j = 0; j < NQ; ++j) f.a[j] = *(const i32x4*)(wa[j] + off);
#pragma unroll
    for (int ts = 0; ts < 2; ++ts) f.b[ts] = *(const i32x4*)(xa[ts] + off);
  };
  auto mma = [&](const Fr& f, int st) {
    if (st >= nst) return;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      if (j >= nq) break;
#pragma unroll
      for (int ts = 0; ts < 2; ++ts)
        acc[j][ts] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, f.a[j]), __builtin_bit_cast(bf16x8, f.b[ts]),
            acc[j][ts], 0, 0, 0);
    }
  };
  constexpr int D = kGDepth;
  Fr f[D];
  // the scheduling barriers keep the loads in step order: loads complete in
  // issue order, so a step is ready once the later steps' loads are the only
  // ones outstanding
#pragma unroll
  for (int u = 0; u < D; ++u) {
    load(f[u], u);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int st = 0; st < nst; st += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      mma(f[u], st + u);
      __builtin_amdgcn_sched_barrier(0);
      load(f[u], st + u + D);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// ------------------------------------------------------------ epilogue --
// Ranking keys of rows 0 .. rows - 1 (logits in LDS at L, pitch LP) into
// LDS at Kd (same pitch), computed by the whole workgroup: sigmoid(logit) +
// bias[c] over the routed columns. Only with a selection bias (without one
// the key is the raw logit and the rows are ranked in place).
__device__ __forceinline__ void gate_keys(const GateP& P, const float* L, float* Kd, int LP,
                                          int rows) {
  for (int r = 0; r < rows; ++r)
    for (int c = threadIdx.x; c < P.n_routed; c += kGThreads)
      Kd[r * LP + c] = sigmoid_key(L[r * LP + c]) + P.bias[c];
}

// One token row per 16-lane group. L points at the row's fp32 logits in LDS
// (columns 0 .. NC - 1 valid), Kr at its ranking keys (gate_keys; L itself
// without a bias). NV >= ceil(n_routed / 16). Taken and non-candidate
// columns hold key -inf; the winner's raw logit is read back from L.
template <int NV>
__device__ __forceinline__ void route_row16(const GateP& P, const float* L, const float* Kr,
                                            long row, bool row_ok) {
  const int lr = threadIdx.x & 15;
  float key[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = lr + 16 * i;
    key[i] = c < P.n_routed ? Kr[c] : -INFINITY;
  }
  float my_x = 0.0f;
  int my_c = 0;
  for (int j = 0; j < P.k; ++j) {
    float bv = key[0];
    int bi = 0;
#pragma unroll
    for (int i = 1; i < NV; ++i)
      if (key[i] > bv) { bv = key[i]; bi = i; }      // first maximum: lowest column
    const float m = row16_reduce(bv, OpMax{});
    const int wc = row16_reduce(bv == m ? lr + 16 * bi : 0x7FFFFFFF, OpMinI{});
    const int bo = (wc & 15) == lr ? wc >> 4 : -1;     // owner lane: take it
#pragma unroll
    for (int i = 0; i < NV; ++i) key[i] = i == bo ? -INFINITY : key[i];
    if (lr == j) { my_c = wc; my_x = L[wc]; }          // carry the raw logit
  }
  const bool active = lr < P.k + P.n_sink;
  if (lr >= P.k && active) my_x = L[P.n_routed + (lr - P.k)];
  float lp = active ? fminf(my_x, 0.0f) - log1pf(expf(-fabsf(my_x))) : -INFINITY;
  const float m = row16_reduce(lp, OpMax{});
  const float e = active ? expf(lp - m) : 0.0f;
  const float wt = e / row16_reduce(e, OpSum{}) * P.scale;
  if (!row_ok) return;
  if (lr < P.k) {
    P.ids[row * P.k + lr] = my_c;
    P.w[row * P.k + lr] = wt;
    if (P.packed) P.packed[row * P.k + lr] = (int)(((uint32_t)my_c << 16) | f32_to_bf16_bits(wt));
  } else if (active) {
    P.sw[row * P.n_sink + (lr - P.k)] = wt;
  }
}

// ------------------------------------------------------------- kernels --
// S == 1: GEMM over the whole K, logits to LDS, epilogue for the 32 rows.
// LDS: the logits [kGBM][LP], then (with a bias) their keys [kGBM][LP].
template <int NQ>
__global__ __launch_bounds__(kGThreads) void gate_fused_kernel(GateP P) {
  extern __shared__ __attribute__((aligned(16))) float sl[];
  const int LP = 16 * P.NS + 4;                    // row pitch (floats)
  const long t0 = (long)blockIdx.x * kGBM;
  f32x4 acc[NQ][2];
  gate_gemm<NQ>(P, acc, t0, 0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    if (4 * j + wave >= P.NS) continue;
#pragma unroll
    for (int ts = 0; ts < 2; ++ts)
      *(f32x4*)(sl + (16 * ts + lr) * LP + 16 * (4 * j + wave) + 4 * lg) = acc[j][ts];
  }
  __syncthreads();
  const int rows = (int)min((long)kGBM, P.T - t0);
  if (P.logits) {
    for (int i = threadIdx.x; i < rows * P.NC; i += kGThreads) {
      const int r = i / P.NC, c = i - r * P.NC;
      P.logits[(t0 + r) * P.NC + c] = sl[r * LP + c];
    }
  }
  float* sk = P.bias ? sl + kGBM * LP : sl;
  if (P.bias) {
    gate_keys(P, sl, sk, LP, rows);
    __syncthreads();
  }
  const int grp = threadIdx.x >> 4;                // 0..15
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int r = 16 * half + grp;
    route_row16<4 * NQ>(P, sl + r * LP, sk + r * LP, t0 + r, t0 + r < P.T);
  }
}

// S > 1: partial sums of one K range.
template <int NQ>
__global__ __launch_bounds__(kGThreads) void gate_part_kernel(GateP P) {
  const long t0 = (long)blockIdx.x * kGBM;
  const int split = blockIdx.y;
  f32x4 acc[NQ][2];
  gate_gemm<NQ>(P, acc, t0, split);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int NCP = 16 * P.NS;
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    if (4 * j + wave >= P.NS) continue;
#pragma unroll
    for (int ts = 0; ts < 2; ++ts) {
      const long row = t0 + 16 * ts + lr;
      if (row < P.T)
        *(f32x4*)(P.part + ((long)split * P.T + row) * NCP + 16 * (4 * j + wave) + 4 * lg) =
            acc[j][ts];
    }
  }
}

// S > 1: add the partial sums in split order for kGRows rows, then the
// epilogue. Each thread owns one 4-column chunk of one row at a time and
// issues the loads of all its splits before adding them in split order.
// LDS: the logits [kGRows][LP], then (with a bias) their keys.
template <int NQ>
__global__ __launch_bounds__(kGThreads) void gate_reduce_route_kernel(GateP P) {
  extern __shared__ __attribute__((aligned(16))) float sl[];
  const int NCP = 16 * P.NS, LP = NCP + 4, n4 = NCP / 4;
  const long t0 = (long)blockIdx.x * kGRows;
  const int rows = (int)min((long)kGRows, P.T - t0);
  const long slot = P.T * (long)NCP;
  for (int i = threadIdx.x; i < rows * n4; i += kGThreads) {
    const int r = i / n4, c = 4 * (i - r * n4);
    const float* src = P.part + (t0 + r) * NCP + c;
    f32x4 v[kGMaxSplits];
#pragma unroll
    for (int q = 0; q < kGMaxSplits; ++q)
      if (q < P.S) v[q] = *(const f32x4*)(src + q * slot);
    f32x4 sum = v[0];
#pragma unroll
    for (int q = 1; q < kGMaxSplits; ++q)
      if (q < P.S) sum += v[q];
    *(f32x4*)(sl + r * LP + c) = sum;
    if (P.logits) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (c + q < P.NC) P.logits[(t0 + r) * P.NC + c + q] = sum[q];
    }
  }
  __syncthreads();
  float* sk = P.bias ? sl + kGRows * LP : sl;
  if (P.bias) {
    gate_keys(P, sl, sk, LP, rows);
    __syncthreads();
  }
  const int grp = threadIdx.x >> 4;
  if (grp < kGRows)                                 // whole 16-lane groups
    route_row16<4 * NQ>(P, sl + grp * LP, sk + grp * LP, t0 + grp, grp < rows);
}

int splits_for(long T, int H) {
  const long tiles = (T + kGBM - 1) / kGBM;
  const int steps = H / 32;
  if (tiles >= kGateFusedTiles) return 1;
  long S = (kGateSplitTarget + tiles - 1) / tiles;
  S = std::max<long>(2, std::min<long>(S, std::min(kGMaxSplits, steps)));
  const long ps = (steps + S - 1) / S;
  return (int)((steps + ps - 1) / ps);
}

template <int NQ>
hipError_t run_gate(GateP& P, hipStream_t s) {
  const unsigned tiles = (unsigned)((P.T + kGBM - 1) / kGBM);
  const int LP = 16 * P.NS + 4;
  const int nb = P.bias ? 2 : 1;                 // logits (+ keys)
  if (P.S == 1) {
    const size_t shm = (size_t)nb * kGBM * LP * 4;   // <= 2 * 32 * 516 * 4 bytes
    static bool attr = false;
    if (!attr) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gate_fused_kernel<NQ>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         2 * kGBM * (16 * 4 * NQ + 4) * 4);
      if (e != hipSuccess) return e;
      attr = true;
    }
    hipLaunchKernelGGL(gate_fused_kernel<NQ>, dim3(tiles), dim3(kGThreads), shm, s, P);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(gate_part_kernel<NQ>, dim3(tiles, (unsigned)P.S), dim3(kGThreads), 0,
                     s, P);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned rb = (unsigned)((P.T + kGRows - 1) / kGRows);
  const size_t shm = (size_t)nb * kGRows * LP * 4;
  hipLaunchKernelGGL(gate_reduce_route_kernel<NQ>, dim3(rb), dim3(kGThreads), shm, s, P);
  return hipGetLastError();
}

}  // namespace

int gate_splits(long T, int H) { return T > 0 ? splits_for(T, H) : 1; }

size_t gate_ws_bytes(long T, int H, int n_cols) {
  if (T <= 0) return 0;
  const int S = splits_for(T, H);
  if (S == 1) return 0;
  const long NCP = 16L * ((n_cols + 15) / 16);
  return ((size_t)S * T * NCP * 4 + 255) & ~(size_t)255;
}

hipError_t launch_gate(const GateArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  GateP P{};
  P.x = (const uint8_t*)a.x;
  P.wg = (const uint8_t*)a.wg;
  P.T = a.T;
  P.H = a.H;
  P.n_routed = a.n_routed;
  P.n_sink = a.n_sink;
  P.NC = a.n_routed + a.n_sink;
  P.k = a.k;
  P.NS = (P.NC + 15) / 16;
  P.S = splits_for(a.T, a.H);
  P.steps = (a.H / 32 + P.S - 1) / P.S;
  P.bias = a.bias;
  P.scale = a.scale;
  P.part = (float*)a.ws;
  P.logits = a.logits;
  P.ids = a.ids;
  P.w = a.w;
  P.sw = a.sw;
  P.packed = a.packed;
  switch ((P.NS + 3) / 4) {
    case 1: return run_gate<1>(P, s);
    case 2: return run_gate<2>(P, s);
    case 3: return run_gate<3>(P, s);
    case 4: return run_gate<4>(P, s);
    case 5: return run_gate<5>(P, s);
    case 6: return run_gate<6>(P, s);
    case 7: return run_gate<7>(P, s);
    case 8: return run_gate<8>(P, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
