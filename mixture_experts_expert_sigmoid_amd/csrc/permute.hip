// Expert-parallel rebase and stable grouping of (token, slot) pairs by local
// expert.
//
// Ids are global; per-expert tables are rank-local, so each id is rebased by
// local_expert_offset and bounds-checked against the local count ("FlashInfer
// 0.6.18 SM100a+SM103a MoE-LoRA AOT" release notes, "Changes since
// 1b699bf"). Tokens are then dispatched per expert in sorted order ("sm100:
// Fused INT4 grouped + SiLU Triton kernel", batchgen PR #239, commit text).
//
// At most kPermBlock (token, slot) pairs: one launch, one workgroup does the
// ranking, the scan and the scatter. Otherwise three launches, no host round
// trip:
//   1. rank: blocks of 1024 pairs; inside a wave, pairs with the same group
//      are matched with ballots (leader's group broadcast, ballot of equals,
//      popcount of lower lanes = stable rank); per-wave counts go to LDS and
//      an exclusive prefix over the 16 waves gives each pair its rank inside
//      the block and each block its per-group count.
//   2. scan (one block): per group, exclusive prefix of the block counts
//      (each group's thread reads its column of counts 32 blocks at a time,
//      all loads in flight, and writes the prefixes back); exclusive prefix
//      over groups -> offsets.
//   3. scatter: sorted row = offsets[group] + prefix[block][group] + rank;
//      the always-on shared group takes pairs T*k + t at rows
//      offsets[E_loc] + t.
#include "permute_dev.h"

namespace moe {

static inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t permute_ws_bytes(long T, int k, int G) {
  long npr = T * (long)k;
  long nblk = (npr + kPermBlock - 1) / kPermBlock;
  return align256((size_t)npr * 4) + align256((size_t)nblk * G * 4) + 256;
}

__global__ __launch_bounds__(1024) void permute_rank_kernel(
    const int* __restrict__ ids, long npr, int E_global, int off, int E_loc,
    int G, int* __restrict__ rank, int* __restrict__ blockcnt,
    int* __restrict__ err_word) {
  extern __shared__ int cnt[];     // [16][G]
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const long p = (long)blockIdx.x * kPermBlock + tid;
  bool oob = false;
  int g = -1;
  if (p < npr) g = local_group(ids[p], E_global, off, E_loc, &oob);
  if (oob) atomicOr(err_word, MOE_DEVERR_BIT_OOB);
  for (int i = tid; i < 16 * G; i += kPermBlock) cnt[i] = 0;
  __syncthreads();

  uint64_t todo = __ballot(g >= 0);
  int r = 0;
  const uint64_t below = (1ull << lane) - 1ull;
  while (todo) {
    int leader = __builtin_ctzll(todo);
    int lg = __builtin_amdgcn_readlane(g, leader);
    uint64_t m = __ballot(g == lg);
    if (g == lg) r = __popcll(m & below);
    if (lane == leader) cnt[w * G + lg] = __popcll(m);
    todo &= ~m;
  }
  __syncthreads();
  for (int gi = tid; gi < G; gi += kPermBlock) {
    int run = 0;
#pragma unroll
    for (int ww = 0; ww < 16; ++ww) {
      int c = cnt[ww * G + gi];
      cnt[ww * G + gi] = run;
      run += c;
    }
    blockcnt[(long)blockIdx.x * G + gi] = run;
  }
  __syncthreads();
  if (g >= 0) rank[p] = cnt[w * G + g] + r;
}

__global__ __launch_bounds__(1024) void permute_scan_kernel(
    int* __restrict__ blockcnt, long nblk, int E_loc, int G, long T,
    int* __restrict__ offsets) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // per-group totals and exclusive per-block prefixes
  int total = 0;
  if (tid < E_loc) {
    // 32 block counts in flight at a time (a dependent walk would pay one
    // memory latency per block)
    for (long b0 = 0; b0 < nblk; b0 += 32) {
      int c[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) c[i] = b0 + i < nblk ? blockcnt[(b0 + i) * G + tid] : 0;
#pragma unroll
      for (int i = 0; i < 32; ++i)
        if (b0 + i < nblk) {
          blockcnt[(b0 + i) * G + tid] = total;
          total += c[i];
        }
    }
  } else if (tid < G) {
    total = (int)T;                       // the shared group
  }
  // exclusive scan of totals over groups (G <= 1024 = one per thread)
  int incl = total;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int wbase = 0;
  for (int i = 0; i < w; ++i) wbase += wsum[i];
  int excl = wbase + incl - total;
  if (tid < G) offsets[tid] = excl;
  if (tid == G - 1) offsets[G] = excl + total;
}

__global__ __launch_bounds__(256) void permute_scatter_kernel(
    const int* __restrict__ ids, long npr, long T, int E_global, int off,
    int E_loc, int G, const int* __restrict__ rank,
    const int* __restrict__ blockcnt, const int* __restrict__ offsets,
    int* __restrict__ sorted_pair, int* __restrict__ pair_row, long np) {
  const long p = (long)blockIdx.x * 256 + threadIdx.x;
  if (p >= np) return;
  if (p < npr) {
    bool oob = false;
    int g = local_group(ids[p], E_global, off, E_loc, &oob);
    if (g >= 0) {
      int pos = offsets[g] + blockcnt[(p / kPermBlock) * G + g] + rank[p];
      sorted_pair[pos] = (int)p;
      pair_row[p] = pos;
    } else {
      pair_row[p] = -1;
    }
  } else {
    int pos = offsets[E_loc] + (int)(p - npr);
    sorted_pair[pos] = (int)p;
    pair_row[p] = pos;
  }
}

__global__ __launch_bounds__(1024) void permute_small_kernel(
    const int* __restrict__ ids, long npr, long T, int E_global, int off,
    int E_loc, int G, int shared, int* __restrict__ offsets,
    int* __restrict__ sorted_pair, int* __restrict__ pair_row,
    int* __restrict__ err_word) {
  extern __shared__ int sm[];
  permute_small_body(ids, npr, T, E_global, off, E_loc, G, shared, offsets, sorted_pair,
                     pair_row, err_word, sm);
}

hipError_t launch_permute(const int* ids, long T, int k, int E_global, int off,
                          int E_loc, int shared, int* offsets,
                          int* sorted_pair, int* pair_row, int* err_word,
                          void* ws, hipStream_t s) {
  const int G = E_loc + (shared ? 1 : 0);
  const long npr = T * (long)k;
  const long nblk = (npr + kPermBlock - 1) / kPermBlock;
  if (npr <= kPermBlock && (size_t)17 * G * sizeof(int) <= 65536) {
    hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(kPermBlock),
                       (16 * G + G) * sizeof(int), s, ids, npr, T, E_global, off,
                       E_loc, G, shared, offsets, sorted_pair, pair_row, err_word);
    return hipGetLastError();
  }
  int* rank = (int*)ws;
  int* blockcnt = (int*)((char*)ws + align256((size_t)npr * 4));
  if (nblk > 0) {
    hipLaunchKernelGGL(permute_rank_kernel, dim3((unsigned)nblk),
                       dim3(kPermBlock), 16 * G * sizeof(int), s, ids, npr,
                       E_global, off, E_loc, G, rank, blockcnt, err_word);
  }
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(kPermBlock), 0, s,
                     blockcnt, nblk, E_loc, G, T, offsets);
  const long np = npr + (shared ? T : 0);
  if (np > 0) {
    hipLaunchKernelGGL(permute_scatter_kernel, dim3((unsigned)((np + 255) / 256)),
                       dim3(256), 0, s, ids, npr, T, E_global, off, E_loc, G,
                       rank, blockcnt, offsets, sorted_pair, pair_row, np);
  }
  return hipGetLastError();
}

}  // namespace moe
