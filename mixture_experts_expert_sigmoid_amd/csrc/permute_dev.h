// Expert-parallel rebase and grouping of (token, slot) pairs, device part
// shared by permute.hip and front.hip (see permute.hip for the sources and
// the three-launch path).
#pragma once
#include "common.h"
#include "launch.h"

namespace moe {

__device__ __forceinline__ int local_group(int id, int E_global, int off,
                                           int E_loc, bool* oob) {
  if (id < 0 || id >= E_global) { *oob = true; return -1; }
  int e = id - off;
  return (e >= 0 && e < E_loc) ? e : -1;
}

// All pairs in one workgroup (npr <= kPermBlock): rank as in
// permute_rank_kernel, exclusive scan of the group totals, scatter.
// Called by all 1024 threads of the workgroup; sm: 17 G ints of LDS.
__device__ __forceinline__ void permute_small_body(
    const int* __restrict__ ids, long npr, long T, int E_global, int off,
    int E_loc, int G, int shared, int* __restrict__ offsets,
    int* __restrict__ sorted_pair, int* __restrict__ pair_row,
    int* __restrict__ err_word, int* sm) {
  int* cnt = sm;                   // cnt [16][G], then base [G]
  int* base = sm + 16 * G;
  __shared__ int wsum[16];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const long p = tid;
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
  // per group: exclusive prefix over the 16 waves, total in base[]
  for (int gi = tid; gi < G; gi += kPermBlock) {
    int run = 0;
#pragma unroll
    for (int ww = 0; ww < 16; ++ww) {
      int c = cnt[ww * G + gi];
      cnt[ww * G + gi] = run;
      run += c;
    }
    base[gi] = run;
  }
  __syncthreads();
  // exclusive scan of the group totals (G <= 1024: one per thread)
  int total = 0;
  if (tid < E_loc) total = base[tid];
  else if (tid < G) total = (int)T;      // the shared group
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
  const int excl = wbase + incl - total;
  if (tid < G) {
    offsets[tid] = excl;
    base[tid] = excl;
  }
  if (tid == G - 1) offsets[G] = excl + total;
  __syncthreads();
  if (g >= 0) {
    const int pos = base[g] + cnt[w * G + g] + r;
    sorted_pair[pos] = (int)p;
    pair_row[p] = pos;
  } else if (p < npr) {
    pair_row[p] = -1;
  }
  if (shared)
    for (long t = tid; t < T; t += kPermBlock) {
      const int pos = base[E_loc] + (int)t;
      sorted_pair[pos] = (int)(npr + t);
      pair_row[npr + t] = pos;
    }
}

}  // namespace moe
