// Router epilogue, device part (route.hip, front.hip): sigmoid-gate top-k
// with log-sigmoid renormalisation and trailing shared-sink columns.
//
// "Enable and fuse the Inkling MoE gate epilogue on Intel XPU" (sglang PR
// #36385): "3. Performance" ranks with iterative masked-max passes instead
// of a sort; "2. Correctness" normalises as exp(lp - logsumexp(lp)) with
// lp = logsigmoid(x) so rows whose logits are all below the fp32 sigmoid
// flush point stay finite; the router-epilogue commit message carries the
// winner's raw logit out of the top-k loop, ranks on sigmoid(x) + bias when
// a selection bias [n_routed] is given (sinks take none), lets the sink
// columns join the normaliser only, and packs (id << 16 | bf16 weight).
//
// One wave64 owns one token row. Lane l holds columns l, l + 64, ... of the
// routed part in registers; each pass takes the wave maximum of the lanes'
// best values, then the lowest column holding it (register-level DPP /
// row-swap reductions), and the owner lane marks the winner taken. Equal
// values resolve to the lower column. After k passes lane j < k holds slot j's raw
// logit and lanes k .. k+S-1 the sink logits; the renormalisation is a wave
// max and a wave sum.
#pragma once
#include "common.h"

namespace moe {

struct OpOrU32 { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a | b; } };

// one token row, called by all 64 lanes of a wave
template <int NV>
__device__ __forceinline__ void route_row(
    const float* __restrict__ logits, long row, long ld, int n_routed,
    int n_sink, int k, const float* __restrict__ bias, float scale,
    int* __restrict__ ids, float* __restrict__ w, float* __restrict__ sw,
    int* __restrict__ packed) {
  const int lane = lane_id();
  const float* x = logits + row * ld;

  // the sink logits are loaded with the row, not after the passes
  const bool sink = lane >= k && lane < k + n_sink;
  const float sink_x = sink ? x[n_routed + (lane - k)] : 0.0f;

  // All of the row's loads are issued before any of them is used: a
  // lane past the last routed column re-reads that column (n_routed >= 1),
  // so the loads need no branch, and no wait sits between two of them.
  float v[NV], key[NV], b[NV];
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = min(lane + 64 * i, n_routed - 1);
    v[i] = x[c];
    b[i] = bias ? bias[c] : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = lane + 64 * i;
    if (c >= n_routed) { taken |= 1u << i; v[i] = 0.0f; }   // not a candidate
    // with a selection bias the key is fp32 sigmoid(x) + bias
    key[i] = bias ? sigmoid_key(v[i]) + b[i] : v[i];
  }

  float my_x = -INFINITY;   // raw logit of the slot / sink this lane reports
  int my_c = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY, braw = 0.0f;
    int bc = 0x7FFFFFFF;       // no candidate yet
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      int c = lane + 64 * i;
      bool cand = !((taken >> i) & 1u);
      if (cand && (key[i] > bv || (key[i] == bv && c < bc))) { bv = key[i]; braw = v[i]; bc = c; }
    }
    // winner: the largest key, then the lowest column holding it
    const float wv = wave_max(bv);
    bc = wave_min_i32(bv == wv ? bc : 0x7FFFFFFF);
    const bool own = (bc & 63) == lane;
    if (own) taken |= 1u << (bc >> 6);
    // the winner carries its raw logit: the key itself without a bias,
    // else the owner lane's value
    float xw = wv;
    if (bias) xw = __uint_as_float(wave_reduce(own ? __float_as_uint(braw) : 0u, OpOrU32{}));
    if (lane == j) { my_x = xw; my_c = bc; }
  }
  const bool active = lane < k + n_sink;
  if (sink) my_x = sink_x;

  // lp = logsigmoid(x) = min(x, 0) - log1p(exp(-|x|));
  // exp(lp - logsumexp(lp)) evaluated as e / sum(e) with e = exp(lp - max lp):
  // lp - max is exact for nearby lp, so rows far below zero (lp ~ -200) keep
  // full fp32 relative accuracy instead of inheriting the rounding of a
  // logsumexp formed at magnitude ~200.
  float lp = active ? fminf(my_x, 0.0f) - log1pf(expf(-fabsf(my_x))) : -INFINITY;
  float m = wave_max(lp);
  float e = active ? expf(lp - m) : 0.0f;
  float wt = e / wave_sum(e) * scale;
  if (lane < k) {
    ids[row * k + lane] = my_c;
    w[row * k + lane] = wt;
    if (packed) packed[row * k + lane] = (int)(((uint32_t)my_c << 16) | f32_to_bf16_bits(wt));
  } else if (active) {
    sw[row * n_sink + (lane - k)] = wt;
  }
}

}  // namespace moe
