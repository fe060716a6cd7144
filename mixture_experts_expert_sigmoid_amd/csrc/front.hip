// Decode front end in one launch: for a small batch (T * top_k <= kPermBlock
// pairs) one workgroup of 1024 threads runs the router epilogue (a wave per
// token row), the activation pass (FP8 quantisation per 128 columns, or the
// f16 copy the 4-bit kernels read) and, after a barrier, the one-workgroup
// permutation -- three launches' work in one. The device code is the same
// as the separate kernels' (route_dev.h, quant_dev.h, act16_dev.h,
// permute_dev.h), so every output is bit-identical to theirs.
#include "act16_dev.h"
#include "launch.h"
#include "permute_dev.h"
#include "quant_dev.h"
#include "route_dev.h"

namespace moe {

template <int NV, int MODE>   // MODE 0: no activation pass, 1: FP8, 2: f16 copy, 3: MXFP8
__global__ __launch_bounds__(1024) void front_small_kernel(FrontArgs a) {
  extern __shared__ int sm[];                    // the permutation's 17 G ints
  const int wave = threadIdx.x >> 6;
  // rows from the last wave down, activation units from the first wave up,
  // so that at T = 1 the routing wave and the activation waves run side by
  // side instead of one wave doing both in turn
  for (long row = 15 - wave; row < a.T; row += 16)
    route_row<NV>(a.logits, row, a.ld, a.n_routed, a.n_sink, a.k, nullptr, a.scale, a.ids,
                  a.w, a.sw, nullptr);
  if constexpr (MODE == 1) {
    const long n = a.T * ((a.H + 511) >> 9);
    for (long wi = wave; wi < n; wi += 16)
      quant_act_unit((const uint16_t*)a.x, wi, a.H, (uint8_t*)a.xq, (float*)a.xs);
  } else if constexpr (MODE == 3) {
    const long n = a.T * ((a.H + 511) >> 9);
    for (long wi = wave; wi < n; wi += 16)
      quant_mx_unit((const uint16_t*)a.x, wi, a.H, (uint8_t*)a.xq, (uint8_t*)a.xs);
  } else if constexpr (MODE == 2) {
    const long n8 = a.T * (long)a.H / 8;
    bool over = false;
    for (long i = threadIdx.x; i < n8; i += 1024) {
      const i32x4 v = *(const i32x4*)((const uint16_t*)a.x + 8 * i);
      *(f16x8*)((uint16_t*)a.xq + 8 * i) = bf16x8_f16p(v);
      over |= bf16x8_f16_overflow(v);
    }
    if (over) atomicOr(a.err_word, MOE_DEVERR_BIT_F16_RANGE);
  }
  __syncthreads();                               // the ids are complete
  permute_small_body(a.ids, a.T * (long)a.k, a.T, a.n_routed, a.off, a.E_loc, a.G, a.shared,
                     a.offsets, a.sorted_pair, a.pair_row, a.err_word, sm);
}

// One workgroup pays only while each wave has a few rows and 512-column
// units to do: up to 64 units of T * ceil(H / 512), 4 per wave (measured:
// 3-5 us faster at T = 1, equal at 8 units per wave, slower beyond).
bool front_small_fits(long T, int k, int G, int H) {
  return T > 0 && T * (long)k <= kPermBlock && (size_t)17 * G * sizeof(int) <= 65536 &&
         T * (long)((H + 511) / 512) <= 64;
}

hipError_t launch_front_small(const FrontArgs& a, int mode, hipStream_t s) {
  if (!front_small_fits(a.T, a.k, a.G, a.H)) return hipErrorNotSupported;
  const size_t shm = (size_t)17 * a.G * sizeof(int);
  const int nv = (a.n_routed + 63) / 64;
#define FS(NV, MODE) \
  hipLaunchKernelGGL((front_small_kernel<NV, MODE>), dim3(1), dim3(kPermBlock), shm, s, a)
#define FSM(NV)                    \
  do {                             \
    if (mode == 1) FS(NV, 1);      \
    else if (mode == 2) FS(NV, 2); \
    else if (mode == 3) FS(NV, 3); \
    else FS(NV, 0);                \
  } while (0)
  if (nv <= 1) FSM(1);
  else if (nv <= 2) FSM(2);
  else if (nv <= 4) FSM(4);
  else if (nv <= 8) FSM(8);
  else FSM(16);
#undef FSM
#undef FS
  return hipGetLastError();
}

// Larger batches: the router epilogue and the activation pass are
// independent, so one launch runs both. The first nb_route workgroups route
// four token rows each (a wave per row, as route_kernel) and are dispatched
// first; the others run the activation pass, four 512-column units each (as
// quant_act_kernel / quant_act_mx_kernel) or 256 runs of 8 columns of the
// f16 copy (as act_f16p_kernel), filling the wave slots the routing leaves
// and taking over as its waves finish. (Interleaving the two kinds of
// workgroups through the grid measured slower at C2 T = 4096: the last
// routing waves then start near the end and lengthen its tail.) The device
// code is the separate kernels', so every output is bit-identical to theirs.
template <int NV, int MODE>
__global__ __launch_bounds__(256) void front_large_kernel(FrontArgs a, long nb_route) {
  const int wave = threadIdx.x >> 6;
  if ((long)blockIdx.x < nb_route) {
    const long row = (long)blockIdx.x * 4 + wave;      // wave-uniform
    if (row < a.T)
      route_row<NV>(a.logits, row, a.ld, a.n_routed, a.n_sink, a.k, nullptr, a.scale, a.ids,
                    a.w, a.sw, nullptr);
    return;
  }
  const long b = (long)blockIdx.x - nb_route;
  if constexpr (MODE == 1 || MODE == 3) {
    const long wi = b * 4 + wave;                      // wave-uniform
    if (wi >= a.T * ((a.H + 511) >> 9)) return;
    if constexpr (MODE == 1)
      quant_act_unit((const uint16_t*)a.x, wi, a.H, (uint8_t*)a.xq, (float*)a.xs);
    else
      quant_mx_unit((const uint16_t*)a.x, wi, a.H, (uint8_t*)a.xq, (uint8_t*)a.xs);
  } else if constexpr (MODE == 2) {
    const long i = b * 256 + threadIdx.x;
    if (i >= a.T * (long)a.H / 8) return;
    const i32x4 v = *(const i32x4*)((const uint16_t*)a.x + 8 * i);
    *(f16x8*)((uint16_t*)a.xq + 8 * i) = bf16x8_f16p(v);
    if (a.err_word && bf16x8_f16_overflow(v)) atomicOr(a.err_word, MOE_DEVERR_BIT_F16_RANGE);
  }
}

hipError_t launch_front_large(const FrontArgs& a, int mode, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const long nb_route = (a.T + 3) / 4;
  long nb_act = 0;
  if (mode == 1 || mode == 3) nb_act = (a.T * ((a.H + 511) / 512) + 3) / 4;
  else if (mode == 2) nb_act = (a.T * (long)a.H / 8 + 255) / 256;
  const dim3 grid((unsigned)(nb_route + nb_act)), block(256);
  const int nv = (a.n_routed + 63) / 64;
#define FL(NV, MODE) \
  hipLaunchKernelGGL((front_large_kernel<NV, MODE>), grid, block, 0, s, a, nb_route)
#define FLM(NV)                    \
  do {                             \
    if (mode == 1) FL(NV, 1);      \
    else if (mode == 2) FL(NV, 2); \
    else if (mode == 3) FL(NV, 3); \
    else FL(NV, 0);                \
  } while (0)
  if (nv <= 1) FLM(1);
  else if (nv <= 2) FLM(2);
  else if (nv <= 4) FLM(4);
  else if (nv <= 8) FLM(8);
  else FLM(16);
#undef FLM
#undef FL
  return hipGetLastError();
}

}  // namespace moe
