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
  for (long row = wave; row < a.T; row += 16)
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

}  // namespace moe
