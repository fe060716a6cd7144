// Router epilogue: one wave64 per token row (route_dev.h).
#include "launch.h"
#include "route_dev.h"

namespace moe {

template <int NV>
__global__ __launch_bounds__(256) void route_kernel(
    const float* __restrict__ logits, long T, long ld, int n_routed,
    int n_sink, int k, const float* __restrict__ bias, float scale,
    int* __restrict__ ids, float* __restrict__ w, float* __restrict__ sw,
    int* __restrict__ packed) {
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= T) return;
  route_row<NV>(logits, row, ld, n_routed, n_sink, k, bias, scale, ids, w, sw, packed);
}

hipError_t launch_route(const float* logits, long T, long ld, int n_routed,
                        int n_sink, int k, const float* bias, float scale,
                        int* ids, float* w, float* sw, int* packed,
                        hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid((unsigned)((T + 3) / 4)), block(256);
  int nv = (n_routed + 63) / 64;
#define RT(NV)                                                                \
  hipLaunchKernelGGL(route_kernel<NV>, grid, block, 0, s, logits, T, ld,      \
                     n_routed, n_sink, k, bias, scale, ids, w, sw, packed)
  if (nv <= 1) RT(1);
  else if (nv <= 2) RT(2);
  else if (nv <= 4) RT(4);
  else if (nv <= 8) RT(8);
  else RT(16);
#undef RT
  return hipGetLastError();
}

}  // namespace moe
