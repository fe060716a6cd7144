// Group-32 INT4 instantiation of the 4-bit grouped GEMM (gemm_w4.h), the
// f16 activation pass its GEMM1 reads, and the format dispatch of the
// 4-bit kernels (INT4 here, NVFP4 and MXFP4 in their own files).
#include "gemm_w4.h"

namespace moe {

// x bf16 [T][H] -> f16 [T][H] with each 8 columns in the order k0, k4, k1,
// k5, k2, k6, k3, k7 (the GEMM1 activation operand); one thread per 8
__global__ __launch_bounds__(256) void act_f16p_kernel(const uint16_t* __restrict__ x, long n8,
                                                       uint16_t* __restrict__ out, int* err) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const i32x4 v = *(const i32x4*)(x + 8 * i);
  *(f16x8*)(out + 8 * i) = bf16x8_f16p(v);
  if (err && bf16x8_f16_overflow(v)) atomicOr(err, MOE_DEVERR_BIT_F16_RANGE);
}

hipError_t launch_act_f16p(const void* x, long T, int H, void* out, int* err, hipStream_t s) {
  const long n8 = T * (long)H / 8;
  if (n8 == 0) return hipSuccess;
  act_f16p_kernel<<<dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s>>>(
      (const uint16_t*)x, n8, (uint16_t*)out, err);
  return hipGetLastError();
}

hipError_t launch_gemm_int4(const GemmParams& P, bool g1, long p_cap, int NT, hipStream_t s,
                            int* sk_grid) {
  return launch_w4_fmt<FMT_INT4>(P, g1, p_cap, NT, s, sk_grid);
}

hipError_t launch_gemm_w4(int fmt, const GemmParams& P, bool g1, long p_cap, int NT,
                          hipStream_t s, int* sk_grid) {
  switch (fmt) {
    case FMT_INT4: return launch_gemm_int4(P, g1, p_cap, NT, s, sk_grid);
    case FMT_NVFP4: return launch_gemm_nvfp4(P, g1, p_cap, NT, s, sk_grid);
    case FMT_MXFP4:
    case FMT_MXFP4_A8:             // GEMM2 (bf16 h); its GEMM1 is gemm_mx.hip's
      return launch_gemm_mxfp4(P, g1, p_cap, NT, s, sk_grid);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
