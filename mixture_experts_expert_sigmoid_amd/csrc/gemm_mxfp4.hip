// MXFP4 (e2m1 codes, e8m0 scale per 32 K) instantiation of the 4-bit grouped GEMM (gemm_w4.h).
#include "gemm_w4.h"

namespace moe {

hipError_t launch_gemm_mxfp4(const GemmParams& P, bool g1, long p_cap, int NT, hipStream_t s,
                             int* sk_grid) {
  return launch_w4_fmt<FMT_MXFP4>(P, g1, p_cap, NT, s, sk_grid);
}

}  // namespace moe
