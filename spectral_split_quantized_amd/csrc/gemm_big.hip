// gemm_big.hip -- translation unit of the register-dequant GEMM (built with
// an instruction-level-parallelism scheduling strategy; see build.py).
#include <hip/hip_runtime.h>

#include "gemm_launch.hpp"
#include "gemm_reg.hpp"
#include "mxfp4_gemm.hpp"

namespace metis {

hipError_t launch_gemm_big(const GemmParams& gp, int splits, hipStream_t st) {
  using Cfg = RegCfg<2, 2, 4, 4>;
  const int64_t tiles = ceil_div<int64_t>(gp.M, Cfg::BM) * ceil_div<int64_t>(gp.N, Cfg::BN);
  if (tiles <= 0) return hipSuccess;
  // LDS is static (one array per pipeline stage)
  hipLaunchKernelGGL((gemm_fp4_reg_kernel<2, 2, 4, 4>), dim3((unsigned)tiles, (unsigned)splits), dim3(Cfg::NT),
                     0, st, gp);
  return hipGetLastError();
}

hipError_t launch_mx_gemm(const MxGemmParams& g, hipStream_t st) {
  const int64_t tiles = ceil_div<int64_t>(g.M, 256) * ceil_div<int64_t>(g.N, 256);
  if (tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL((mx_gemm_kernel<2, 2, 4, 4>), dim3((unsigned)tiles), dim3(256), 0, st, g);
  return hipGetLastError();
}

}  // namespace metis
