// gemm_launch.hpp -- host entry of the register-dequant GEMM translation unit.
#pragma once

#include <hip/hip_runtime.h>

namespace metis {

struct GemmParams;

// C = alpha A B^T (+ K-extension) with 256 x 256 tiles; requires K % 256 == 0
// and 16-byte aligned code, scale and extension rows.
// splits > 1 writes raw partial sums per split (see gemm_fp4_kernel).
hipError_t launch_gemm_big(const GemmParams& gp, int splits, hipStream_t st);

struct MxGemmParams;

// C = A B^T of two MXFP4 operands with 256 x 256 tiles; requires K % 1024 == 0
// and 16-byte aligned code and scale rows.
hipError_t launch_mx_gemm(const MxGemmParams& g, hipStream_t st);

}  // namespace metis
