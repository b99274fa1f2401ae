// status.hpp -- per-device numeric failure flag of the decomposition and
// quantisation kernels (one definition: included by the translation unit
// that holds those kernels only).
#pragma once

#include "common.hpp"

namespace metis {

// ----------------------------------------------------------- status flag --

// Per-device numeric failure flag (bit 0: non-finite input, bit 1: Cholesky
// breakdown, bit 2: row-sample selection overflow).
__device__ int g_metis_status;

__device__ inline void raise_status(int bits) { atomicOr(&g_metis_status, bits); }

constexpr int kStatusNonFinite = 1;
constexpr int kStatusCholesky = 2;
constexpr int kStatusSample = 4;

__global__ void fill_u32_kernel(uint32_t* p, uint32_t v, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ void copy_f32_kernel(const float* __restrict__ src, float* __restrict__ dst, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

}  // namespace metis
