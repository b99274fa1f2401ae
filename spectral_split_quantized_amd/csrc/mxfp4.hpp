// mxfp4.hpp -- MXFP4 quantiser (the product of two MXFP4 operands is in
// mxfp4_gemm.hpp).
//
// The pages name MXFP4 only as the other FP4 format ("Full-Stack FP4: Stable
// LLM Pretraining with Quantized Projections, Optimizers, and Attention",
// 局限性: its NVFP4 recipes are not claimed for MXFP4).  The format follows the
// OCP Microscaling (MX) definition: 32 consecutive elements along K share a
// power-of-two scale X = 2^(floor(log2 amax) - 2), stored as an E8M0 byte
// (e + 127, clamped to [-127, 127]; an all-zero block takes byte 0); each
// element is x / X rounded to the nearest E2M1 value (ties to even mantissa,
// saturating at 6), or stochastically with the path's Philox draws indexed
// by the output position outer * K + k.  Every step is exact in binary32.
#pragma once

#include "gemm_common.hpp"

namespace metis {

struct MxQuantParams {
  const void* src;
  int dtype;
  int64_t rows, cols, ld;
  uint8_t* codes;   // [outer][K / 2]
  uint8_t* scales;  // [outer][K / 32]
  int sr;           // stochastic rounding (else nearest)
  uint64_t seed;
  uint32_t tag, step;
};

// shared exponent of a block with largest magnitude amax
__device__ inline int mx_exponent(float amax) {
  if (!(amax > 0.0f)) return -127;
  int ex;
  frexpf(amax, &ex);  // amax = f 2^ex, f in [0.5, 1): floor(log2 amax) = ex - 1
  return max(-127, min(127, ex - 1 - 2));
}

// 32 values -> 16 code bytes (as 4 words) and the scale byte; with draws
// (complemented 16-bit draws, one per element) the rounding is stochastic
__device__ inline uint8_t mx_encode32(const float* v, uint32_t* w, const uint32_t* hc) {
  float amax = 0.0f;
  bool bad = false;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const float a = fabsf(v[j]);
    bad |= !(a <= 3.402823466e38f);  // NaN or infinity (fmaxf would drop a NaN)
    amax = fmaxf(amax, a);
  }
  if (bad) raise_status(kStatusNonFinite);
  const int e = mx_exponent(amax);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t word = 0;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float y = ldexpf(v[8 * q + t], -e);  // exact: a power-of-two scaling
      const uint32_t m = hc ? e2m1_sr_c(fabsf(y), hc[8 * q + t]) : e2m1_rne(fabsf(y));
      const uint32_t c = m | (y < 0.0f ? 8u : 0u);
      word |= c << (4 * t);
    }
    w[q] = word;
  }
  return (uint8_t)(e + 127);
}

// complemented draws of 32 consecutive positions e0 .. e0 + 31 of the
// output layout (e0 % 32 == 0)
__device__ inline void mx_draws32(uint64_t e0, const MxQuantParams& p, uint32_t (&hc)[32]) {
  uint32_t a[16], b[16];
  draws16(e0, p.tag, p.step, p.seed, a);
  draws16(e0 + 16, p.tag, p.step, p.seed, b);
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    hc[j] = a[j];
    hc[16 + j] = b[j];
  }
}

// K along a row: one thread per 32-element block
__global__ void mx_quant_rows_kernel(MxQuantParams p) {
  const int64_t nb = p.cols >> 5;
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= p.rows * nb) return;
  const int64_t r = id / nb, b = id - r * nb;
  float v[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) v[j] = load_as_float(p.src, p.dtype, r * p.ld + b * 32 + j);
  uint32_t w[4], hc[32];
  if (p.sr) mx_draws32((uint64_t)r * p.cols + b * 32, p, hc);
  p.scales[r * nb + b] = mx_encode32(v, w, p.sr ? hc : nullptr);
  *(uint4*)(p.codes + r * (p.cols >> 1) + b * 16) = make_uint4(w[0], w[1], w[2], w[3]);
}

// K down a column (the output is the quantised transpose): one thread per
// (column, 32-row block); neighbouring threads read neighbouring columns
__global__ void mx_quant_cols_kernel(MxQuantParams p) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t b = blockIdx.y;
  if (c >= p.cols) return;
  float v[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) v[j] = load_as_float(p.src, p.dtype, (b * 32 + j) * p.ld + c);
  uint32_t w[4], hc[32];
  if (p.sr) mx_draws32((uint64_t)c * p.rows + b * 32, p, hc);
  p.scales[c * (p.rows >> 5) + b] = mx_encode32(v, w, p.sr ? hc : nullptr);
  *(uint4*)(p.codes + c * (p.rows >> 1) + b * 16) = make_uint4(w[0], w[1], w[2], w[3]);
}

}  // namespace metis
