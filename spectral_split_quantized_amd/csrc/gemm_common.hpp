// gemm_common.hpp -- operands and helpers shared by the NVFP4 GEMM kernels
// (gemm.hpp: LDS-staged fp16 tiles for every shape; gemm_reg.hpp: register
// expansion for the large products).  Declarations only: no kernels here.
#pragma once

#include "common.hpp"

namespace metis {

struct GemmParams {
  int64_t M, N, K;
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const uint8_t* b_codes;
  const uint8_t* b_scales;
  const float* sa;  // tensor scales (device) or null
  const float* sb;
  int64_t kext;     // multiple of 64; 0 = none
  const uint16_t* a_ext;  // bf16 [M][kext]
  const uint16_t* b_ext;  // bf16 [N][kext]
  float* C;
  int64_t ldc;
};

// 8 E2M1 codes (one dword, element 0 in the low nibble) -> 8 fp16 values
// grid(code) * s_b.  v_cvt_scalef32_pk_f16_fp4 applies only the exponent of
// its scale operand, so it is used with scale 1 (exact grid values, low
// nibble first) and the E4M3 block scale is applied by one packed fp16
// multiply; the product is exact (<= 6 significant bits, in fp16 range).
__device__ inline uint4 dequant8(uint32_t w, half2_t s) {
  const half2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s;
  const half2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s;
  const half2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s;
  const half2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s;
  uint4 o;
  o.x = __builtin_bit_cast(uint32_t, h0);
  o.y = __builtin_bit_cast(uint32_t, h1);
  o.z = __builtin_bit_cast(uint32_t, h2);
  o.w = __builtin_bit_cast(uint32_t, h3);
  return o;
}

// Scaling of a split product's output.  C = alpha (sum + ext / alpha) with
// alpha = s_a s_b, the residual operands' tensor scales: the K-extension is
// prepared already divided by alpha (times ext_mul), so the GEMM applies
// alpha once, in the epilogue, after the extension (the accumulators never
// leave the matrix registers to be scaled in the middle).  A product below
// 2^-64 works with alpha 2^64 and the epilogue applies the extra 2^-64, so
// ext_mul stays below 2^86; alpha == 0 (a residual that is all zeros)
// drops the residual sum and leaves the extension unscaled.  The extension's
// preparation and every GEMM that reads it evaluate this from the same two
// scales.
struct EpiScale {
  float ext_mul;  // factor of the K-extension values
  float post;     // epilogue factor
  float post2;    // second epilogue factor (a power of two, 1 if unused)
  bool skip_main; // alpha == 0: the residual sum is not accumulated
};

__device__ inline EpiScale epi_scale(const float* sa, const float* sb) {
  float alpha = 1.0f;
  if (sa) alpha *= sa[0];
  if (sb) alpha *= sb[0];
  EpiScale e{1.0f, 1.0f, 1.0f, false};
  if (!(alpha > 0.0f)) {
    e.skip_main = true;
  } else if (alpha < 0x1p-64f) {
    const float a2 = alpha * 0x1p64f;  // exact
    e.ext_mul = __fdiv_rn(1.0f, a2);
    e.post = a2;
    e.post2 = 0x1p-64f;
  } else {
    e.ext_mul = __fdiv_rn(1.0f, alpha);
    e.post = alpha;
  }
  return e;
}

__device__ inline int64_t remap_tile(int64_t bid, int64_t tiles_m, int64_t tiles_n) {
  const int64_t total = tiles_m * tiles_n;
  int64_t pid = bid;
  if (total % 8 == 0) pid = (bid % 8) * (total / 8) + bid / 8;  // XCD-contiguous
  // group 8 tile-rows together (column-major inside a group)
  const int64_t group = 8;
  const int64_t per_group = group * tiles_n;
  const int64_t gid = pid / per_group;
  const int64_t first_m = gid * group;
  const int64_t gsize = min(tiles_m - first_m, group);
  const int64_t in = pid % per_group;
  const int64_t tm = first_m + in % gsize;
  const int64_t tn = in / gsize;
  return tm * tiles_n + tn;
}

extern __shared__ __align__(16) _Float16 g_gemm_smem[];

// Layout of the bf16 K-extension operands ([rows rounded up to 32][kext],
// kext % 64 == 0) in MFMA fragment order: per 32-row group g and 16-wide K
// sub-step kk, the 64 lanes' 8-element slices (lane h * 32 + i holds row
// g * 32 + i, elements 8 h .. 8 h + 7 of the sub-step) are 1 KB contiguous,
// so one wave loads a fragment with one fully coalesced instruction.
__device__ inline int64_t ext_off(int64_t row, int64_t col, int64_t kext) {
  const int64_t g = row >> 5, kk = col >> 4;
  const int64_t lane = ((col >> 3) & 1) * 32 + (row & 31);
  return ((g * (kext >> 4) + kk) * 64 + lane) * 8 + (col & 7);
}

}  // namespace metis
