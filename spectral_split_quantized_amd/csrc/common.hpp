// common.hpp -- shared device/host helpers of libmetis (gfx950).
//
// Philox4x32-10: Salmon, Moraes, Dror & Shaw, "Parallel Random Numbers: As
// Easy as 1, 2, 3" (SC'11), section 3.  Draw layout (the Metis pages fix
// none): key = (seed lo, seed hi), counter = (q lo, q hi, tag, step).
//   32-bit draws: q = e >> 2, element e takes word e & 3.
//   16-bit draws: q = e >> 3, element e takes half (e & 1) (low half first) of
//   word (e >> 1) & 3.  Used for stochastic rounding (u = h * 2^-16) and for
//   the Gaussian test matrix (Omega = T[h]).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace metis {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr uint32_t kPhiloxM0 = 0xD2511F53u;
constexpr uint32_t kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u;
constexpr uint32_t kPhiloxW1 = 0xBB67AE85u;

// Draw roles, bits 8..11 of the tag.
enum : uint32_t {
  kRoleResid = 0,  // both orientations of an operand (role 1 unused)
  kRoleU = 2,
  kRoleV = 3,
  kRoleOmega = 4,
  kRoleSample = 5
};

__host__ __device__ inline uint32_t tag_with_role(uint32_t tag, uint32_t role) {
  return (tag & ~0xF00u) | ((role & 0xFu) << 8);
}

struct Philox4 {
  uint32_t v[4];
};

__host__ __device__ inline Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)kPhiloxM0 * c0;
    const uint64_t p1 = (uint64_t)kPhiloxM1 * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
  Philox4 out;
  out.v[0] = c0;
  out.v[1] = c1;
  out.v[2] = c2;
  out.v[3] = c3;
  return out;
}

// The same ten rounds on the GPU: each round's two three-way XORs as one
// v_bitop3_b32 each (truth table 0x96 = a ^ b ^ c).
__device__ inline Philox4 philox4x32_10_dev(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                            uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)kPhiloxM0 * c0;
    const uint64_t p1 = (uint64_t)kPhiloxM1 * c2;
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
  Philox4 out;
  out.v[0] = c0;
  out.v[1] = c1;
  out.v[2] = c2;
  out.v[3] = c3;
  return out;
}

__device__ inline Philox4 philox_block(uint64_t q, uint32_t tag, uint32_t step, uint64_t seed) {
  return philox4x32_10_dev((uint32_t)q, (uint32_t)(q >> 32), tag, step, (uint32_t)seed, (uint32_t)(seed >> 32));
}

// 32-bit draw of element e.
__device__ inline uint32_t philox_word(uint64_t e, uint32_t tag, uint32_t step,
                                                uint64_t seed) {
  const Philox4 b = philox_block(e >> 2, tag, step, seed);
  return b.v[e & 3];
}

// 16-bit half of a block for element offset o = e & 7.
__host__ __device__ inline uint32_t philox_half_of(const Philox4& b, uint32_t o) {
  return (b.v[(o >> 1) & 3] >> ((o & 1) * 16)) & 0xFFFFu;
}

// ----------------------------------------------------------------- formats --

// E4M3 ("FN": bias 7, max 448) value of a non-negative byte, exact in fp32.
__host__ __device__ inline float e4m3_decode(uint32_t b) {
  const int e = (int)((b >> 3) & 0xF);
  const int m = (int)(b & 7);
  if (e == 0) return ldexpf((float)m, -9);
  return ldexpf((float)(8 + m), e - 10);
}

// Round-to-nearest-even E4M3 byte of t >= 0, saturating at 448 (0x7E).
// Every step is exact in binary32: scalings by powers of two, 2f - 1 with
// f in [0.5, 1), and rintf (round half to even).
__host__ __device__ inline uint32_t e4m3_encode_rne_sat(float t) {
  if (!(t < 448.0f)) return 0x7Eu;          // also +inf (NaN never reaches here)
  if (t < 0.015625f) {                      // below 2^-6: subnormal grid 2^-9
    const float q = rintf(t * 512.0f);      // 0..8; 8 encodes 2^-6 = 0x08
    return (uint32_t)q;
  }
  int ex;
  const float f = frexpf(t, &ex);           // t = f 2^ex, f in [0.5, 1)
  int e = ex - 1;                           // t = (2f) 2^e
  int mq = (int)rintf((2.0f * f - 1.0f) * 8.0f);
  if (mq == 8) {
    mq = 0;
    e += 1;
  }
  if (e > 8 || (e == 8 && mq == 7)) return 0x7Eu;
  return (uint32_t)(((e + 7) << 3) | mq);
}

// E2M1 magnitude index of y >= 0.  On y >= 0 the grid is three uniform
// segments: steps of 0.5 on [0, 2) (codes 0..4), 1 on [2, 4) (codes 4..6) and
// 2 on [4, 6] (codes 6..7).  With j = clamp(floor(log2 y), 0, 2) the segment
// index (read from the exponent field), the position of y in code units is
// y 2^(1-j) + 2j: a power-of-two scaling, exact in binary32, plus an even
// integer.  y is first clamped to 6, whose position is code 7, so y >= 6
// saturates.  NaN gives an unspecified code.  e2m1_segment_biased returns
// 127 + j.
__host__ __device__ inline uint32_t e2m1_segment_biased(float yc) {  // 127 + j
  const uint32_t e = __builtin_bit_cast(uint32_t, yc) >> 23;  // biased exponent (yc >= 0)
  return e < 127u ? 127u : (e > 129u ? 129u : e);
}

// Round to nearest with ties to the even code: rint (ties to even) of the
// scaled position gives exactly the ties 0.25 -> 0, 0.75 -> 1, 1.25 -> 1,
// 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4 of the grid (adding the even 2j
// keeps the parity).
__host__ __device__ inline uint32_t e2m1_rne(float y) {
  const float yc = fminf(y, 6.0f);
  const uint32_t m = e2m1_segment_biased(yc);
  return (uint32_t)rintf(ldexpf(yc, 128 - (int)m)) + 2u * (m - 127u);
}

// Stochastic rounding with a 16-bit draw h (u = h 2^-16), given as its
// complement hc = 0xFFFF - h: with position n + p (n its integer part, p in
// [0, 1)) the code is n + 1 iff u < p22, p22 = floor(p 2^22) / 2^22 (p to 22
// binary digits), i.e. iff f = floor(p 2^22) >= 64 h + 1.  F = floor(y
// 2^(23-j)) is exact (y has 24 significant bits and y 2^(23-j) < 2^26), and
// F + j 2^23 = n 2^22 + f; adding 64 hc + 63 = 2^22 - 64 h - 1 carries into
// bit 22 exactly when f >= 64 h + 1.
__host__ __device__ inline uint32_t e2m1_sr_c(float y, uint32_t hc) {
  const float yc = fminf(y, 6.0f);
  const uint32_t m = e2m1_segment_biased(yc);
  const uint32_t f = (uint32_t)floorf(ldexpf(yc, 150 - (int)m));
  return (f + ((m - 127u) << 23) + (hc << 6) + 63u) >> 22;
}

__host__ __device__ inline uint32_t e2m1_sr(float y, uint32_t h) { return e2m1_sr_c(y, 0xFFFFu - h); }

// --------------------------------------------- gfx950 conversion instructions --
//
// The same E2M1 and E4M3 roundings by gfx950's conversion instructions, each
// checked on the GPU against the definitions above over every rounding
// boundary of the two grids and ~10^5 further values:
//   v_cvt_scalef32_pk_fp4_f32 (scale 1): nearest E2M1 value with ties to the
//     even code, saturating at 6, the sign bit copied from the input (zeros
//     included): sign << 3 | e2m1_rne(|y|).  The first source lands in the
//     low nibble of the selected byte.
//   v_cvt_scalef32_sr_pk_fp4_f32 (scale 1, random word r): adds bits 31..10
//     of r to the 22 bits of |y| below its E2M1 spacing (further bits
//     dropped) and keeps the carry; the second element uses bits 30..9.
//     With r = hc << 16 | 0xFFFF that is e2m1_sr_c(|y|, hc), signed as above.
//   v_cvt_scalef32_pk_fp8_f32 (scale 1) of min(t, 448), t >= 0: the E4M3
//     byte of e4m3_encode_rne_sat(t); v_cvt_f32_fp8 decodes it exactly.

typedef float float2_t __attribute__((ext_vector_type(2)));
typedef short short2_t __attribute__((ext_vector_type(2)));

// Codes of y[0..7] (already scaled, signed), nearest-even: y[0] in the low
// nibble.
__device__ inline uint32_t e2m1_pack8_rne(const float* y) {
  uint32_t w = 0u;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], 1.0f, 3);
  return w;
}

// The random word that makes the stochastic conversion decide u < p22 for
// the complemented draw hc.
__device__ inline uint32_t sr_word(uint32_t hc) { return (hc << 16) | 0xFFFFu; }

// One stochastic conversion of the pair v = (y0, y1) into byte SEL of w; the
// other bytes of w are kept.  Written as assembly with w tied to the
// destination: the compiler's builtin for this instruction does not place
// its `old` operand in the destination register, so the kept bytes would be
// whatever that register held.
template <int SEL>
__device__ __forceinline__ uint32_t cvt_sr_fp4_byte(uint32_t w, float2_t v, uint32_t r) {
  if constexpr (SEL == 0)
    asm volatile("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0" : "+v"(w) : "v"(v), "v"(r));
  else if constexpr (SEL == 1)
    asm volatile("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0 op_sel:[0,0,1,0]" : "+v"(w) : "v"(v), "v"(r));
  else if constexpr (SEL == 2)
    asm volatile("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0 op_sel:[0,0,0,1]" : "+v"(w) : "v"(v), "v"(r));
  else
    asm volatile("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0 op_sel:[0,0,1,1]" : "+v"(w) : "v"(v), "v"(r));
  return w;
}

// The random word that makes the conversion's second element decide u < p22
// for the complemented draw hc: that element adds bits 30..9 of the word.
__device__ inline uint32_t sr_word_hi(uint32_t hc) { return (hc << 15) | 0x7FFFu; }

// Codes of y[0..7] rounded stochastically with the complemented draws
// hc[0..7].  Each conversion takes a pair (y[2i], y[2i+1]) but its two
// elements draw from overlapping bits of one random word, so every pair is
// converted twice: once with the word of the even element (whose low nibble
// is kept, in `a`) and once with the word of the odd one (high nibble, `b`).
__device__ inline uint32_t e2m1_pack8_sr(const float* y, const uint32_t* hc) {
  uint32_t a = 0u, b = 0u;
  const float2_t v0 = {y[0], y[1]}, v1 = {y[2], y[3]}, v2 = {y[4], y[5]}, v3 = {y[6], y[7]};
  a = cvt_sr_fp4_byte<0>(a, v0, sr_word(hc[0]));
  b = cvt_sr_fp4_byte<0>(b, v0, sr_word_hi(hc[1]));
  a = cvt_sr_fp4_byte<1>(a, v1, sr_word(hc[2]));
  b = cvt_sr_fp4_byte<1>(b, v1, sr_word_hi(hc[3]));
  a = cvt_sr_fp4_byte<2>(a, v2, sr_word(hc[4]));
  b = cvt_sr_fp4_byte<2>(b, v2, sr_word_hi(hc[5]));
  a = cvt_sr_fp4_byte<3>(a, v3, sr_word(hc[6]));
  b = cvt_sr_fp4_byte<3>(b, v3, sr_word_hi(hc[7]));
  return __builtin_amdgcn_bitop3_b32(a, b, 0x0F0F0F0Fu, 0xE4);  // (a & m) | (b & ~m)
}

// Largest |x| of 16 values, as the binary32 bits of a non-negative value
// (which order like unsigned integers): integer maxima need no NaN
// canonicalisation of their operands.
__device__ inline uint32_t abs_max16_bits(const float* x) {
  uint32_t m = 0u;
#pragma unroll
  for (int i = 0; i < 16; i += 2)
    m = max(m, max(__float_as_uint(x[i]) & 0x7FFFFFFFu, __float_as_uint(x[i + 1]) & 0x7FFFFFFFu));
  return m;
}

// E4M3 byte of t >= 0, nearest-even, saturating at 448.
__device__ inline uint32_t e4m3_encode_hw(float t) {
  const short2_t r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32((short2_t){0, 0}, fminf(t, 448.0f), 0.0f, 1.0f,
                                                              false);
  return (uint32_t)(uint16_t)r[0] & 0xFFu;
}

__device__ inline float e4m3_decode_hw(uint32_t b) { return __builtin_amdgcn_cvt_f32_fp8((int)b, 0); }


// ------------------------------------------------------------------- misc --

template <typename T>
__host__ __device__ inline T ceil_div(T a, T b) {
  return (a + b - 1) / b;
}

__device__ inline float load_as_float(const void* p, int dtype, int64_t idx) {
  if (dtype == 0) {
    const uint16_t b = ((const uint16_t*)p)[idx];
    return __uint_as_float((uint32_t)b << 16);
  }
  return ((const float*)p)[idx];
}

// 16-byte direct global -> LDS load: lane L writes lds + 16 L (the LDS
// address must be wave-uniform).
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ inline void dma16(const void* g, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t*)lds, 16, 0, 0);
}

// Workgroup barrier for an LDS-DMA ring.  Every wave first waits for its own
// DMAs into the stage about to be read (s_waitcnt vmcnt(0)); the LDS is
// written only by those DMAs, so no release fence is needed.  The empty asm
// keeps the compiler from moving LDS reads above the barrier.
__device__ inline void ring_barrier() {
  __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (15 << 8));  // vmcnt(0) only
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ inline double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}


}  // namespace metis
