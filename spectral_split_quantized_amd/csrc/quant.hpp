// quant.hpp -- NVFP4 fake quantisation of an operand or of its residual
// M_R = M - U diag(S) V^T ("Metis: Training LLMs with FP4 Quantization",
// 关键设计 1; NVFP4 format from section 研究背景与动机).
//
// Two sweeps over M:
//   pass 1 (quant_amax_kernel): residual tile -> |max| -> one atomicMax per
//           wave (float bits of a non-negative value order like unsigned
//           ints, so the result is independent of arrival order);
//   pass 2 (quant_kernel): residual tile again (bit-identical: the same MFMA
//           chain and the same binary32 operations), quantised on store in
//           both K orientations.
// The rank-k product (U S)(V)^T of a tile runs on MFMA: U S and V are split
// into fp16 hi + lo parts (pre-scaled by powers of two into fp16 range) and
// the three significant cross terms are concatenated along K, so one
// v_mfma_f32_32x32x16_f16 chain yields the product to ~2^-22 relative.
//
// Quantiser (per 16-block along K; A_T = tensor amax):
//   s_g = RN(A_T / 2688), d = RN(6 s_g), t = RN(a_b / d),
//   s_b = E4M3 RNE saturating, s_eff = RN(s_b s_g), inv = RN(1 / s_eff),
//   y = RN(|x| inv), magnitude = E2M1 RNE or stochastic (16-bit Philox draw),
//   code = sign(x) << 3 | magnitude.  Every step is one binary32 operation with
//   round-to-nearest-even, written with the _rn intrinsics so the compiler can
//   neither contract nor approximate it.
#pragma once

#include "common.hpp"
#include "status.hpp"

namespace metis {

constexpr int kQT_R = 128;   // tile rows (4 waves x 32)
constexpr int kQT_C = 64;    // tile cols (two 32-wide MFMA tiles)
constexpr int kQThreads = 256;
constexpr int kQMaxKK = 12;  // K of the rank-k product / 16 (k <= 64)

// ---------------------------------------------------- residual operand prep --

// The rank-k product of a tile is evaluated transposed, P^T = V (U S)^T, on
// fp16 MFMA from hi/lo splits:
//   vcat row (a column c of M) = [hi(V) | lo(V) | hi(V)],
//   ucat row (a row r of M)    = [hi(US) | hi(US) | lo(US)],
// so vcat . ucat = hi hi + lo hi + hi lo, each segment kp = round_up(k, 16)
// wide (kc = 3 kp).  U S is pre-scaled by a power of two `pre` so its largest
// entry is below 2^14, V by 256; pscale = 1 / (pre 256) undoes both.  Both
// are stored fragment-major, rows padded to 32:
//   (row, kidx) -> ((row/32 * kc/16 + kidx/16) * 64 + lane) * 8 + kidx%8,
//   lane = (kidx%16)/8 * 32 + row%32,
// so one wave's fragment load is 1 KB of contiguous memory.
constexpr float kVPre = 256.0f;

// Everything the residual sweeps read besides M, in one launch:
//  - pre and pscale: pre is the power of two that puts the largest entry of
//    the row operand U S below 2^14.  Its bound is S[0] for given factors, or
//    sqrt of the largest Gram diagonal entry when the row operand is the
//    projection P = M V (equal to U S up to the rediagonalisation's
//    orthogonal rotation, and |P_ij| <= sqrt(G_jj)).  pscale = 1 / (pre kVPre)
//    goes to memory for the sweeps; every workgroup forms pre itself.
//  - the ucat and vcat fragments: one thread per padded row and 8-wide group
//    of the k index writes whole 16-byte fragment pieces, 32 threads (32
//    consecutive rows) one contiguous 512-byte run;
//  - nzero words at zero cleared (the sweeps' amax words), by workgroup 0.
struct ResidPrep {
  const float* U;   // rows x k
  const float* S;   // k (null: S = 1, the row operand is P)
  const float* V;   // cols x k
  const double* G;  // k x k Gram matrix of P (null: bound from S[0])
  int64_t rows, cols;
  int k, kp;
  float* pscale;
  _Float16* ucat;
  _Float16* vcat;
  uint32_t* zero;
  int nzero;
};

__device__ inline int64_t frag_off(int64_t row, int kidx, int kc) {
  const int lane = ((kidx & 15) >> 3) * 32 + (int)(row & 31);
  return (((row >> 5) * (kc >> 4) + (kidx >> 4)) * 64 + lane) * 8 + (kidx & 7);
}

inline int64_t resid_prep_threads(int64_t rows, int64_t cols, int kp) {
  return (((rows + 31) & ~(int64_t)31) + ((cols + 63) & ~(int64_t)63)) * (kp / 8);
}

// A thread's eight factor entries (and the matching S entries) are loaded
// before the scale is formed, from clamped in-bounds indices, so the loads
// overlap each other and the Gram-diagonal read; entries outside the factor
// are then set to zero.
__global__ __launch_bounds__(256) void resid_prep_kernel(ResidPrep p) {
  __shared__ float pre_s;
  const int tid = threadIdx.x;
  const int ng = p.kp >> 3, kc = 3 * p.kp;
  const int64_t per_rb = 32 * (int64_t)ng;  // threads per 32 padded rows
  const int64_t nu = ((p.rows + 31) >> 5) * per_rb;
  const int64_t nv = ((p.cols + 63) >> 6) * 2 * per_rb;
  const int64_t id = (int64_t)blockIdx.x * 256 + tid;
  const bool live = id < nu + nv;
  const bool is_u = id < nu;
  const int64_t lid = is_u ? id : id - nu;
  const int64_t rb = live ? lid / per_rb : 0;  // per_rb > 0 when any thread is live
  const int rem = (int)(lid - rb * per_rb);
  const int j0 = 8 * (rem >> 5);
  const int64_t r = rb * 32 + (rem & 31);
  const int64_t n = is_u ? p.rows : p.cols;
  const float* F = is_u ? p.U : p.V;
  float fv[8], sv[8];
  if (live) {
    const int64_t rc = r < n ? r : n - 1;  // n >= 1 for a live thread
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int jc = j0 + t < p.k ? j0 + t : p.k - 1;  // k >= 1 when kp > 0
      fv[t] = F[rc * p.k + jc];
      sv[t] = (is_u && p.S) ? p.S[jc] : 1.0f;
    }
  }
  if (tid < 64) {
    // max_j (float) sqrt(G_jj) = (float) sqrt(max_j G_jj): both are monotone
    float s0 = 0.0f;
    if (p.G) {
      for (int j = tid; j < p.k; j += 64) s0 = fmaxf(s0, (float)sqrt(p.G[(int64_t)j * p.k + j]));
      s0 = wave_max(s0);
    } else {
      s0 = p.k > 0 ? p.S[0] : 0.0f;
    }
    if (tid == 0) {
      int ex = 0;
      if (s0 > 0.0f) frexpf(s0, &ex);  // s0 < 2^ex
      pre_s = ldexpf(1.0f, 14 - ex);
      if (blockIdx.x == 0) p.pscale[0] = ldexpf(1.0f, ex - 14 - 8);  // 1 / (pre * kVPre)
    }
  }
  if (blockIdx.x == 0)
    for (int i = tid; i < p.nzero; i += 256) p.zero[i] = 0u;
  __syncthreads();
  if (!live) return;
  half8_t h, l;
  if (is_u) {
    const float pre = pre_s;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      float x = 0.0f;
      if (j0 + t < p.k && r < p.rows) x = __fmul_rn(__fmul_rn(fv[t], sv[t]), pre);
      h[t] = (_Float16)x;
      l[t] = (_Float16)__fsub_rn(x, (float)h[t]);
    }
    *(half8_t*)(p.ucat + frag_off(r, j0, kc)) = h;
    *(half8_t*)(p.ucat + frag_off(r, p.kp + j0, kc)) = h;
    *(half8_t*)(p.ucat + frag_off(r, 2 * p.kp + j0, kc)) = l;
  } else {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      float v = 0.0f;
      if (j0 + t < p.k && r < p.cols) v = __fmul_rn(fv[t], kVPre);
      h[t] = (_Float16)v;
      l[t] = (_Float16)__fsub_rn(v, (float)h[t]);
    }
    *(half8_t*)(p.vcat + frag_off(r, j0, kc)) = h;
    *(half8_t*)(p.vcat + frag_off(r, p.kp + j0, kc)) = l;
    *(half8_t*)(p.vcat + frag_off(r, 2 * p.kp + j0, kc)) = h;
  }
}

// ------------------------------------------------------------- quantiser --

constexpr int kAmaxSlots = 16;
constexpr int kAmaxSlotStride = 32;

struct QuantParams {
  const void* M;
  int dtype;  // 0 bf16, 1 f32
  int64_t rows, cols, ld;
  const _Float16* ucat;  // fragment-major (null: no factors)
  const _Float16* vcat;
  int kc;
  const float* pscale;
  uint32_t* amax;
  // streaming sweeps only: kAmaxSlots partial maxima, kAmaxSlotStride words
  // apart (one cache line each), so the workgroups' atomics spread over many
  // addresses instead of queueing on one
  uint32_t* amax_slots;
  uint8_t* codes0;  // axis 0 (K = rows): [cols][rows/2]
  uint8_t* scales0;
  float* sg0;
  uint8_t* codes1;  // axis 1 (K = cols): [rows][cols/2]
  uint8_t* scales1;
  float* sg1;
  float* resid;  // optional rows x cols export
  int axes;      // bit 0: axis 0, bit 1: axis 1
  int sr;
  // SR draws: 1 = by the element's row-major position in M (tag1), shared by
  // both orientations; 0 = by its position in each orientation's own layout
  // (tag0 along axis 0, tag1 along axis 1)
  int shared_draws;
  uint64_t seed;
  uint32_t tag0, tag1, step;
  int tiles_per_wg;  // column tiles walked by one workgroup
};

struct QuantBlockOut {
  uint32_t lo, hi;  // 16 packed codes
  uint32_t scale;   // E4M3 byte
};

// hc: complemented 16-bit draws (0xFFFF - h) of the 16 elements (SR only).
// y = RN(x inv) keeps the sign of x, so the conversion's sign bit is the sign
// of x (zeros included) and its magnitude that of RN(|x| inv).
__device__ inline QuantBlockOut quant_block16(const float (&x)[16], const uint32_t (&hc)[16],
                                              float s_g, float d, bool sr) {
  const float a = __uint_as_float(abs_max16_bits(x));
  const float t = __fdiv_rn(a, d);
  const uint32_t sb = e4m3_encode_hw(t);
  const float s_eff = __fmul_rn(e4m3_decode_hw(sb), s_g);
  // a zero block scale gives inv = 0, hence y = +-0 and a signed zero code
  // for every (finite) element of the block
  const float inv = sb != 0u ? __fdiv_rn(1.0f, s_eff) : 0.0f;
  float y[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) y[i] = __fmul_rn(x[i], inv);
  QuantBlockOut o;
  o.scale = sb;
  if (sr) {
    o.lo = e2m1_pack8_sr(y, hc);
    o.hi = e2m1_pack8_sr(y + 8, hc + 8);
  } else {
    o.lo = e2m1_pack8_rne(y);
    o.hi = e2m1_pack8_rne(y + 8);
  }
  return o;
}

// Complemented 16-bit draws of n <= 16 consecutive indices e0 .. e0+n-1 at
// any alignment (one Philox block per element; the ragged edge only).
__device__ inline void draws16_any(uint64_t e0, int n, uint32_t tag, uint32_t step, uint64_t seed,
                                   uint32_t (&hc)[16]) {
  for (int i = 0; i < 16; ++i) {
    const uint64_t e = e0 + (uint64_t)i;
    hc[i] = i < n ? 0xFFFFu - philox_half_of(philox_block(e >> 3, tag, step, seed), (uint32_t)(e & 7)) : 0u;
  }
}

// Complemented 16-bit draws (0xFFFF - h) of 16 consecutive indices
// e0 .. e0+15 with e0 % 8 == 0.
__device__ inline void draws16(uint64_t e0, uint32_t tag, uint32_t step, uint64_t seed,
                               uint32_t (&hc)[16]) {
  Philox4 b0 = philox_block(e0 >> 3, tag, step, seed);
  Philox4 b1 = philox_block((e0 >> 3) + 1, tag, step, seed);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    b0.v[w] = ~b0.v[w];
    b1.v[w] = ~b1.v[w];
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    hc[i] = philox_half_of(b0, (uint32_t)i);
    hc[8 + i] = philox_half_of(b1, (uint32_t)i);
  }
}

// 16 consecutive elements of row `row` starting at column `col` (n valid).
__device__ inline void load_row16(const void* M, int dtype, int64_t base, int n, bool vec_ok,
                                  float (&x)[16]) {
  if (n == 16 && vec_ok && dtype == 0) {
    const uint4 q0 = *(const uint4*)((const uint16_t*)M + base);
    const uint4 q1 = *(const uint4*)((const uint16_t*)M + base + 8);
    const uint32_t w[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else if (n == 16 && vec_ok && dtype == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 f = *(const float4*)((const float*)M + base + 4 * i);
      x[4 * i] = f.x;
      x[4 * i + 1] = f.y;
      x[4 * i + 2] = f.z;
      x[4 * i + 3] = f.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = i < n ? load_as_float(M, dtype, base + i) : 0.0f;
  }
}

// Bring the 16 accumulator values of one transposed 32x32 MFMA tile into
// column order: lanes 0-31 end with columns 0-15, lanes 32-63 with columns
// 16-31 of M row lane%32.  (The MFMA leaves lane l holding columns
// 8(v/4) + 4(l/32) + v%4; v_permlane32_swap exchanges the upper half of its
// first operand with the lower half of its second.)
__device__ inline void gather_cols16(const f32x16_t& acc, float (&out)[16]) {
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[b]), __float_as_uint(acc[8 + b]),
                                                    false, false);
    const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[4 + b]),
                                                    __float_as_uint(acc[12 + b]), false, false);
    out[b] = __uint_as_float(s[0]);
    out[4 + b] = __uint_as_float(s[1]);
    out[8 + b] = __uint_as_float(t[0]);
    out[12 + b] = __uint_as_float(t[1]);
  }
}

// This lane's two 16-column blocks of row `row` in the 64-column tile at c0
// (zero outside the operand); the bf16 fast path takes four 16-byte loads.
__device__ inline void load_tile_x(const QuantParams& p, int64_t row, bool row_ok, int64_t c0, int hh,
                                   bool vec_ok, float (&x)[2][16]) {
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int64_t gc = c0 + 32 * b + 16 * hh;
    const int n = (int)max((int64_t)0, min((int64_t)16, p.cols - gc));
    if (row_ok && n > 0)
      load_row16(p.M, p.dtype, row * p.ld + gc, n, vec_ok, x[b]);
    else
#pragma unroll
      for (int i = 0; i < 16; ++i) x[b][i] = 0.0f;
  }
}

__device__ inline void unpack_bf16x16(const uint4& q0, const uint4& q1, float (&x)[16]) {
  const uint32_t w[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// The rank-k product (V (U S)^T) of this wave's 32 rows x the tile's 64
// columns on MFMA: Bf holds the tile's vcat fragments, uf this wave's ucat
// fragments; a0 covers columns 0..31, a1 columns 32..63.
template <int NKK>
__device__ __forceinline__ void lowrank_mfma(const uint4* Bf, const half8_t (&uf)[NKK], int lane, f32x16_t& a0,
                                             f32x16_t& a1) {
  a0 = f32x16_t{};
  a1 = f32x16_t{};
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    const half8_t v0 = __builtin_bit_cast(half8_t, Bf[kk * 64 + lane]);
    const half8_t v1 = __builtin_bit_cast(half8_t, Bf[(NKK + kk) * 64 + lane]);
    a0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(v0, uf[kk], a0, 0, 0, 0);
    a1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(v1, uf[kk], a1, 0, 0, 0);
  }
}

// x -= pscale * product, one rounding per element: x - p ps with p ps exact
// (ps is a power of two), evaluated as one fused multiply-add.
__device__ __forceinline__ void lowrank_subtract(const f32x16_t& a0, const f32x16_t& a1, float ps,
                                                 float (&x)[2][16]) {
  float p0[16], p1[16];
  gather_cols16(a0, p0);
  gather_cols16(a1, p1);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    x[0][i] = __fmaf_rn(-p0[i], ps, x[0][i]);
    x[1][i] = __fmaf_rn(-p1[i], ps, x[1][i]);
  }
}

template <int NKK>
__device__ inline void subtract_lowrank(const uint4* Bf, const half8_t (&uf)[NKK], float ps, int lane,
                                        float (&x)[2][16]) {
  f32x16_t a0, a1;
  lowrank_mfma<NKK>(Bf, uf, lane, a0, a1);
  lowrank_subtract(a0, a1, ps, x);
}

// Pass 1: tensor |max| of the residual (or of M when NKK == 0).  A workgroup
// owns a 128-row panel and walks `tiles_per_wg` 64-column tiles; while tile t
// is formed, tile t+1's vcat fragments stream into the other LDS buffer by
// direct global->LDS loads and its M rows into registers, so one barrier per
// tile and no exposed load latency.  The two buffers are distinct arrays and
// the loop is unrolled by two so every LDS access names its buffer statically.
template <int NKK>
__device__ __forceinline__ void quant_amax_body(const QuantParams& p, int64_t bx, int64_t by) {
  constexpr bool HAS_F = NKK > 0;
  constexpr int BFU = HAS_F ? NKK * 2 * 64 : 1;  // uint4 per tile
  __shared__ uint4 Bf0[BFU];
  __shared__ uint4 Bf1[BFU];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int hh = lane >> 5;
  const int64_t r0 = bx * kQT_R;
  const int64_t ntc = ceil_div<int64_t>(p.cols, kQT_C);
  const int64_t ct0 = by * p.tiles_per_wg;
  const int64_t ct1 = min(ntc, ct0 + p.tiles_per_wg);
  const int64_t row = r0 + wave * 32 + (lane & 31);
  const bool row_ok = row < p.rows;
  const bool vec_ok = ((p.ld & 7) == 0) && (((uintptr_t)p.M & 15) == 0);
  // whole 16-byte-aligned bf16 tiles go through the register prefetch
  const bool fast = p.dtype == 0 && vec_ok && row_ok;
  const int64_t full_tiles = p.cols / kQT_C;

  half8_t uf[HAS_F ? NKK : 1];
  if (HAS_F) {
    const int64_t g = (r0 >> 5) + wave;
    const int64_t gmax = (p.rows + 31) >> 5;
    const half8_t z = {};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      uf[kk] = g < gmax ? *(const half8_t*)(p.ucat + ((g * NKK + kk) * 64 + lane) * 8) : z;
  }
  const float ps = HAS_F ? p.pscale[0] : 0.0f;

  auto issue = [&](int64_t ct, uint4* buf, uint4 (&raw)[4]) {
    if (HAS_F) {
      const uint4* src = (const uint4*)p.vcat + ct * BFU;
      for (int i = wave; i < 2 * NKK; i += 4) dma16(src + i * 64 + lane, (uint8_t*)(buf + i * 64));
    }
    if (fast && ct < full_tiles) {
      const uint16_t* m = (const uint16_t*)p.M + row * p.ld + ct * kQT_C + 16 * hh;
      raw[0] = *(const uint4*)m;
      raw[1] = *(const uint4*)(m + 8);
      raw[2] = *(const uint4*)(m + 32);
      raw[3] = *(const uint4*)(m + 40);
    }
  };
  float runmax = 0.0f;
  bool bad = false;
  auto body = [&](int64_t ct, const uint4* buf, const uint4 (&raw)[4]) {
    const int64_t c0 = ct * kQT_C;
    float x[2][16];
    if (fast && ct < full_tiles) {
      unpack_bf16x16(raw[0], raw[1], x[0]);
      unpack_bf16x16(raw[2], raw[3], x[1]);
    } else {
      load_tile_x(p, row, row_ok, c0, hh, vec_ok, x);
    }
    if (HAS_F) subtract_lowrank<HAS_F ? NKK : 1>(buf, uf, ps, lane, x);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t gc = c0 + 32 * b + 16 * hh;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float a = (row_ok && gc + i < p.cols) ? fabsf(x[b][i]) : 0.0f;
        bad |= !(a <= 3.402823466e38f);
        runmax = fmaxf(runmax, a);
      }
    }
  };

  uint4 rawA[4] = {}, rawB[4] = {};
  if (ct0 < ct1) issue(ct0, Bf0, rawA);
  for (int64_t ct = ct0; ct < ct1; ct += 2) {
    ring_barrier();  // tile ct has landed in Bf0; every wave is done with Bf1
    if (ct + 1 < ct1) issue(ct + 1, Bf1, rawB);
    body(ct, Bf0, rawA);
    if (ct + 1 >= ct1) break;
    ring_barrier();  // tile ct+1 has landed in Bf1; every wave is done with Bf0
    if (ct + 2 < ct1) issue(ct + 2, Bf0, rawA);
    body(ct + 1, Bf1, rawB);
  }
  if (bad) raise_status(kStatusNonFinite);
  runmax = wave_max(runmax);
  if (lane == 0) atomicMax(p.amax, __float_as_uint(runmax));
}

template <int NKK>
__global__ __launch_bounds__(kQThreads) __attribute__((amdgpu_waves_per_eu(2, 8)))
void quant_amax_kernel(QuantParams p) {
  quant_amax_body<NKK>(p, blockIdx.x, blockIdx.y);
}

// Two operands in one launch (the factors U and V, quantised directly):
// workgroups [0, na) take a, the others b.
__global__ __launch_bounds__(kQThreads) __attribute__((amdgpu_waves_per_eu(2, 8)))
void quant_amax_pair_kernel(QuantParams a, QuantParams b, int na) {
  if ((int)blockIdx.x < na)
    quant_amax_body<0>(a, blockIdx.x, blockIdx.y);
  else
    quant_amax_body<0>(b, (int64_t)blockIdx.x - na, blockIdx.y);
}

// Pass 2: quantise the residual in the orientations `axes` asks for.  NKK =
// kc / 16 of the rank-k product (0: no factors, direct quantisation); SR
// selects stochastic rounding.  A workgroup owns a 128-row panel and walks
// `tiles_per_wg` tiles of 64 columns.  Wave w owns rows 32w..32w+31; after
// gather_cols16 lane l holds row 32w + l%32 at columns 16(l/32) .. +15 and
// 32 + 16(l/32) .. +15: two axis-1 blocks, matching 32-byte row loads of M.
// The residual is formed by the same subtract_lowrank as in pass 1, so both
// sweeps see bit-identical values.  Axis-0 blocks (16 rows of one column) go
// through an LDS transpose inside the wave's own 32-row slab of R, so only the
// vcat fragments need workgroup barriers: they land by LDS-DMA, and the next
// tile's fragments (and its M rows, into registers) are requested as soon as
// every wave has finished its MFMAs, so they arrive while this tile is
// quantised.
//
// Positions outside the operand are never stored: an axis-1 block is written
// only for a valid row and 16 valid columns (cols % 16 == 0 for axis 1), an
// axis-0 block only for a valid column and 16 valid rows (rows % 16 == 0 for
// axis 0), so the values computed there need no masking.
template <int NKK, bool SR>
__device__ __forceinline__ void quant_body(const QuantParams& p, int64_t bx, int64_t by) {
  constexpr bool HAS_F = NKK > 0;
  constexpr int BFU = HAS_F ? NKK * 2 * 64 : 1;  // uint4 per tile
  __shared__ float R[kQT_R][kQT_C + 4];
  __shared__ uint4 Bf[BFU];
  // complemented draws of the tile in M's layout, read back by axis 0 when
  // the two orientations share them (row pitch 72: 16-byte aligned rows)
  __shared__ __attribute__((aligned(16))) uint16_t H[SR ? kQT_R : 1][SR ? kQT_C + 8 : 1];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int hh = lane >> 5;
  const int64_t r0 = bx * kQT_R;
  const int64_t ntc = ceil_div<int64_t>(p.cols, kQT_C);
  const int64_t ct0 = by * p.tiles_per_wg;
  const int64_t ct1 = min(ntc, ct0 + p.tiles_per_wg);
  const int64_t row = r0 + wave * 32 + (lane & 31);
  const bool row_ok = row < p.rows;
  const bool vec_ok = ((p.ld & 7) == 0) && (((uintptr_t)p.M & 15) == 0);
  const bool fast = p.dtype == 0 && vec_ok && row_ok;
  const int64_t full_tiles = p.cols / kQT_C;

  half8_t uf[HAS_F ? NKK : 1];
  if (HAS_F) {
    const int64_t g = (r0 >> 5) + wave;
    const int64_t gmax = (p.rows + 31) >> 5;
    const half8_t z = {};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      uf[kk] = g < gmax ? *(const half8_t*)(p.ucat + ((g * NKK + kk) * 64 + lane) * 8) : z;
  }
  const float ps = HAS_F ? p.pscale[0] : 0.0f;

  float s_g = 1.0f, d = 6.0f;
  {
    const float at = __uint_as_float(p.amax[0]);
    if (at > 0.0f) {
      s_g = __fdiv_rn(at, 2688.0f);
      d = __fmul_rn(6.0f, s_g);
    }
    if (bx == 0 && by == 0 && tid == 0) {
      if (p.sg0) p.sg0[0] = s_g;
      if (p.sg1) p.sg1[0] = s_g;
    }
  }
  const bool ax0 = (p.axes & 1) != 0;
  const bool ax1 = (p.axes & 2) != 0;
  const bool shared = SR && p.shared_draws != 0;
  // row-major draws aligned to Philox blocks (the fast path's condition)
  const bool draws_aligned = (p.cols & 7) == 0;

  // tile ct's vcat fragments -> Bf (LDS-DMA) and, on the fast path, its two
  // 16-column blocks of this lane's row -> raw
  auto issue = [&](int64_t ct, uint4 (&raw)[4]) {
    if (HAS_F) {
      const uint4* src = (const uint4*)p.vcat + ct * BFU;
      for (int i = wave; i < 2 * NKK; i += 4) dma16(src + i * 64 + lane, (uint8_t*)(Bf + i * 64));
    }
    if (fast && ct < full_tiles) {
      const uint16_t* m = (const uint16_t*)p.M + row * p.ld + ct * kQT_C + 16 * hh;
      raw[0] = *(const uint4*)m;
      raw[1] = *(const uint4*)(m + 8);
      raw[2] = *(const uint4*)(m + 32);
      raw[3] = *(const uint4*)(m + 40);
    }
  };

  uint4 raw[4] = {};
  if (ct0 < ct1) issue(ct0, raw);
  for (int64_t ct = ct0; ct < ct1; ++ct) {
    const int64_t c0 = ct * kQT_C;
    float x[2][16];
    if (fast && ct < full_tiles) {
      unpack_bf16x16(raw[0], raw[1], x[0]);
      unpack_bf16x16(raw[2], raw[3], x[1]);
    } else {
      load_tile_x(p, row, row_ok, c0, hh, vec_ok, x);
    }
    if (HAS_F) {
      ring_barrier();  // tile ct's fragments have landed in Bf
      subtract_lowrank<HAS_F ? NKK : 1>(Bf, uf, ps, lane, x);
      // every wave has read Bf (its MFMAs consumed the reads) before the
      // next tile's DMA overwrites it
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
    if (ct + 1 < ct1) issue(ct + 1, raw);

    // ---- axis 1 (and the export) from registers
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t gc = c0 + 32 * b + 16 * hh;
      if (!row_ok || gc >= p.cols) continue;
      if (p.resid) {
        const int n = (int)min((int64_t)16, p.cols - gc);
        float* dst = p.resid + row * p.cols + gc;
        for (int i = 0; i < n; ++i) dst[i] = x[b][i];
      }
      uint32_t hc[16];
      if (SR && (ax1 || (ax0 && shared))) {
        const uint64_t e0 = (uint64_t)row * (uint64_t)p.cols + (uint64_t)gc;
        const int n = (int)min((int64_t)16, p.cols - gc);
        if (n == 16 && draws_aligned)
          draws16(e0, p.tag1, p.step, p.seed, hc);
        else
          draws16_any(e0, n, p.tag1, p.step, p.seed, hc);
        if (ax0 && shared) {
          const int lr = wave * 32 + (lane & 31), lc = 32 * b + 16 * hh;
          uint32_t w[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) w[i] = hc[2 * i] | (hc[2 * i + 1] << 16);
          *(uint4*)&H[lr][lc] = make_uint4(w[0], w[1], w[2], w[3]);
          *(uint4*)&H[lr][lc + 8] = make_uint4(w[4], w[5], w[6], w[7]);
        }
      }
      if (ax1) {
        const QuantBlockOut o = quant_block16(x[b], hc, s_g, d, SR);
        *(uint2*)(p.codes1 + row * (p.cols >> 1) + (gc >> 1)) = make_uint2(o.lo, o.hi);
        p.scales1[row * (p.cols >> 4) + (gc >> 4)] = (uint8_t)o.scale;
      }
    }
    if (!ax0) continue;

    // ---- axis 0: transpose through this wave's slab of R (rows 32w..32w+31);
    // LDS operations of one wave complete in order, so the slab needs no
    // barrier, only a compiler fence
    const int lr = wave * 32 + (lane & 31);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int lc = 32 * b + 16 * hh;
#pragma unroll
      for (int i = 0; i < 16; i += 4)
        *(float4*)&R[lr][lc + i] = make_float4(x[b][i], x[b][i + 1], x[b][i + 2], x[b][i + 3]);
    }
    asm volatile("" ::: "memory");
    const int64_t gcol = c0 + lane;
    const int64_t grow0 = r0 + wave * 32;
    if (gcol < p.cols && grow0 < p.rows) {
      const bool two = grow0 + 16 < p.rows;  // rows % 16 == 0: blocks are whole
      uint32_t packed[4] = {0u, 0u, 0u, 0u};
      uint32_t sc = 0;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        if (b == 1 && !two) break;
        const int lr0 = wave * 32 + 16 * b;
        float xc[16];
        uint32_t hc[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) xc[i] = R[lr0 + i][lane];
        if (shared) {
#pragma unroll
          for (int i = 0; i < 16; ++i) hc[i] = H[lr0 + i][lane];
        } else if (SR) {
          draws16((uint64_t)gcol * (uint64_t)p.rows + (uint64_t)(grow0 + 16 * b), p.tag0, p.step, p.seed, hc);
        }
        const QuantBlockOut o = quant_block16(xc, hc, s_g, d, SR);
        packed[2 * b] = o.lo;
        packed[2 * b + 1] = o.hi;
        sc |= o.scale << (8 * b);
      }
      // rows % 16 == 0 makes every 8-byte code group 8-byte aligned; the
      // pair is 16-byte aligned only when rows % 32 == 0
      uint8_t* cdst = p.codes0 + gcol * (p.rows >> 1) + (grow0 >> 1);
      uint8_t* sdst = p.scales0 + gcol * (p.rows >> 4) + (grow0 >> 4);
      if (two && (((uintptr_t)cdst & 15) == 0)) {
        *(uint4*)cdst = make_uint4(packed[0], packed[1], packed[2], packed[3]);
      } else {
        *(uint2*)cdst = make_uint2(packed[0], packed[1]);
        if (two) *(uint2*)(cdst + 8) = make_uint2(packed[2], packed[3]);
      }
      if (two && (((uintptr_t)sdst & 1) == 0)) {
        *(uint16_t*)sdst = (uint16_t)sc;
      } else {
        sdst[0] = (uint8_t)sc;
        if (two) sdst[1] = (uint8_t)(sc >> 8);
      }
    }
    asm volatile("" ::: "memory");  // the slab is rewritten by the next tile
  }
}

template <int NKK, bool SR>
__global__ __launch_bounds__(kQThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void quant_kernel(QuantParams p) {
  quant_body<NKK, SR>(p, blockIdx.x, blockIdx.y);
}

// Two operands in one launch, as quant_amax_pair_kernel.
template <bool SR>
__global__ __launch_bounds__(kQThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void quant_pair_kernel(QuantParams a, QuantParams b, int na) {
  if ((int)blockIdx.x < na)
    quant_body<0, SR>(a, blockIdx.x, blockIdx.y);
  else
    quant_body<0, SR>(b, (int64_t)blockIdx.x - na, blockIdx.y);
}

}  // namespace metis
