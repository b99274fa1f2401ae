// quant.hpp -- NVFP4 fake quantisation of an operand or of its residual
// M_R = M - U diag(S) V^T ("Metis: Training LLMs with FP4 Quantization",
// 关键设计 1; NVFP4 format from section 研究背景与动机).
//
// Two sweeps over M, both HBM-bound:
//   pass 1: residual tile -> |max| -> one atomicMax per wave (float bits of a
//           non-negative value order like unsigned ints, so the result is
//           independent of arrival order);
//   pass 2: residual tile again (bit-identical: same instruction sequence),
//           quantised on store in both K orientations.
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

namespace metis {

constexpr int kQT_R = 64;    // tile rows
constexpr int kQT_C = 128;   // tile cols
constexpr int kQThreads = 256;

// ---------------------------------------------------- residual operand prep --

// acat[i][0:KP] = hi(U_i S pre), acat[i][KP:2KP] = hi(...), acat[i][2KP:3KP] = lo(...)
// bcat[c][0:KP] = hi(V_c vpre),  bcat[c][KP:2KP] = lo(...),  bcat[c][2KP:3KP] = hi(...)
// so that acat . bcat = hi hi + hi lo + lo hi.  pscale receives
// 1 / (pre * vpre), a power of two.
constexpr float kVPre = 256.0f;

__global__ void resid_scale_kernel(const float* __restrict__ S, int k, float* __restrict__ pre_out,
                                   float* __restrict__ pscale_out) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  const float s0 = k > 0 ? S[0] : 0.0f;
  int ex = 0;
  if (s0 > 0.0f) frexpf(s0, &ex);  // s0 < 2^ex
  const float pre = ldexpf(1.0f, 14 - ex);
  pre_out[0] = pre;
  pscale_out[0] = ldexpf(1.0f, ex - 14 - 8);  // 1 / (pre * kVPre)
}

__global__ void resid_prep_kernel(const float* __restrict__ U, const float* __restrict__ S,
                                  const float* __restrict__ V, int64_t rows, int64_t cols, int k,
                                  int kp, const float* __restrict__ pre_p, _Float16* __restrict__ acat,
                                  _Float16* __restrict__ bcat) {
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (rows + cols) * kp;
  if (id >= total) return;
  const int64_t r = id / kp;
  const int j = (int)(id % kp);
  const int kc = 3 * kp;
  if (r < rows) {
    float x = 0.0f;
    if (j < k) x = __fmul_rn(__fmul_rn(U[r * k + j], S[j]), pre_p[0]);
    const _Float16 h = (_Float16)x;
    const _Float16 l = (_Float16)__fsub_rn(x, (float)h);
    _Float16* a = acat + r * kc;
    a[j] = h;
    a[kp + j] = h;
    a[2 * kp + j] = l;
  } else {
    const int64_t c = r - rows;
    float v = 0.0f;
    if (j < k) v = __fmul_rn(V[c * k + j], kVPre);
    const _Float16 h = (_Float16)v;
    const _Float16 l = (_Float16)__fsub_rn(v, (float)h);
    _Float16* b = bcat + c * kc;
    b[j] = h;
    b[kp + j] = l;
    b[2 * kp + j] = h;
  }
}

// ------------------------------------------------------------- quantiser --

struct QuantParams {
  const void* M;
  int dtype;  // 0 bf16, 1 f32
  int64_t rows, cols, ld;
  const _Float16* acat;  // rows x kc (null: no factors)
  const _Float16* bcat;  // cols x kc
  int kc;
  const float* pscale;
  uint32_t* amax;
  uint8_t* codes0;  // axis 0 (K = rows): [cols][rows/2]
  uint8_t* scales0;
  float* sg0;
  uint8_t* codes1;  // axis 1 (K = cols): [rows][cols/2]
  uint8_t* scales1;
  float* sg1;
  float* resid;  // optional rows x cols export
  int axes;      // bit 0: axis 0, bit 1: axis 1
  int sr;
  uint64_t seed;
  uint32_t tag0, tag1, step;
};

struct QuantBlockOut {
  uint32_t lo, hi;  // 16 packed codes
  uint32_t scale;   // E4M3 byte
};

__device__ inline QuantBlockOut quant_block16(const float (&x)[16], const uint32_t (&h)[16],
                                              float s_g, float d, bool sr) {
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(x[i]));
  const float t = __fdiv_rn(a, d);
  const uint32_t sb = e4m3_encode_rne_sat(t);
  const float s_b = e4m3_decode(sb);
  const float s_eff = __fmul_rn(s_b, s_g);
  const float inv = __fdiv_rn(1.0f, s_eff);
  QuantBlockOut o;
  o.lo = 0;
  o.hi = 0;
  o.scale = sb;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float ax = fabsf(x[i]);
    uint32_t m = 0;
    if (sb != 0u && ax != 0.0f) {
      const float y = __fmul_rn(ax, inv);
      m = sr ? e2m1_sr(y, h[i]) : e2m1_rne(y);
    }
    const uint32_t code = ((__float_as_uint(x[i]) >> 31) << 3) | m;
    if (i < 8)
      o.lo |= code << (4 * i);
    else
      o.hi |= code << (4 * (i - 8));
  }
  return o;
}

// 16-bit draws of 16 consecutive logical elements e0 .. e0+15 (n valid).
__device__ inline void draws16(uint64_t e0, int n, uint32_t tag, uint32_t step, uint64_t seed,
                               uint32_t (&h)[16]) {
  if (n <= 0) return;
  const uint64_t qa = e0 >> 3;
  const uint64_t qb = (e0 + (uint64_t)(n - 1)) >> 3;
  Philox4 b0 = philox_block(qa, tag, step, seed);
  Philox4 b1 = (qb > qa) ? philox_block(qa + 1, tag, step, seed) : b0;
  Philox4 b2 = (qb > qa + 1) ? philox_block(qa + 2, tag, step, seed) : b1;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint64_t e = e0 + (uint64_t)i;
    const uint64_t q = e >> 3;
    const Philox4& b = (q == qa) ? b0 : ((q == qa + 1) ? b1 : b2);
    h[i] = (i < n) ? philox_half_of(b, (uint32_t)(e & 7)) : 0u;
  }
}

// Product tile (U S)(V)^T of the 64 x 128 tile at (r0, c0) into R (fp32,
// unscaled).  4 waves in 2 x 2: each wave covers 32 rows x 64 cols.
__device__ inline void resid_product_tile(const QuantParams& p, int64_t r0, int64_t c0,
                                          float (*R)[kQT_C + 4]) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wr = wave >> 1, wc = wave & 1;
  const int64_t arow = r0 + wr * 32 + (lane & 31);
  const int64_t bc0 = c0 + wc * 64 + (lane & 31);
  const int64_t bc1 = bc0 + 32;
  const bool av = arow < p.rows, bv0 = bc0 < p.cols, bv1 = bc1 < p.cols;
  const int koff = (lane >> 5) * 8;
  f32x16_t acc0 = {}, acc1 = {};
  const half8_t z = {};
  for (int kk = 0; kk < p.kc; kk += 16) {
    const half8_t a = av ? *(const half8_t*)(p.acat + arow * p.kc + kk + koff) : z;
    const half8_t b0 = bv0 ? *(const half8_t*)(p.bcat + bc0 * p.kc + kk + koff) : z;
    const half8_t b1 = bv1 ? *(const half8_t*)(p.bcat + bc1 * p.kc + kk + koff) : z;
    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b0, acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b1, acc1, 0, 0, 0);
  }
  const int col = wc * 64 + (lane & 31);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int row = wr * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
    R[row][col] = acc0[v];
    R[row][col + 32] = acc1[v];
  }
}

// PASS2 = false: amax sweep.  PASS2 = true: quantise sweep.
template <bool HAS_F, bool PASS2>
__global__ __launch_bounds__(kQThreads) void quant_kernel(QuantParams p) {
  __shared__ float R[kQT_R][kQT_C + 4];
  __shared__ uint16_t H0[PASS2 ? kQT_R : 1][PASS2 ? kQT_C + 2 : 1];
  const int tid = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.y * kQT_R;
  const int64_t c0 = (int64_t)blockIdx.x * kQT_C;

  if (HAS_F) resid_product_tile(p, r0, c0, R);

  // this thread's two axis-1 blocks: rows tid/8 and tid/8 + 32, cols (tid%8)*16
  const int lc = (tid & 7) * 16;
  const int64_t gc = c0 + lc;
  const int nvalid_c = (int)max((int64_t)0, min((int64_t)16, p.cols - gc));
  float x[2][16];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int lr = (tid >> 3) + 32 * b;
    const int64_t gr = r0 + lr;
    const bool rv = gr < p.rows;
    const int64_t base = gr * p.ld + gc;
    if (rv && nvalid_c == 16 && p.dtype == 0 && ((base & 7) == 0)) {
      const uint4 q0 = *(const uint4*)((const uint16_t*)p.M + base);
      const uint4 q1 = *(const uint4*)((const uint16_t*)p.M + base + 8);
      const uint32_t w[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        x[b][2 * i] = __uint_as_float(w[i] << 16);
        x[b][2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    } else if (rv && nvalid_c == 16 && p.dtype == 1 && ((base & 3) == 0)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 f = *(const float4*)((const float*)p.M + base + 4 * i);
        x[b][4 * i] = f.x;
        x[b][4 * i + 1] = f.y;
        x[b][4 * i + 2] = f.z;
        x[b][4 * i + 3] = f.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        x[b][i] = (rv && i < nvalid_c) ? load_as_float(p.M, p.dtype, base + i) : 0.0f;
    }
  }
  if (HAS_F) __syncthreads();
  const float ps = HAS_F ? p.pscale[0] : 0.0f;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int lr = (tid >> 3) + 32 * b;
    const bool rv = r0 + lr < p.rows;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float v = x[b][i];
      if (HAS_F) v = __fsub_rn(v, __fmul_rn(R[lr][lc + i], ps));
      if (!(rv && i < nvalid_c)) v = 0.0f;
      x[b][i] = v;
      if (PASS2) R[lr][lc + i] = v;
    }
  }

  if (!PASS2) {
    float m = 0.0f;
    bool bad = false;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float a = fabsf(x[b][i]);
        bad |= !(a <= 3.402823466e38f);
        m = fmaxf(m, a);
      }
    if (bad) raise_status(kStatusNonFinite);
    m = wave_max(m);
    if ((tid & 63) == 0) atomicMax(p.amax, __float_as_uint(m));
    return;
  }

  // ---- pass 2: tensor scale from the amax of pass 1
  const float at = __uint_as_float(p.amax[0]);
  float s_g = 1.0f, d = 6.0f;
  if (at > 0.0f) {
    s_g = __fdiv_rn(at, 2688.0f);
    d = __fmul_rn(6.0f, s_g);
  }
  if (blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) {
    if (p.sg0) p.sg0[0] = s_g;
    if (p.sg1) p.sg1[0] = s_g;
  }
  const bool sr = p.sr != 0;

#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int lr = (tid >> 3) + 32 * b;
    const int64_t gr = r0 + lr;
    if (gr >= p.rows || nvalid_c <= 0) continue;
    const uint64_t e0 = (uint64_t)gr * (uint64_t)p.cols + (uint64_t)gc;
    if (p.resid) {
      float* dst = p.resid + gr * p.cols + gc;
      for (int i = 0; i < nvalid_c; ++i) dst[i] = x[b][i];
    }
    if ((p.axes & 2) && nvalid_c == 16) {
      uint32_t h[16];
      if (sr) draws16(e0, 16, p.tag1, p.step, p.seed, h);
      const QuantBlockOut o = quant_block16(x[b], h, s_g, d, sr);
      *(uint2*)(p.codes1 + gr * (p.cols >> 1) + (gc >> 1)) = make_uint2(o.lo, o.hi);
      p.scales1[gr * (p.cols >> 4) + (gc >> 4)] = (uint8_t)o.scale;
    }
    if ((p.axes & 1) && sr) {
      uint32_t h[16];
      draws16(e0, nvalid_c, p.tag0, p.step, p.seed, h);
#pragma unroll
      for (int i = 0; i < 16; ++i) H0[lr][lc + i] = (uint16_t)h[i];
    }
  }
  if (!(p.axes & 1)) return;
  __syncthreads();
  // axis 0: column tid % 128, row blocks (tid/128)*2 + {0, 1}
  const int lcol = tid & (kQT_C - 1);
  const int64_t gcol = c0 + lcol;
  if (gcol >= p.cols) return;
  uint32_t packed[4];
  uint32_t sc = 0;
  int nb = 0;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int lr0 = (tid >> 7) * 32 + 16 * b;
    if (r0 + lr0 >= p.rows) break;
    float xc[16];
    uint32_t h[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      xc[i] = R[lr0 + i][lcol];
      h[i] = sr ? (uint32_t)H0[lr0 + i][lcol] : 0u;
    }
    const QuantBlockOut o = quant_block16(xc, h, s_g, d, sr);
    packed[2 * b] = o.lo;
    packed[2 * b + 1] = o.hi;
    sc |= o.scale << (8 * b);
    ++nb;
  }
  const int64_t grow0 = r0 + (tid >> 7) * 32;
  // rows % 16 == 0 makes every 8-byte code group 8-byte aligned; the pair is
  // 16-byte aligned only when rows % 32 == 0
  uint8_t* cdst = p.codes0 + gcol * (p.rows >> 1) + (grow0 >> 1);
  uint8_t* sdst = p.scales0 + gcol * (p.rows >> 4) + (grow0 >> 4);
  if (nb == 2 && (((uintptr_t)cdst & 15) == 0)) {
    *(uint4*)cdst = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  } else {
    for (int b = 0; b < nb; ++b) *(uint2*)(cdst + 8 * b) = make_uint2(packed[2 * b], packed[2 * b + 1]);
  }
  for (int b = 0; b < nb; ++b) sdst[b] = (uint8_t)(sc >> (8 * b));
}

}  // namespace metis
