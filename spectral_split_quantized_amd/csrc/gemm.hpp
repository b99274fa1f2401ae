// gemm.hpp -- NVFP4 x NVFP4 -> fp32 GEMM for the Metis split products
// ("Metis: Training LLMs with FP4 Quantization", 关键设计 1: the split forward
// GEMM; 整体框架: the same split in every forward and backward GEMM).
//
// C[m][n] = alpha * sum_k A[m][k] B[n][k]  (+ a bf16 K-extension)
// A: codes [M][K/2] (even k in the low nibble), E4M3 scales [M][K/16];
// B: the same with N rows.  Both operands are K-contiguous ("TN").
//
// A dequantised element grid(code) * s_b has at most 6 significant bits and
// lies in [2^-10, 2688], so it is exact in fp16; products of two fp16 values
// are exact in fp32, and the MFMA accumulates them in fp32.  The per-tensor
// scales are applied once in the epilogue (alpha).  The K-extension holds
// the low-rank terms of the split as bf16 hi/lo pairs; it is accumulated
// after alpha has been applied to the main sum.
//
// Tiling: BM x BN output tile per workgroup of WM x WN waves, each wave
// (BM/WM) x (BN/WN) as 32 x 32 MFMA tiles; K step 64; FP4 codes are loaded to
// registers one tile ahead, dequantised once per element and stored to a
// double-buffered LDS area laid out in MFMA fragment order (one barrier per
// K step).  Skinny products (one side = the rank k) split K across
// workgroups and reduce the partial sums in a fixed order.  Workgroup ids are remapped so that each XCD
// (ids are dealt round-robin over 8 XCDs) walks a contiguous, row-grouped
// range of tiles and so shares A and B panels in its own L2.
#pragma once

#include "gemm_common.hpp"

namespace metis {

// BM x BN tile, WM x WN waves; each wave owns (BM/WM) x (BN/WN) as 32 x 32
// MFMA tiles.  K step 64.
template <int BM, int BN, int WM, int WN>
struct GemmCfg {
  static constexpr int kThreads = WM * WN * 64;
  static constexpr int BK = 64;
  static constexpr int TM = BM / WM / 32;
  static constexpr int TN = BN / WN / 32;
  static constexpr int GA = BM / 32;
  static constexpr int GB = BN / 32;
  static constexpr int NCA = (BM * 2 + kThreads - 1) / kThreads;  // FP4 chunks / thread
  static constexpr int NCB = (BN * 2 + kThreads - 1) / kThreads;
  static constexpr int LDS_A = BM * BK;  // halfs per stage
  static constexpr int LDS_B = BN * BK;
  static_assert(TM >= 1 && TN >= 1, "wave tile smaller than one MFMA tile");
};

// offset (in halfs) of the 8-half fragment slot for (kk, group, lane)
template <int G>
__device__ inline int frag_off(int kk, int g, int ln) {
  return ((kk * G + g) * 64 + ln) * 8;
}

struct RawChunk {
  uint4 codes;
  uint32_t sc;   // two E4M3 scale bytes (low byte: first 16 elements)
  bool k0, k1;   // first / second 16 elements inside K
  bool valid;    // row inside the matrix
};

__device__ inline RawChunk load_chunk(const uint8_t* codes, const uint8_t* scales, int64_t nrows,
                                      int64_t K, int64_t row, int64_t kbase, int64_t kend) {
  RawChunk c;
  c.valid = row < nrows;
  c.k0 = kbase < kend;
  c.k1 = kbase + 16 < kend;
  c.codes = make_uint4(0, 0, 0, 0);
  c.sc = 0;
  if (c.valid && c.k0) {
    const uint8_t* cp = codes + row * (K >> 1) + (kbase >> 1);
    const uint8_t* sp = scales + row * (K >> 4) + (kbase >> 4);
    if (c.k1) {
      if (((uintptr_t)cp & 15) == 0) {
        c.codes = *(const uint4*)cp;
      } else {  // K % 32 != 0: rows start on 8-byte boundaries only
        const uint2 a = *(const uint2*)cp;
        const uint2 b = *(const uint2*)(cp + 8);
        c.codes = make_uint4(a.x, a.y, b.x, b.y);
      }
      c.sc = (uint32_t)sp[0] | ((uint32_t)sp[1] << 8);
    } else {
      const uint2 h = *(const uint2*)cp;
      c.codes = make_uint4(h.x, h.y, 0, 0);
      c.sc = sp[0];
    }
  }
  return c;
}

// Dequantise one 32-element chunk of row `lrow` (K half `h` of the K step)
// into its four fragment slots.
template <int G>
__device__ inline void store_chunk(_Float16* lds, const RawChunk& c, int lrow, int h) {
  const _Float16 f0 = (_Float16)e4m3_decode(c.sc & 0xFFu);
  const _Float16 f1 = (_Float16)e4m3_decode((c.sc >> 8) & 0xFFu);
  const half2_t s0 = {f0, f0};
  const half2_t s1 = {f1, f1};
  const uint32_t w[4] = {c.codes.x, c.codes.y, c.codes.z, c.codes.w};
  const int g = lrow >> 5, r = lrow & 31;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint4 v = dequant8(w[i], (i < 2) ? s0 : s1);
    const bool ok = c.valid && ((i < 2) ? c.k0 : c.k1);
    if (!ok) v = make_uint4(0, 0, 0, 0);
    const int kk = 2 * h + (i >> 1);
    const int ln = (i & 1) * 32 + r;
    *(uint4*)(lds + frag_off<G>(kk, g, ln)) = v;
  }
}


// gridDim.x = tiles, gridDim.y = K splits.  With splits > 1 the split's raw
// partial sum goes to C + split * M * ldc (alpha and the K-extension are
// not allowed then).
template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64) void gemm_fp4_kernel(GemmParams p) {
  using Cfg = GemmCfg<BM, BN, WM, WN>;
  constexpr int BK = Cfg::BK, TM = Cfg::TM, TN = Cfg::TN, GA = Cfg::GA, GB = Cfg::GB;
  constexpr int NT = Cfg::kThreads;
  constexpr int kStage = Cfg::LDS_A + Cfg::LDS_B;
  auto lds_a = [&](int buf) { return g_gemm_smem + buf * kStage; };
  auto lds_b = [&](int buf) { return g_gemm_smem + buf * kStage + Cfg::LDS_A; };

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave / WN, wn = wave % WN;
  const int64_t tiles_m = ceil_div<int64_t>(p.M, BM);
  const int64_t tiles_n = ceil_div<int64_t>(p.N, BN);
  const int64_t tile = remap_tile(blockIdx.x, tiles_m, tiles_n);
  const int64_t m0 = (tile / tiles_n) * BM;
  const int64_t n0 = (tile % tiles_n) * BN;
  const int64_t nsplit = gridDim.y;
  const int64_t kper = ceil_div<int64_t>(ceil_div<int64_t>(p.K, BK), nsplit) * BK;
  const int64_t kbeg = (int64_t)blockIdx.y * kper;
  const int64_t kend = min(p.K, kbeg + kper);

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16_t{};

  const int64_t nk = kend > kbeg ? ceil_div<int64_t>(kend - kbeg, BK) : 0;
  RawChunk ra[Cfg::NCA], rb[Cfg::NCB];

  auto load_tile = [&](int64_t kt) {
    const int64_t kb = kbeg + kt * BK;
#pragma unroll
    for (int i = 0; i < Cfg::NCA; ++i) {
      const int c = tid + i * NT;
      if (c < BM * 2)
        ra[i] = load_chunk(p.a_codes, p.a_scales, p.M, p.K, m0 + (c >> 1), kb + (c & 1) * 32, kend);
    }
#pragma unroll
    for (int i = 0; i < Cfg::NCB; ++i) {
      const int c = tid + i * NT;
      if (c < BN * 2)
        rb[i] = load_chunk(p.b_codes, p.b_scales, p.N, p.K, n0 + (c >> 1), kb + (c & 1) * 32, kend);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < Cfg::NCA; ++i) {
      const int c = tid + i * NT;
      if (c < BM * 2) store_chunk<GA>(lds_a(buf), ra[i], c >> 1, c & 1);
    }
#pragma unroll
    for (int i = 0; i < Cfg::NCB; ++i) {
      const int c = tid + i * NT;
      if (c < BN * 2) store_chunk<GB>(lds_b(buf), rb[i], c >> 1, c & 1);
    }
  };
  auto compute_f16 = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      half8_t af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *(const half8_t*)(lds_a(buf) + frag_off<GA>(kk, wm * TM + i, lane));
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[j] = *(const half8_t*)(lds_b(buf) + frag_off<GB>(kk, wn * TN + j, lane));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  };

  if (nk > 0) {
    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int64_t kt = 0; kt < nk; ++kt) {
      const int buf = (int)(kt & 1);
      const bool more = kt + 1 < nk;
      if (more) load_tile(kt + 1);
      compute_f16(buf);
      if (more) store_tile(buf ^ 1);
      __syncthreads();
    }
  }

  float alpha = 1.0f;
  if (p.sa) alpha *= p.sa[0];
  if (p.sb) alpha *= p.sb[0];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] *= alpha;

  // ---- K-extension: bf16 operands copied into the same fragment layout
  if (p.kext > 0) {
    const int64_t ne = p.kext / BK;
    for (int64_t kt = 0; kt < ne; ++kt) {
      // 8 chunks of 8 bf16 per row and K step
      for (int c = tid; c < BM * 8; c += NT) {
        const int lrow = c >> 3, c8 = c & 7;
        const int64_t row = m0 + lrow;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (row < p.M) v = *(const uint4*)(p.a_ext + ext_off(row, kt * BK + c8 * 8, p.kext));
        *(uint4*)(lds_a(0) + frag_off<GA>(c8 >> 1, lrow >> 5, (c8 & 1) * 32 + (lrow & 31))) = v;
      }
      for (int c = tid; c < BN * 8; c += NT) {
        const int lrow = c >> 3, c8 = c & 7;
        const int64_t row = n0 + lrow;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (row < p.N) v = *(const uint4*)(p.b_ext + ext_off(row, kt * BK + c8 * 8, p.kext));
        *(uint4*)(lds_b(0) + frag_off<GB>(c8 >> 1, lrow >> 5, (c8 & 1) * 32 + (lrow & 31))) = v;
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        bf16x8_t af[TM], bfr[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
          af[i] = *(const bf16x8_t*)(lds_a(0) + frag_off<GA>(kk, wm * TM + i, lane));
#pragma unroll
        for (int j = 0; j < TN; ++j)
          bfr[j] = *(const bf16x8_t*)(lds_b(0) + frag_off<GB>(kk, wn * TN + j, lane));
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
      __syncthreads();
    }
  }

  // ---- epilogue: lane holds column lane%32 and rows 8(v/4) + 4(lane/32) + v%4
  float* C = p.C + (int64_t)blockIdx.y * p.M * p.ldc;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t col = n0 + (wn * TN + j) * 32 + (lane & 31);
      if (col >= p.N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + (wm * TM + i) * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (row < p.M) C[row * p.ldc + col] = acc[i][j][v];
      }
    }
  }
}



template <int BM, int BN, int WM, int WN>
inline size_t gemm_lds_bytes() {
  using Cfg = GemmCfg<BM, BN, WM, WN>;
  return 2 * (size_t)(Cfg::LDS_A + Cfg::LDS_B) * sizeof(_Float16);
}

// out[i] = sum over splits of part[s][i] (fixed order: deterministic)
__global__ void reduce_splits_kernel(const float* __restrict__ part, int splits, int64_t count,
                                     float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  float s = 0.0f;
  for (int k = 0; k < splits; ++k) s += part[(int64_t)k * count + i];
  out[i] = s;
}

// --------------------------------------------------- split-term operand prep --

// One side of a split product, described by its quantised parts.
struct SplitSide {
  const uint8_t* codes;   // factor codes [k][len/2]
  const uint8_t* scales;  // [k][len/16]
  const float* ts;        // tensor scale (device)
  int k;
  int64_t len;            // length of each factor vector (rows of the factor)
};

// Dequantised factor entry (without tensor scale) of row `idx` (< len) in
// factor column q: grid(code) * s_b, exact in bf16.
__device__ inline float factor_val(const SplitSide& f, int q, int64_t idx) {
  const uint8_t byte = f.codes[(int64_t)q * (f.len >> 1) + (idx >> 1)];
  const uint32_t code = (idx & 1) ? (byte >> 4) : (byte & 0xF);
  const float g[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
  const float s_b = e4m3_decode(f.scales[(int64_t)q * (f.len >> 4) + (idx >> 4)]);
  const float v = g[code & 7] * s_b;
  return (code & 8) ? -v : v;
}

__device__ inline uint16_t bf16_rn_bits(float x) {
  const __bf16 b = (__bf16)x;
  return __builtin_bit_cast(uint16_t, b);
}
__device__ inline float bf16_bits_to_float(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

struct ExtParams {
  // out = L_R R_R^T + P' J^T + H G  with
  //   P'[i][p] = s_LR s_E praw[i][p] S_R[p]          (rows x kR)
  //   G[q][j]  = S_L[q] (s_F s_RR t1[q][j] + sum_p s_F s_E t2[q][p] S_R[p] J[j][p])
  int64_t rows, cols;
  int kR, kL, ksR, ksL;   // ks*: segment widths (multiples of 16)
  int64_t kext;
  const float* praw;  // rows x kR
  const float* t1;    // kL x cols
  const float* t2;    // kL x kR
  const float* S_R;
  const float* S_L;
  const float* s_LR;
  const float* s_RR;
  const float* s_E;
  const float* s_F;
  SplitSide H;        // along output rows (len = rows), k = kL
  SplitSide J;        // along output cols (len = cols), k = kR
  uint16_t* a_ext;    // rows x kext
  uint16_t* b_ext;    // cols x kext
};

// A_ext[i] = [hi(P'' s_J) | lo(..) | H_bar | H_bar | 0 ...]
// (rows past e.rows up to the next multiple of 32 are written as zeros)
__global__ void ext_prep_a_kernel(ExtParams e) {
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t i = id / e.kext;
  const int col = (int)(id % e.kext);
  if (i >= ((e.rows + 31) & ~(int64_t)31)) return;
  uint16_t out = 0;
  if (i >= e.rows) {
  } else if (col < 2 * e.ksR) {
    const int p = col % e.ksR;
    if (p < e.kR) {
      const float v = e.praw[i * e.kR + p] * (e.s_LR[0] * e.s_E[0]) * e.S_R[p] * e.J.ts[0];
      const uint16_t hi = bf16_rn_bits(v);
      out = (col < e.ksR) ? hi : bf16_rn_bits(v - bf16_bits_to_float(hi));
    }
  } else if (col < 2 * e.ksR + 2 * e.ksL) {
    const int q = (col - 2 * e.ksR) % e.ksL;
    if (q < e.kL) out = bf16_rn_bits(factor_val(e.H, q, i));
  }
  e.a_ext[ext_off(i, col, e.kext)] = out;
}

// B_ext[j] = [J_bar | J_bar | hi(s_H G) | lo(..) | 0 ...]: one thread per
// output column j (rows past e.cols up to the next multiple of 32 are zero)
// and, along blockIdx.y, one group of 8 rows q of G; the group-0 workgroups
// also write J_bar and the zero tail.  The column's J_bar entries stay in
// registers and the group's 8 rows of the folded T2 in LDS; the row is
// written in 8-element chunks.
__device__ inline uint4 pack8_bf16(const float* v) {
  uint4 o;
  o.x = (uint32_t)bf16_rn_bits(v[0]) | ((uint32_t)bf16_rn_bits(v[1]) << 16);
  o.y = (uint32_t)bf16_rn_bits(v[2]) | ((uint32_t)bf16_rn_bits(v[3]) << 16);
  o.z = (uint32_t)bf16_rn_bits(v[4]) | ((uint32_t)bf16_rn_bits(v[5]) << 16);
  o.w = (uint32_t)bf16_rn_bits(v[6]) | ((uint32_t)bf16_rn_bits(v[7]) << 16);
  return o;
}

constexpr int kExtMaxK = 96;
__global__ __launch_bounds__(256) void ext_prep_b_kernel(ExtParams e) {
  __shared__ float t2f[8][kExtMaxK + 1];
  const int tid = threadIdx.x;
  const int64_t j = (int64_t)blockIdx.x * 256 + tid;
  const int q0 = 8 * blockIdx.y;  // this workgroup's rows of G
  const float sJ = e.J.ts[0];
  const float sFE = e.s_F[0] * e.s_E[0];
  const float sFR = e.s_F[0] * e.s_RR[0];
  const float sH = e.H.ts[0];
  for (int idx = tid; idx < 8 * e.kR; idx += 256) {
    const int t = idx / e.kR, pp = idx - t * e.kR;
    const int q = q0 + t;
    t2f[t][pp] = q < e.kL ? sFE * e.t2[(int64_t)q * e.kR + pp] * e.S_R[pp] * sJ : 0.0f;
  }
  __syncthreads();
  if (j >= ((e.cols + 31) & ~(int64_t)31)) return;
  uint16_t* out = e.b_ext;
  if (j >= e.cols) {
    if (blockIdx.y == 0)
      for (int64_t c = 0; c < e.kext; c += 8) *(uint4*)(out + ext_off(j, c, e.kext)) = make_uint4(0, 0, 0, 0);
    return;
  }
  float jr[kExtMaxK];
#pragma unroll
  for (int pp = 0; pp < kExtMaxK; ++pp) jr[pp] = (pp < e.kR) ? factor_val(e.J, pp, j) : 0.0f;
  if (blockIdx.y == 0) {
    // J_bar, twice, and the zero tail
    for (int c = 0; c < e.ksR; c += 8) {
      float v[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        float x = 0.0f;
#pragma unroll
        for (int pp = 0; pp < kExtMaxK; pp += 8)
          if (pp == c) x = jr[pp + t];  // static register index
        v[t] = x;
      }
      const uint4 w = pack8_bf16(v);
      *(uint4*)(out + ext_off(j, c, e.kext)) = w;
      *(uint4*)(out + ext_off(j, e.ksR + c, e.kext)) = w;
    }
    for (int64_t c = 2 * e.ksR + 2 * e.ksL; c < e.kext; c += 8)
      *(uint4*)(out + ext_off(j, c, e.kext)) = make_uint4(0, 0, 0, 0);
  }
  if (q0 >= e.ksL) return;
  // G[q] = s_H S_L[q] (s_F s_RR T1[q][j] + sum_p T2f[q][p] J[j][p]) as hi / lo
  float hi[8], lo[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int q = q0 + t;
    float g = 0.0f;
    if (q < e.kL) {
      float acc = sFR * e.t1[(int64_t)q * e.cols + j];
#pragma unroll
      for (int pp = 0; pp < kExtMaxK; ++pp)
        if (pp < e.kR) acc += t2f[t][pp] * jr[pp];
      g = sH * e.S_L[q] * acc;
    }
    const uint16_t h = bf16_rn_bits(g);
    hi[t] = bf16_bits_to_float(h);
    lo[t] = g - hi[t];
  }
  *(uint4*)(out + ext_off(j, 2 * e.ksR + q0, e.kext)) = pack8_bf16(hi);
  *(uint4*)(out + ext_off(j, 2 * e.ksR + e.ksL + q0, e.kext)) = pack8_bf16(lo);
}

}  // namespace metis
