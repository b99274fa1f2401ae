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
// the low-rank terms of the split as bf16 hi/lo pairs, divided by alpha
// (epi_scale), and is accumulated into the same unscaled sum.
//
// Tiling: BM x BN output tile per workgroup of WM x WN waves, each wave
// (BM/WM) x (BN/WN) as 32 x 32 MFMA tiles; K step 64; FP4 codes are loaded to
// registers one tile ahead, dequantised once per element and stored to a
// double-buffered LDS area laid out in MFMA fragment order (one barrier per
// K step).  Workgroup ids are remapped so that each XCD (ids are dealt
// round-robin over 8 XCDs) walks a contiguous, row-grouped range of tiles and
// so shares A and B panels in its own L2.  The rank-k side products (one
// operand of at most 64 rows) have their own kernel, gemm_thin_kernel.
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
// not allowed then); the library launches one split.
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

  const EpiScale es = epi_scale(p.sa, p.sb);
  const int64_t nk = kend > kbeg && !es.skip_main ? ceil_div<int64_t>(kend - kbeg, BK) : 0;
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
        if (row < p.M) {
          float y = acc[i][j][v] * es.post;
          if (es.post2 != 1.0f) y *= es.post2;
          C[row * p.ldc + col] = y;
        }
      }
    }
  }
}



template <int BM, int BN, int WM, int WN>
inline size_t gemm_lds_bytes() {
  using Cfg = GemmCfg<BM, BN, WM, WN>;
  return 2 * (size_t)(Cfg::LDS_A + Cfg::LDS_B) * sizeof(_Float16);
}

// ------------------------------------------------ thin products (k <= 64) --
//
// part (M x 64, fp32) = A B^T for a large NVFP4 A (M x K) and a thin NVFP4 B
// (nb <= 64 rows over the same K): the rank-k side products of the split.
// B is dequantised once (thin_bfrag_kernel) into fp16 MFMA B fragments; each
// 4-wave workgroup streams them through a double-buffered LDS ring by direct
// global->LDS loads while every wave expands its own 32 rows of A in
// registers (hardware fp4 -> fp16 conversion and one packed fp16 multiply by
// the E4M3 block scale: exact), one K step of 64 ahead.  K is walked in the
// permuted order "lane half h, element i of sub-step kk <-> k = 32 h + 8 kk
// + i" on both operands (a permutation of K leaves the sum unchanged), so a
// lane loads its 32 A codes of a step with one 16-byte load.  K splits along
// gridDim.y write fp32 partial sums [split][M][64]; the consumer adds them in
// split order.
constexpr int kThinRows = 128;  // rows per workgroup: 4 waves x 32

// fragment id = ((kb * 4 + kk) * 2 + nt) * 64 + lane holds the 8 values
// B[nt * 32 + lane % 32][kb * 64 + 32 (lane / 32) + 8 kk + i], i < 8 (zero
// outside B).  Up to two B operands over the same K per launch: the first
// nks * 512 threads form the first, the next nks * 512 the second.
struct ThinB {
  const uint8_t* codes;
  const uint8_t* scales;
  int nb;
  uint4* bfrag;
};

__global__ void thin_bfrag_kernel(ThinB b0, ThinB b1, int64_t K) {
  int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nks = (K + 63) >> 6;
  const bool second = id >= nks * 512;
  if (second) id -= nks * 512;
  if (id >= nks * 512 || (second && !b1.bfrag)) return;
  const uint8_t* __restrict__ codes = second ? b1.codes : b0.codes;
  const uint8_t* __restrict__ scales = second ? b1.scales : b0.scales;
  const int nb = second ? b1.nb : b0.nb;
  uint4* __restrict__ bfrag = second ? b1.bfrag : b0.bfrag;
  const int lane = (int)(id & 63);
  const int nt = (int)((id >> 6) & 1);
  const int kk = (int)((id >> 7) & 3);
  const int64_t kb = id >> 9;
  const int row = nt * 32 + (lane & 31);
  const int64_t k0 = kb * 64 + 32 * (lane >> 5) + 8 * kk;
  uint4 v = make_uint4(0, 0, 0, 0);
  if (row < nb && k0 < K) {  // K % 16 == 0: the 8 values lie inside K and one scale block
    const uint32_t w = *(const uint32_t*)(codes + row * (K >> 1) + (k0 >> 1));
    const _Float16 sb = (_Float16)e4m3_decode(scales[row * (K >> 4) + (k0 >> 4)]);
    v = dequant8(w, half2_t{sb, sb});
  }
  bfrag[id] = v;
}

struct ThinParams {
  const uint8_t* a_codes;   // [M][K/2]
  const uint8_t* a_scales;  // [M][K/16]
  const uint4* bfrag;       // thin_bfrag_kernel output for B
  int64_t M, K;
  int64_t steps;            // K steps of 64 per split
  float* part;              // [gridDim.y][M][64]
};

// Four-buffer ring, three K steps in flight.  Every step issues the same
// vector-memory operations per lane (2 direct-to-LDS B loads, then the A
// codes and scales: kThinAOps<A16>), so "step t has landed" is an exact
// vmcnt of the steps issued after it.  Loads that fall outside A (rows past
// M, the half of a last K step beyond K) read a valid address and are
// zeroed afterwards.
template <bool A16>
struct ThinOps {
  static constexpr int kA = A16 ? 2 : 4;  // uint4 + ushort, or 2 uint2 + 2 bytes
  static constexpr int kStep = 2 + kA;
};

template <int N>
__device__ inline void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Up to three thin products (same K) in one launch: product i owns the
// workgroups [first[i], first[i + 1]) of a 1-D grid, as a (row block, split)
// grid of gx[i] row blocks.
struct ThinBatch {
  ThinParams p[3];
  int64_t gx[3];
  int64_t first[4];
};

template <bool A16>
__global__ __launch_bounds__(256) void gemm_thin_kernel(ThinBatch tb) {
  __shared__ uint4 B0[512];
  __shared__ uint4 B1[512];
  __shared__ uint4 B2[512];
  __shared__ uint4 B3[512];
  const int64_t blk = blockIdx.x;
  const int which = blk < tb.first[1] ? 0 : (blk < tb.first[2] ? 1 : 2);
  const ThinParams& p = tb.p[which];
  const int64_t lb = blk - tb.first[which];
  const int64_t bx = lb % tb.gx[which], by = lb / tb.gx[which];
  constexpr int OPS = ThinOps<A16>::kStep;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int hh = lane >> 5;
  const int64_t row = bx * kThinRows + wave * 32 + (lane & 31);
  const bool row_ok = row < p.M;
  const int64_t nks = (p.K + 63) >> 6;
  const int64_t s0 = by * p.steps;
  const int64_t s1 = min(nks, s0 + p.steps);
  const int64_t lrow = row_ok ? row : p.M - 1;
  const uint8_t* arow = p.a_codes + lrow * (p.K >> 1);
  const uint8_t* srow = p.a_scales + lrow * (p.K >> 4);

  struct AReg {
    uint4 c;
    uint32_t s;
    bool ok;
  };
  auto issue = [&](int64_t kb, uint4* buf, AReg& a) {
    dma16(p.bfrag + kb * 512 + wave * 64 + lane, (uint8_t*)(buf + wave * 64));
    dma16(p.bfrag + kb * 512 + (wave + 4) * 64 + lane, (uint8_t*)(buf + (wave + 4) * 64));
    int64_t k0 = kb * 64 + 32 * hh;  // this lane's 32 elements of the step
    a.ok = row_ok && k0 < p.K;
    if (k0 >= p.K) k0 -= 32;         // a valid address; the values are dropped
    const uint8_t* c = arow + (k0 >> 1);
    const uint8_t* sc = srow + (k0 >> 4);
    if (A16) {
      a.c = *(const uint4*)c;
      a.s = *(const uint16_t*)sc;
    } else {
      // K % 32 == 16: rows start on 8-byte boundaries; the last step of K
      // holds 16 elements in this lane's half (k0 + 32 > K), read twice
      const bool full = k0 + 32 <= p.K;
      const uint2 x = *(const uint2*)c, y = *(const uint2*)(c + (full ? 8 : 0));
      const uint32_t b0 = sc[0], b1 = sc[full ? 1 : 0];
      a.c = make_uint4(x.x, x.y, full ? y.x : 0u, full ? y.y : 0u);
      a.s = b0 | ((full ? b1 : 0u) << 8);
    }
  };
  f32x16_t acc0 = {}, acc1 = {};
  auto compute = [&](const uint4* buf, const AReg& a) {
    const uint4 cw = a.ok ? a.c : make_uint4(0, 0, 0, 0);
    const uint32_t sw = a.ok ? a.s : 0u;
    const half2_t sc = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, false));
    const half2_t sA = {sc.x, sc.x}, sB = {sc.y, sc.y};
    const uint32_t w[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const half8_t af = __builtin_bit_cast(half8_t, dequant8(w[kk], kk < 2 ? sA : sB));
      const half8_t b0 = __builtin_bit_cast(half8_t, buf[(kk * 2) * 64 + lane]);
      const half8_t b1 = __builtin_bit_cast(half8_t, buf[(kk * 2 + 1) * 64 + lane]);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, b0, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, b1, acc1, 0, 0, 0);
    }
  };
  // wait for step t given how many later steps have been issued, then a
  // workgroup barrier (the LDS is written only by the direct loads)
  auto land = [&](int64_t later) {
    if (later >= 2) vm_wait<2 * OPS>();
    else if (later == 1) vm_wait<OPS>();
    else vm_wait<0>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  AReg r0{}, r1{}, r2{}, r3{};
  if (s0 < s1) issue(s0, B0, r0);
  if (s0 + 1 < s1) issue(s0 + 1, B1, r1);
  if (s0 + 2 < s1) issue(s0 + 2, B2, r2);
  for (int64_t t = s0; t < s1; t += 4) {
    // buffer (t + 3) % 4 was last read at step t - 1, before this barrier
    land(min((int64_t)2, s1 - 1 - t));
    if (t + 3 < s1) issue(t + 3, B3, r3);
    compute(B0, r0);
    if (t + 1 >= s1) break;
    land(min((int64_t)2, s1 - 2 - t));
    if (t + 4 < s1) issue(t + 4, B0, r0);
    compute(B1, r1);
    if (t + 2 >= s1) break;
    land(min((int64_t)2, s1 - 3 - t));
    if (t + 5 < s1) issue(t + 5, B1, r1);
    compute(B2, r2);
    if (t + 3 >= s1) break;
    land(min((int64_t)2, s1 - 4 - t));
    if (t + 6 < s1) issue(t + 6, B2, r2);
    compute(B3, r3);
  }
  // lane holds column lane % 32 of each n-tile and rows 8(v/4) + 4(lane/32) + v%4
  float* out = p.part + by * p.M * 64;
  const int64_t rbase = bx * kThinRows + wave * 32 + 4 * hh;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int64_t r = rbase + 8 * (v >> 2) + (v & 3);
    if (r < p.M) {
      out[r * 64 + (lane & 31)] = acc0[v];
      out[r * 64 + 32 + (lane & 31)] = acc1[v];
    }
  }
}

// sum over splits s < S (in split order) of the 8 floats at base + s *
// stride (32-byte aligned); the loads of four splits are issued together.
__device__ inline void sum_parts8(const float* base, int64_t stride, int S, float (&acc)[8]) {
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = 0.0f;
  int s = 0;
  for (; s + 4 <= S; s += 4) {
    float4 x[4][2];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float4* b = (const float4*)(base + (int64_t)(s + u) * stride);
      x[u][0] = b[0];
      x[u][1] = b[1];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      acc[0] += x[u][0].x; acc[1] += x[u][0].y; acc[2] += x[u][0].z; acc[3] += x[u][0].w;
      acc[4] += x[u][1].x; acc[5] += x[u][1].y; acc[6] += x[u][1].z; acc[7] += x[u][1].w;
    }
  }
  for (; s < S; ++s) {
    const float4* b = (const float4*)(base + (int64_t)s * stride);
    const float4 x0 = b[0], x1 = b[1];
    acc[0] += x0.x; acc[1] += x0.y; acc[2] += x0.z; acc[3] += x0.w;
    acc[4] += x1.x; acc[5] += x1.y; acc[6] += x1.z; acc[7] += x1.w;
  }
}

// out[i] = sum over splits of part[s][i] (split order), count % 8 == 0; one
// thread per 8 outputs.
__global__ void sum_parts_kernel(const float* __restrict__ part, int S, int64_t count, float* __restrict__ out) {
  const int64_t i8 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (i8 >= count) return;
  float acc[8];
  sum_parts8(part + i8, count, S, acc);
  *(float4*)(out + i8) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  *(float4*)(out + i8 + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
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

__device__ inline uint4 pack8_bf16(const float* v) {
  uint4 o;
  o.x = (uint32_t)bf16_rn_bits(v[0]) | ((uint32_t)bf16_rn_bits(v[1]) << 16);
  o.y = (uint32_t)bf16_rn_bits(v[2]) | ((uint32_t)bf16_rn_bits(v[3]) << 16);
  o.z = (uint32_t)bf16_rn_bits(v[4]) | ((uint32_t)bf16_rn_bits(v[5]) << 16);
  o.w = (uint32_t)bf16_rn_bits(v[6]) | ((uint32_t)bf16_rn_bits(v[7]) << 16);
  return o;
}

struct ExtParams {
  // out = L_R R_R^T + P' J^T + H G  with
  //   P'[i][p] = s_LR s_E praw[i][p] S_R[p]          (rows x kR)
  //   G[q][j]  = S_L[q] (s_F s_RR t1[q][j] + sum_p s_F s_E t2[q][p] S_R[p] J[j][p])
  // praw, t1 and t2 arrive as thin-product partial sums, added in split order:
  //   praw[i][p] = sum_s pa[s][i][p], t1[q][j] = sum_s p1[s][j][q]
  //   (row length 64; split strides rows and cols)
  int64_t rows, cols;
  int kR, kL, ksR, ksL;   // ks*: segment widths (multiples of 16)
  int64_t kext;
  const float* praw;  // [sa][rows][64]
  const float* t1;    // [s1][cols][64]
  const float* t2;    // kL x 64 (summed over its splits before the prep)
  int sa, s1;
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

// A_ext[i] = [hi(P'' s_J) | lo(..) | H_bar | H_bar | 0 ...] (P'' times the
// epilogue's ext_mul, as G below): one thread per
// row and 8-column chunk (rows past e.rows up to the next multiple of 32 are
// written as zeros).  Item id of the rows x chunks grid.
__device__ void ext_prep_a_item(const ExtParams& e, int64_t id) {
  const int64_t chunks = e.kext >> 3;
  const int64_t i = id / chunks;
  const int col0 = (int)(id % chunks) * 8;
  float v[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  uint4 out = make_uint4(0, 0, 0, 0);
  if (i < e.rows && col0 < 2 * e.ksR) {
    const int p0 = col0 % e.ksR;
    const bool lo_half = col0 >= e.ksR;
    const float sc = (e.s_LR[0] * e.s_E[0]);
    const float emul = epi_scale(e.s_LR, e.s_RR).ext_mul;
    float acc[8];
    sum_parts8(e.praw + i * 64 + p0, e.rows * 64, e.sa, acc);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int p = p0 + t;
      if (p < e.kR) {
        const float x = acc[t] * sc * e.S_R[p] * e.J.ts[0] * emul;
        const float hi = bf16_bits_to_float(bf16_rn_bits(x));
        v[t] = lo_half ? x - hi : hi;
      }
    }
    out = pack8_bf16(v);
  } else if (i < e.rows && col0 < 2 * e.ksR + 2 * e.ksL) {
    const int q0 = (col0 - 2 * e.ksR) % e.ksL;
#pragma unroll
    for (int t = 0; t < 8; ++t)
      if (q0 + t < e.kL) v[t] = factor_val(e.H, q0 + t, i);
    out = pack8_bf16(v);
  }
  *(uint4*)(e.a_ext + ext_off(i, col0, e.kext)) = out;
}

// Workgroup bx of nba walks the items bx * 256 + tid, + 256 nba, ...: the
// launch's static LDS (for the B side) limits how many workgroups a CU
// holds, so A_ext is formed by a few workgroups that loop.
__device__ void ext_prep_a(const ExtParams& e, int64_t bx, int64_t nba) {
  const int64_t total = ((e.rows + 31) & ~(int64_t)31) * (e.kext >> 3);
  for (int64_t id = bx * 256 + threadIdx.x; id < total; id += nba * 256) ext_prep_a_item(e, id);
}

// B_ext[j] = [J_bar | J_bar | hi(s_H G) | lo(..) | 0 ...]: one workgroup per
// 64 output columns (rows past e.cols up to the next multiple of 32 are
// zero).  The columns' J_bar and the folded T2 (e.t2: already summed over
// its splits) are staged in LDS; thread (c, part) handles column c and the
// 8-wide chunk groups part, part + 4, ...: J_bar chunks (written twice), G
// chunks (hi and lo from one evaluation) and the zero tail.
constexpr int kExtMaxK = 64;
__device__ void ext_prep_b(const ExtParams& e, int64_t bx, float (*jv)[kExtMaxK + 1],
                           float (*t2f)[kExtMaxK + 1]) {
  const int tid = threadIdx.x;
  const int64_t j0 = bx * 64;
  const float sJ = e.J.ts[0];
  const float sFE = e.s_F[0] * e.s_E[0];
  const float sFR = e.s_F[0] * e.s_RR[0];
  const float sH = e.H.ts[0];
  const float emul = epi_scale(e.s_LR, e.s_RR).ext_mul;
  for (int idx = tid; idx < 64 * e.kR; idx += 256) {
    const int c = idx & 63, pp = idx >> 6;
    jv[c][pp] = (j0 + c < e.cols) ? factor_val(e.J, pp, j0 + c) : 0.0f;
  }
  for (int idx = tid; idx < e.kL * e.kR; idx += 256) {
    const int q = idx / e.kR, pp = idx - q * e.kR;
    t2f[q][pp] = sFE * e.t2[q * 64 + pp] * e.S_R[pp] * sJ;
  }
  __syncthreads();
  const int c = tid & 63, part = tid >> 6;
  const int64_t j = j0 + c;
  if (j >= ((e.cols + 31) & ~(int64_t)31)) return;
  uint16_t* out = e.b_ext;
  const bool live = j < e.cols;
  const uint4 zero = make_uint4(0, 0, 0, 0);
  // J_bar, twice
  for (int p0 = 8 * part; p0 < e.ksR; p0 += 32) {
    float v[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    if (live)
#pragma unroll
      for (int t = 0; t < 8; ++t)
        if (p0 + t < e.kR) v[t] = jv[c][p0 + t];
    const uint4 w = pack8_bf16(v);
    *(uint4*)(out + ext_off(j, p0, e.kext)) = w;
    *(uint4*)(out + ext_off(j, e.ksR + p0, e.kext)) = w;
  }
  // G[q] = s_H S_L[q] (s_F s_RR T1[q][j] + sum_p T2f[q][p] J[j][p]) as hi / lo
  for (int q0 = 8 * part; q0 < e.ksL; q0 += 32) {
    float hi[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    float lo[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    if (live) {
      float t1[8];
      sum_parts8(e.t1 + j * 64 + q0, e.cols * 64, e.s1, t1);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int q = q0 + t;
        if (q < e.kL) {
          float acc = sFR * t1[t];
          for (int pp = 0; pp < e.kR; ++pp) acc += t2f[q][pp] * jv[c][pp];
          const float g = sH * e.S_L[q] * acc * emul;
          hi[t] = bf16_bits_to_float(bf16_rn_bits(g));
          lo[t] = g - hi[t];
        }
      }
    }
    *(uint4*)(out + ext_off(j, 2 * e.ksR + q0, e.kext)) = pack8_bf16(hi);
    *(uint4*)(out + ext_off(j, 2 * e.ksR + e.ksL + q0, e.kext)) = pack8_bf16(lo);
  }
  for (int64_t c0 = 2 * e.ksR + 2 * e.ksL + 8 * part; c0 < e.kext; c0 += 32)
    *(uint4*)(out + ext_off(j, c0, e.kext)) = zero;
}

// Both operands of the K-extension in one launch: workgroups [0, nba) form
// A_ext, the rest B_ext (64 columns each).
__global__ __launch_bounds__(256) void ext_prep_kernel(ExtParams e, int64_t nba) {
  __shared__ float jv[64][kExtMaxK + 1];         // J_bar[j0 + c][p]
  __shared__ float t2f[kExtMaxK][kExtMaxK + 1];  // s_F s_E T2[q][p] S_R[p] s_J
  const int64_t blk = blockIdx.x;
  if (blk < nba)
    ext_prep_a(e, blk, nba);
  else
    ext_prep_b(e, blk - nba, jv, t2f);
}

}  // namespace metis
