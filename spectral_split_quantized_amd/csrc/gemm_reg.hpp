// gemm_reg.hpp -- register-dequant NVFP4 GEMM for the large split products
// ("Metis: Training LLMs with FP4 Quantization", 关键设计 1: the split
// forward GEMM; 整体框架: the same split in every forward and backward GEMM).
// Same contract as gemm_fp4_kernel in gemm.hpp (C = alpha A B^T + the bf16
// K-extension), restricted to K % 64 == 0 with 16-byte aligned code rows.
// It lives in its own translation unit so that it can be scheduled for
// instruction-level parallelism without changing the other kernels.
#pragma once

#include <type_traits>

#include "gemm_common.hpp"

namespace metis {
// ---------------------------------------------------------------------------
// Register-dequant variant for K % 64 == 0 (the large products).  The raw
// FP4 codes (32 bytes per row and K step) and E4M3 scales (4 bytes) travel
// from global memory straight into an NS-stage LDS ring by LDS-DMA loads
// (global_load_lds, no registers, NS - 1 steps ahead), and every wave
// expands its own MFMA fragments in registers just before use.  LDS traffic
// per MFMA is a quarter of an fp16-staged tile, and the expansion (4
// conversions + 4 packed multiplies per 8 elements) issues between the
// matrix instructions of the same wave.  Rows past M / N are clamped to the
// last row (their results are never stored).
//
// K order inside a step: the product sums over K, so any permutation used
// alike by both operands gives the same result.  MFMA lane half h at
// sub-step kk takes the row's elements 32 h + 8 kk .. + 7, so each lane
// reads 16 contiguous code bytes of its row and the LDS image is exactly
// what the DMA writes.  LDS per stage and operand: codes of row g*32 + i,
// half h at ((g * 2 + h) * 32 + i) * 16 (one 64-lane DMA per 32-row group
// g), scales of row r at r * 4.
template <int WM, int WN, int TM, int TN, int NS>
struct RegCfg {
  static constexpr int NT = WM * WN * 64;
  static constexpr int NW = WM * WN;
  static constexpr int BM = WM * TM * 32;
  static constexpr int BN = WN * TN * 32;
  static constexpr int BK = 64;
  static constexpr int GA = BM / 32, GB = BN / 32;  // code DMAs per operand
  static constexpr int QA = BM / 64, QB = BN / 64;  // scale DMAs per operand
  static constexpr int CODE_A = BM * 32;
  static constexpr int SC_A = BM * 4;
  static constexpr int CODE_B = BN * 32;
  static constexpr int SC_B = BN * 4;
  static constexpr int STAGE = CODE_A + SC_A + CODE_B + SC_B;  // bytes
  static constexpr int LDS = NS * STAGE;
  static constexpr int DA = GA / NW, DB = GB / NW, SA = QA / NW, SB = QB / NW;  // per wave
  static constexpr int DMAS = DA + DB + SA + SB;  // DMA instructions per wave and step
  static_assert(GA % NW == 0 && GB % NW == 0 && QA % NW == 0 && QB % NW == 0, "DMA split");
};

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ inline void dma16(const void* g, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t*)lds, 16, 0, 0);
}
__device__ inline void dma4(const void* g, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t*)lds, 4, 0, 0);
}

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt in bits 3:0
// and 15:14, expcnt 6:4, lgkmcnt 11:8)
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier for the DMA ring.  Every wave first waits for its own
// DMAs into the stage about to be read (wait_vmcnt); the LDS is written only
// by those DMAs, so no release fence is needed (__syncthreads() would drain
// every DMA in flight, including the ones meant to stay in flight).  The
// empty asm keeps the compiler from moving LDS reads above the barrier.
__device__ inline void ring_barrier() {
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ inline uint32_t u4_get(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

template <int WM, int WN, int TM, int TN, int NS>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_fp4_reg_kernel(GemmParams p) {
  using Cfg = RegCfg<WM, WN, TM, TN, NS>;
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK;
  static_assert(NS >= 2 && NS <= 4, "stage count");
  // one array per stage: the compiler then sees that a read of one stage
  // does not alias the DMA writes in flight into the others, and does not
  // wait for them
  __shared__ __attribute__((aligned(16))) uint8_t st0[Cfg::STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t st1[Cfg::STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t st2[NS > 2 ? Cfg::STAGE : 16];
  __shared__ __attribute__((aligned(16))) uint8_t st3[NS > 3 ? Cfg::STAGE : 16];
  auto stage_base = [&](auto sc) -> uint8_t* {
    constexpr int S = decltype(sc)::value;
    if constexpr (S == 0) return st0;
    else if constexpr (S == 1) return st1;
    else if constexpr (S == 2) return st2;
    else return st3;
  };
  auto code_a = [&](auto sc) { return stage_base(sc); };
  auto sc_a = [&](auto sc) { return stage_base(sc) + Cfg::CODE_A; };
  auto code_b = [&](auto sc) { return stage_base(sc) + Cfg::CODE_A + Cfg::SC_A; };
  auto sc_b = [&](auto sc) { return stage_base(sc) + Cfg::CODE_A + Cfg::SC_A + Cfg::CODE_B; };

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave / WN, wn = wave % WN;
  const int64_t tiles_m = ceil_div<int64_t>(p.M, BM);
  const int64_t tiles_n = ceil_div<int64_t>(p.N, BN);
  const int64_t tile = remap_tile(blockIdx.x, tiles_m, tiles_n);
  const int64_t m0 = (tile / tiles_n) * BM;
  const int64_t n0 = (tile % tiles_n) * BN;
  const int64_t nsplit = gridDim.y;
  const int64_t kper = ceil_div<int64_t>(p.K / BK, nsplit) * BK;
  const int64_t kbeg = (int64_t)blockIdx.y * kper;
  const int64_t kend = min(p.K, kbeg + kper);
  const int64_t nk = kend > kbeg ? (kend - kbeg) / BK : 0;

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16_t{};

  // this lane's DMA sources at K step 0 (rows clamped into the matrix)
  const uint8_t* ga[Cfg::DA];
  const uint8_t* gb[Cfg::DB];
  const uint8_t* gsa[Cfg::SA];
  const uint8_t* gsb[Cfg::SB];
#pragma unroll
  for (int d = 0; d < Cfg::DA; ++d) {
    const int64_t row = min(m0 + (wave + d * Cfg::NW) * 32 + (lane & 31), p.M - 1);
    ga[d] = p.a_codes + row * (p.K >> 1) + (kbeg >> 1) + 16 * (lane >> 5);
  }
#pragma unroll
  for (int d = 0; d < Cfg::DB; ++d) {
    const int64_t row = min(n0 + (wave + d * Cfg::NW) * 32 + (lane & 31), p.N - 1);
    gb[d] = p.b_codes + row * (p.K >> 1) + (kbeg >> 1) + 16 * (lane >> 5);
  }
#pragma unroll
  for (int d = 0; d < Cfg::SA; ++d) {
    const int64_t row = min(m0 + (wave + d * Cfg::NW) * 64 + lane, p.M - 1);
    gsa[d] = p.a_scales + row * (p.K >> 4) + (kbeg >> 4);
  }
#pragma unroll
  for (int d = 0; d < Cfg::SB; ++d) {
    const int64_t row = min(n0 + (wave + d * Cfg::NW) * 64 + lane, p.N - 1);
    gsb[d] = p.b_scales + row * (p.K >> 4) + (kbeg >> 4);
  }
  // DMA of K step kt into stage s (wave-uniform LDS destinations)
  auto issue = [&](int64_t kt, auto s) {
    const int64_t co = kt * (BK / 2), so = kt * (BK / 16);
#pragma unroll
    for (int d = 0; d < Cfg::DA; ++d) dma16(ga[d] + co, code_a(s) + (wave + d * Cfg::NW) * 1024);
#pragma unroll
    for (int d = 0; d < Cfg::DB; ++d) dma16(gb[d] + co, code_b(s) + (wave + d * Cfg::NW) * 1024);
#pragma unroll
    for (int d = 0; d < Cfg::SA; ++d) dma4(gsa[d] + so, sc_a(s) + (wave + d * Cfg::NW) * 256);
#pragma unroll
    for (int d = 0; d < Cfg::SB; ++d) dma4(gsb[d] + so, sc_b(s) + (wave + d * Cfg::NW) * 256);
  };

  uint4 ac[TM], bc[TN];      // 16 code bytes per fragment
  uint32_t as[TM], bs[TN];   // fp16 scales of this lane's two blocks
  const int hsh = 16 * (lane >> 5);
  auto read_frags = [&](auto s) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int g = wm * TM + i;
      ac[i] = *(const uint4*)(code_a(s) + (g * 64 + lane) * 16);
      as[i] = *(const uint32_t*)(sc_a(s) + (g * 32 + (lane & 31)) * 4);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int g = wn * TN + j;
      bc[j] = *(const uint4*)(code_b(s) + (g * 64 + lane) * 16);
      bs[j] = *(const uint32_t*)(sc_b(s) + (g * 32 + (lane & 31)) * 4);
    }
  };
  // blocks 2h and 2h + 1 of the row -> {s_2h, s_2h+1} in fp16 (exact)
  auto cvt_scales = [&]() {
#pragma unroll
    for (int i = 0; i < TM; ++i)
      as[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(as[i] >> hsh, 1.0f, false));
#pragma unroll
    for (int j = 0; j < TN; ++j)
      bs[j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bs[j] >> hsh, 1.0f, false));
  };
  auto pair = [](uint32_t s2, int kk) {
    const uint32_t h = (kk < 2) ? (s2 & 0xFFFFu) : (s2 >> 16);
    return __builtin_bit_cast(half2_t, h | (h << 16));
  };
  auto expand = [&](int kk, half8_t* af, half8_t* bf) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
      af[i] = __builtin_bit_cast(half8_t, dequant8(u4_get(ac[i], kk), pair(as[i], kk)));
#pragma unroll
    for (int j = 0; j < TN; ++j)
      bf[j] = __builtin_bit_cast(half8_t, dequant8(u4_get(bc[j], kk), pair(bs[j], kk)));
  };
  auto mfmas = [&](const half8_t* af, const half8_t* bf) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
  };
  // One MFMA then four VALU instructions, TM * TN times: the expansion of
  // the next sub-step issues in the shadow of this sub-step's matrix ops.
  auto interleave = [&]() {
#pragma unroll
    for (int t = 0; t < TM * TN; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
    }
  };

  // Step kt computes from stage kt % NS: its fragments are in registers and
  // sub-step 0 is already expanded (a0, b0).  It first issues the DMA of
  // step kt + NS - 1 into the stage step kt - 1 used (every wave finished
  // reading it before the previous barrier); sub-steps 0..2 multiply while
  // the next sub-step expands.  Before the barrier each wave waits for its
  // own DMA of step kt + 1 (the (NS - 2) * DMAS instructions issued after it
  // may stay in flight); after the barrier it reads step kt + 1's fragments,
  // and sub-step 3's MFMAs cover their latency and then the expansion of
  // step kt + 1's sub-step 0.  DMAs past the last step repeat it into stages
  // that are never read again.  The loop is unrolled NS times so that every
  // stage is named at compile time.
  half8_t a0[TM], b0[TN], a1[TM], b1[TN];
  auto step = [&](int64_t kt, auto sc) {
    constexpr int S = decltype(sc)::value;
    constexpr int SN = (S + NS - 1) % NS;  // stage of step kt + NS - 1
    constexpr int S1 = (S + 1) % NS;       // stage of step kt + 1
    const int64_t kn = kt + NS - 1;
    mfmas(a0, b0);
    expand(1, a1, b1);
    issue(kn < nk ? kn : nk - 1, std::integral_constant<int, SN>{});
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    mfmas(a1, b1);
    expand(2, a0, b0);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    mfmas(a0, b0);
    expand(3, a1, b1);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<(NS - 2) * Cfg::DMAS>();
    ring_barrier();
    read_frags(std::integral_constant<int, S1>{});
    mfmas(a1, b1);
    cvt_scales();
    expand(0, a0, b0);
    // four MFMAs cover the LDS reads, then one MFMA per five VALU
#pragma unroll
    for (int t = 0; t < 4; ++t) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
    for (int t = 4; t < TM * TN; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  if (nk > 0) {
    // steps 0 .. NS - 2 into stages 0 .. NS - 2; step 0 issues step NS - 1
    issue((int64_t)0, std::integral_constant<int, 0>{});
    if constexpr (NS > 2) issue(nk > 1 ? (int64_t)1 : nk - 1, std::integral_constant<int, 1>{});
    if constexpr (NS > 3) issue(nk > 2 ? (int64_t)2 : nk - 1, std::integral_constant<int, 2>{});
    wait_vmcnt<(NS - 2) * Cfg::DMAS>();
    ring_barrier();
    read_frags(std::integral_constant<int, 0>{});
    cvt_scales();
    expand(0, a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    for (int64_t kt = 0; kt < nk; kt += NS) {
      step(kt, std::integral_constant<int, 0>{});
      if (kt + 1 < nk) step(kt + 1, std::integral_constant<int, 1>{});
      if constexpr (NS > 2) if (kt + 2 < nk) step(kt + 2, std::integral_constant<int, 2>{});
      if constexpr (NS > 3) if (kt + 3 < nk) step(kt + 3, std::integral_constant<int, 3>{});
    }
  }

  float alpha = 1.0f;
  if (p.sa) alpha *= p.sa[0];
  if (p.sb) alpha *= p.sb[0];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] *= alpha;

  // ---- K-extension (bf16, kext % 64 == 0): fragments straight from global
  // memory, four 16-wide sub-steps in flight ahead of the one multiplying
  if (p.kext > 0) {
    const uint16_t* ap[TM];
    const uint16_t* bp[TN];
    // 32-row groups past the matrix are clamped to its last group (padded
    // rows are zeros; their results are never stored)
    const int64_t gla = (p.M - 1) >> 5, glb = (p.N - 1) >> 5;
#pragma unroll
    for (int i = 0; i < TM; ++i)
      ap[i] = p.a_ext + ext_off(min((m0 >> 5) + wm * TM + i, gla) * 32 + (lane & 31), 8 * (lane >> 5), p.kext);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      bp[j] = p.b_ext + ext_off(min((n0 >> 5) + wn * TN + j, glb) * 32 + (lane & 31), 8 * (lane >> 5), p.kext);
    bf16x8_t ea[4][TM], eb[4][TN];
    // sub-step kk of a fragment is 512 elements past sub-step kk - 1
    auto eload = [&](int u, int64_t k0) {
#pragma unroll
      for (int i = 0; i < TM; ++i) ea[u][i] = *(const bf16x8_t*)(ap[i] + (k0 >> 4) * 512);
#pragma unroll
      for (int j = 0; j < TN; ++j) eb[u][j] = *(const bf16x8_t*)(bp[j] + (k0 >> 4) * 512);
    };
#pragma unroll
    for (int u = 0; u < 4; ++u) eload(u, 16 * u);
    for (int64_t k0 = 0; k0 < p.kext; k0 += 64) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ea[u][i], eb[u][j], acc[i][j], 0, 0, 0);
        // the last four refills repeat the final sub-step (never used)
        const int64_t kn = k0 + 64 + 16 * u;
        eload(u, kn < p.kext ? kn : p.kext - 16);
      }
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

}  // namespace metis
