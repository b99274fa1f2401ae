// mxfp4_gemm.hpp -- C = A B^T of two MXFP4 operands (format: mxfp4.hpp) on
// gfx950's block-scaled FP4 matrix instruction.  Lives in the translation
// unit of the other large GEMM (instruction-level-parallelism scheduling).
//
// v_mfma_scale_f32_32x32x64_f8f6f4 with both operands in FP4 takes, in lane
// l, the 32 K-consecutive elements 32 (l / 32) .. + 31 of row l % 32 (16
// bytes, element 2i in the low nibble of byte i) and that row's E8M0 scale of
// the same 32-block (byte 0 of a register).  No element is expanded in
// registers.
#pragma once

#include <type_traits>

#include "gemm_common.hpp"

namespace metis {

struct MxGemmParams {
  int64_t M, N, K;  // K % 1024 == 0
  const uint8_t* a_codes;   // [M][K / 2]
  const uint8_t* a_scales;  // [M][K / 32]
  const uint8_t* b_codes;   // [N][K / 2]
  const uint8_t* b_scales;  // [N][K / 32]
  float* C;
  int64_t ldc;
};

typedef int int32x8_t __attribute__((ext_vector_type(8)));

// C = A B^T with 256 x 256 tiles (4 waves of 128 x 128, 4 x 4 instructions of
// 32 x 32 x 64 each).  The codes travel global -> LDS by DMA into a two-slot
// ring one K-stage (256) ahead, in the swizzled image of the NVFP4 kernel: a
// row's 128 code bytes of a stage as 16-byte chunks, chunk c of row R at
// ((R / 8) * 64 + (R % 8) * 8 + (c ^ (R % 8))) * 16, which lane half h of
// sub-step kk reads as chunk 2 kk + h.  The scales of two stages (16 bytes a
// row) travel the same way into a second two-slot ring, one pair of stages
// ahead.  Rows past M / N are clamped to the last row (never stored).
template <int WM, int WN, int TM, int TN>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mx_gemm_kernel(MxGemmParams p) {
  constexpr int NW = WM * WN, BM = WM * TM * 32, BN = WN * TN * 32;
  constexpr int CODE_A = BM * 128, STAGE = CODE_A + BN * 128;  // bytes
  constexpr int SCW_A = BM * 16, SCW = SCW_A + BN * 16;
  constexpr int PCA = BM / 8 / NW, PCB = BN / 8 / NW, PSA = BM / 64 / NW, PSB = BN / 64 / NW;
  static_assert(PCA * 8 * NW == BM && PCB * 8 * NW == BN && PSA * 64 * NW == BM && PSB * 64 * NW == BN, "DMA split");
  __shared__ __attribute__((aligned(16))) uint8_t st0[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t st1[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sw0[SCW];
  __shared__ __attribute__((aligned(16))) uint8_t sw1[SCW];
  auto code_a = [&](auto s) -> uint8_t* {
    if constexpr (decltype(s)::value == 0) return st0;
    else return st1;
  };
  auto code_b = [&](auto s) { return code_a(s) + CODE_A; };
  auto scw_a = [&](auto w) -> uint8_t* {
    if constexpr (decltype(w)::value == 0) return sw0;
    else return sw1;
  };
  auto scw_b = [&](auto w) { return scw_a(w) + SCW_A; };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wm = wave / WN, wn = wave % WN;
  const int64_t tiles_m = ceil_div<int64_t>(p.M, BM), tiles_n = ceil_div<int64_t>(p.N, BN);
  const int64_t tile = remap_tile(blockIdx.x, tiles_m, tiles_n);
  const int64_t m0 = (tile / tiles_n) * BM, n0 = (tile % tiles_n) * BN;
  const int64_t nk = p.K / 256;
  const int64_t cbytes = p.K >> 1, sbytes = p.K >> 5;

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16_t{};

  // a code DMA moves 8 whole rows: its row group starts at a wave-uniform row
  // (groups past the matrix are clamped to its last group; M and N are
  // multiples of 8), and each lane adds the same 32-bit offset to it
  const int dr = lane >> 3, dc = (lane & 7) ^ dr;
  const uint32_t lane_off = (uint32_t)(dr * cbytes + 16 * dc);
  const int64_t sra = m0 + wave * 64 + lane, srb = n0 + wave * 64 + lane;
  auto issue_codes = [&](int64_t kt, auto s) {
#pragma unroll
    for (int d = 0; d < PCA; ++d) {
      const int64_t g = min(m0 + (wave + d * NW) * 8, p.M - 8);
      dma16(p.a_codes + g * cbytes + kt * 128 + lane_off, code_a(s) + (wave + d * NW) * 1024);
    }
#pragma unroll
    for (int d = 0; d < PCB; ++d) {
      const int64_t g = min(n0 + (wave + d * NW) * 8, p.N - 8);
      dma16(p.b_codes + g * cbytes + kt * 128 + lane_off, code_b(s) + (wave + d * NW) * 1024);
    }
  };
  // scales of stages 2 w and 2 w + 1: 16 bytes a row, row R at R * 16
  auto issue_scales = [&](int64_t w, auto ws) {
#pragma unroll
    for (int d = 0; d < PSA; ++d)
      dma16(p.a_scales + min(sra + 64 * NW * d, p.M - 1) * sbytes + w * 16, scw_a(ws) + (wave + d * NW) * 1024);
#pragma unroll
    for (int d = 0; d < PSB; ++d)
      dma16(p.b_scales + min(srb + 64 * NW * d, p.N - 1) * sbytes + w * 16, scw_b(ws) + (wave + d * NW) * 1024);
  };

  const int hh = lane >> 5, li = lane & 31, lr8 = li & 7;
  // one K-stage from code slot s with scale window ws (half: which of its two stages)
  auto stage = [&](auto s, auto ws, int half) {
    uint32_t sa[TM], sb[TN];  // this lane's four scale bytes of the stage (byte kk: sub-step kk)
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const uint2 g = *(const uint2*)(scw_a(ws) + ((wm * TM + i) * 32 + li) * 16 + half * 8);
      sa[i] = __builtin_amdgcn_perm(g.y, g.x, hh ? 0x07050301u : 0x06040200u);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const uint2 g = *(const uint2*)(scw_b(ws) + ((wn * TN + j) * 32 + li) * 16 + half * 8);
      sb[j] = __builtin_amdgcn_perm(g.y, g.x, hh ? 0x07050301u : 0x06040200u);
    }
    // fragments of sub-step kk + 1 are read from LDS under the 16 matrix
    // instructions of sub-step kk (one read after each of the first eight)
    uint4 fa[2][TM], fb[2][TN];
    auto read = [&](int kk, int buf) {
      const int sw = ((2 * kk + hh) ^ lr8) * 16 + lr8 * 128;
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[buf][i] = *(const uint4*)(code_a(s) + ((wm * TM + i) * 32 + li) / 8 * 1024 + sw);
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[buf][j] = *(const uint4*)(code_b(s) + ((wn * TN + j) * 32 + li) / 8 * 1024 + sw);
    };
    read(0, 0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int cur = kk & 1;
      if (kk < 3) read(kk + 1, cur ^ 1);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const uint4 a = fa[cur][i], b = fb[cur][j];
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              int32x8_t{(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0},
              int32x8_t{(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0}, acc[i][j], 4, 4, 0,
              (int)(sa[i] >> (8 * kk)), 0, (int)(sb[j] >> (8 * kk)));
        }
#pragma unroll
      for (int t = 0; t < TM * TN; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        if (kk < 3 && t < TM + TN) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // stages 2 w (slot 0) and 2 w + 1 (slot 1) of window w (scale slot w % 2)
  auto pair = [&](int64_t w, auto ws) {
    using WN_ = std::integral_constant<int, 1 - decltype(ws)::value>;
    const int64_t kt = 2 * w;
    issue_codes(kt + 1, S1{});
    stage(S0{}, ws, 0);
    ring_barrier();
    // past the last pair the DMAs repeat data into slots never read again
    issue_codes(kt + 2 < nk ? kt + 2 : kt + 1, S0{});
    issue_scales(w + 1 < nk / 2 ? w + 1 : w, WN_{});
    stage(S1{}, ws, 1);
    ring_barrier();
  };
  issue_codes(0, S0{});
  issue_scales(0, S0{});
  ring_barrier();
  for (int64_t w = 0; w < nk / 2; w += 2) {  // nk / 2 is even (K % 1024 == 0)
    pair(w, S0{});
    pair(w + 1, S1{});
  }

  // ---- epilogue: lane holds column lane % 32 and rows 8 (v / 4) + 4 (lane / 32) + v % 4
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t col = n0 + (wn * TN + j) * 32 + li;
      if (col >= p.N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + (wm * TM + i) * 32 + 8 * (v >> 2) + 4 * hh + (v & 3);
        if (row < p.M) __builtin_nontemporal_store(acc[i][j][v], &p.C[row * p.ldc + col]);
      }
    }
  }
}

}  // namespace metis
