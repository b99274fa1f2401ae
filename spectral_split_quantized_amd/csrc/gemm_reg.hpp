// gemm_reg.hpp -- register-dequant NVFP4 GEMM for the large split products
// ("Metis: Training LLMs with FP4 Quantization", 关键设计 1: the split
// forward GEMM; 整体框架: the same split in every forward and backward GEMM).
// Same contract as gemm_fp4_kernel in gemm.hpp (C = alpha (A B^T + the bf16
// K-extension prepared divided by alpha)), restricted to K % 256 == 0 with 16-byte aligned code and
// scale rows.  It lives in its own translation unit so that it can be
// scheduled for instruction-level parallelism without changing the other
// kernels.
#pragma once

#include <type_traits>

#include "gemm_common.hpp"

namespace metis {

// ---------------------------------------------------------------------------
// The raw FP4 codes and E4M3 scales travel from global memory straight into
// a two-stage LDS ring by LDS-DMA loads (global_load_lds: no registers, one
// 256-wide K stage ahead), and every wave expands its own MFMA fragments in
// registers just before use (4 conversions + 4 packed fp16 multiplies per 8
// elements, issued between the matrix instructions of the same wave).
// Rows past M / N are clamped to the last row (their results are never
// stored).
//
// Stage (K = 256 per row): 128 code bytes (one cache line) and 16 scale
// bytes.  One 64-lane DMA moves 8 rows x 128 bytes: lane L takes row L / 8,
// 16-byte chunk (L % 8) ^ (row % 8), so each instruction reads whole lines
// and the XOR swizzle keeps the fragment reads below free of bank conflicts.
// LDS: chunk c of row R at ((R / 8) * 64 + (R % 8) * 8 + (c ^ (R % 8))) * 16;
// the 16 scale bytes of row R at R * 16.
//
// K order inside a stage: the product sums over K, so any permutation used
// alike by both operands gives the same result.  In 64-wide sub-block j,
// MFMA lane half h at sub-step kk takes elements 64 j + 32 h + 8 kk .. + 7:
// each lane reads one 16-byte chunk (c = 2 j + h) per fragment and
// sub-block, and the scale bytes 4 j + 2 h and 4 j + 2 h + 1.
template <int WM, int WN, int TM, int TN>
struct RegCfg {
  static constexpr int NT = WM * WN * 64;
  static constexpr int NW = WM * WN;
  static constexpr int BM = WM * TM * 32;
  static constexpr int BN = WN * TN * 32;
  static constexpr int BK = 256;                       // K per stage
  static constexpr int CODE_A = BM * 128;
  static constexpr int SC_A = BM * 16;
  static constexpr int CODE_B = BN * 128;
  static constexpr int SC_B = BN * 16;
  static constexpr int STAGE = CODE_A + SC_A + CODE_B + SC_B;  // bytes
  static constexpr int DCA = BM / 8, DCB = BN / 8;     // code DMAs per operand
  static constexpr int DSA = BM / 64, DSB = BN / 64;   // scale DMAs per operand
  static constexpr int PCA = DCA / NW, PCB = DCB / NW, PSA = DSA / NW, PSB = DSB / NW;
  static_assert(DCA % NW == 0 && DCB % NW == 0 && DSA % NW == 0 && DSB % NW == 0, "DMA split");
};

__device__ inline uint32_t u4_get(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

template <int WM, int WN, int TM, int TN>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_fp4_reg_kernel(GemmParams p) {
  using Cfg = RegCfg<WM, WN, TM, TN>;
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, NW = Cfg::NW;
  // one array per stage: a read of one stage then does not alias the DMA
  // writes in flight into the other, and the compiler does not wait for them
  __shared__ __attribute__((aligned(16))) uint8_t st0[Cfg::STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t st1[Cfg::STAGE];
  auto stage_base = [&](auto sc) -> uint8_t* {
    if constexpr (decltype(sc)::value == 0) return st0;
    else return st1;
  };
  auto code_a = [&](auto sc) { return stage_base(sc); };
  auto sc_a = [&](auto sc) { return stage_base(sc) + Cfg::CODE_A; };
  auto code_b = [&](auto sc) { return stage_base(sc) + Cfg::CODE_A + Cfg::SC_A; };
  auto sc_b = [&](auto sc) { return stage_base(sc) + Cfg::CODE_A + Cfg::SC_A + Cfg::CODE_B; };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;

  const int tid = threadIdx.x;
  // the wave index is uniform: keep it (and every LDS destination derived
  // from it) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
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
  const EpiScale es = epi_scale(p.sa, p.sb);
  const int64_t nk = kend > kbeg && !es.skip_main ? (kend - kbeg) / BK : 0;

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16_t{};

  // this lane's DMA rows (clamped into the matrix when the DMA is issued;
  // addresses are formed per DMA so that no pointer array stays live)
  const int dr = lane >> 3;                      // row inside an 8-row DMA
  const int dc = (lane & 7) ^ dr;                // chunk this lane fetches
  const int64_t cra = m0 + wave * 8 + dr, crb = n0 + wave * 8 + dr;  // + 8 NW d
  const int64_t sra = m0 + wave * 64 + lane, srb = n0 + wave * 64 + lane;  // + 64 NW d
  const int64_t cbytes = p.K >> 1, sbytes = p.K >> 4;
  // DMA of stage kt into ring slot s (wave-uniform LDS destinations)
  auto issue = [&](int64_t kt, auto s) {
    const int64_t co = ((kbeg + kt * BK) >> 1) + 16 * dc, so = (kbeg + kt * BK) >> 4;
#pragma unroll
    for (int d = 0; d < Cfg::PCA; ++d)
      dma16(p.a_codes + min(cra + 8 * NW * d, p.M - 1) * cbytes + co, code_a(s) + (wave + d * NW) * 1024);
#pragma unroll
    for (int d = 0; d < Cfg::PCB; ++d)
      dma16(p.b_codes + min(crb + 8 * NW * d, p.N - 1) * cbytes + co, code_b(s) + (wave + d * NW) * 1024);
#pragma unroll
    for (int d = 0; d < Cfg::PSA; ++d)
      dma16(p.a_scales + min(sra + 64 * NW * d, p.M - 1) * sbytes + so, sc_a(s) + (wave + d * NW) * 1024);
#pragma unroll
    for (int d = 0; d < Cfg::PSB; ++d)
      dma16(p.b_scales + min(srb + 64 * NW * d, p.N - 1) * sbytes + so, sc_b(s) + (wave + d * NW) * 1024);
  };

  // fragment reads: row R = g * 32 + (lane & 31), chunk c = 2 j + h
  const int hh = lane >> 5, li = lane & 31, lr8 = li & 7;
  // two register sets of raw fragments: a sub-block's codes and scales are
  // read into one set while the previous sub-block expands from the other
  uint4 ac[2][TM], bc[2][TN];      // 16 code bytes per fragment
  uint32_t as[2][TM], bs[2][TN];   // fp16 scales of this lane's two blocks
  using F0 = std::integral_constant<int, 0>;
  using F1 = std::integral_constant<int, 1>;
  auto read_frags = [&](auto s, int j, auto f) {
    constexpr int F = decltype(f)::value;
    const int sw = ((2 * j + hh) ^ lr8) * 16 + lr8 * 128;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int R = (wm * TM + i) * 32 + li;
      ac[F][i] = *(const uint4*)(code_a(s) + (R >> 3) * 1024 + sw);
      as[F][i] = *(const uint32_t*)(sc_a(s) + R * 16 + 4 * j);
    }
#pragma unroll
    for (int jn = 0; jn < TN; ++jn) {
      const int R = (wn * TN + jn) * 32 + li;
      bc[F][jn] = *(const uint4*)(code_b(s) + (R >> 3) * 1024 + sw);
      bs[F][jn] = *(const uint32_t*)(sc_b(s) + R * 16 + 4 * j);
    }
  };
  // blocks 4 j + 2 h and 4 j + 2 h + 1 -> {s, s'} in fp16 (exact)
  auto cvt_scales = [&](auto f) {
    constexpr int F = decltype(f)::value;
#pragma unroll
    for (int i = 0; i < TM; ++i)
      as[F][i] = __builtin_bit_cast(uint32_t,
                                    __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(as[F][i] >> (16 * hh), 1.0f, false));
#pragma unroll
    for (int jn = 0; jn < TN; ++jn)
      bs[F][jn] = __builtin_bit_cast(uint32_t,
                                     __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bs[F][jn] >> (16 * hh), 1.0f, false));
  };
  // {s, s} or {s', s'}: a broadcast the packed multiply takes by operand
  // selection, with no instruction of its own
  auto pair = [](uint32_t s2, int kk) {
    const half2_t h = __builtin_bit_cast(half2_t, s2);
    return (kk < 2) ? __builtin_shufflevector(h, h, 0, 0) : __builtin_shufflevector(h, h, 1, 1);
  };
  auto expand = [&](int kk, half8_t* af, half8_t* bf, auto f) {
    constexpr int F = decltype(f)::value;
#pragma unroll
    for (int i = 0; i < TM; ++i)
      af[i] = __builtin_bit_cast(half8_t, dequant8(u4_get(ac[F][i], kk), pair(as[F][i], kk)));
#pragma unroll
    for (int jn = 0; jn < TN; ++jn)
      bf[jn] = __builtin_bit_cast(half8_t, dequant8(u4_get(bc[F][jn], kk), pair(bs[F][jn], kk)));
  };
  auto mfmas = [&](const half8_t* af, const half8_t* bf) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int jn = 0; jn < TN; ++jn)
        acc[i][jn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[jn], acc[i][jn], 0, 0, 0);
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
  // the sub-block's last sub-step: its raw fragments were read a sub-block
  // earlier, so the scale conversion and the expansion of the next sub-step
  // 0 spread evenly over the MFMAs (six VALU each)
  auto interleave_tail = [&]() {
#pragma unroll
    for (int t = 0; t < TM * TN; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
    }
  };

  // K-extension stages (bf16, kext % 64 == 0) travel through the same LDS
  // ring after the FP4 stages: stage e holds sub-steps 4 e .. 4 e + 3 of the
  // tile's 32-row groups, each (group, sub-step) fragment the 1 KB block the
  // extension layout stores contiguously, at ((group * 4 + sub-step) * 1 KB)
  // for A and EA KB further for B.  Groups past the matrix are clamped to
  // its last group (padded rows are zeros; their results are never stored).
  constexpr int EA = (BM / 32) * 4, EB = (BN / 32) * 4;  // 1 KB blocks per stage
  static_assert(EA % NW == 0 && EB % NW == 0 && (EA + EB) * 1024 <= Cfg::STAGE, "extension stage");
  const int64_t ne = p.kext >> 6, kx16 = p.kext >> 4;
  const int64_t gla = (p.M - 1) >> 5, glb = (p.N - 1) >> 5;
  auto issue_ext = [&](int64_t e, auto s) __attribute__((always_inline)) {
#pragma unroll
    for (int d = 0; d < EA / NW; ++d) {
      const int idx = wave + d * NW;
      const int64_t g = min((m0 >> 5) + (idx >> 2), gla);
      dma16(p.a_ext + ((g * kx16 + 4 * e + (idx & 3)) * 64 + lane) * 8, stage_base(s) + idx * 1024);
    }
#pragma unroll
    for (int d = 0; d < EB / NW; ++d) {
      const int idx = wave + d * NW;
      const int64_t g = min((n0 >> 5) + (idx >> 2), glb);
      dma16(p.b_ext + ((g * kx16 + 4 * e + (idx & 3)) * 64 + lane) * 8, stage_base(s) + (EA + idx) * 1024);
    }
  };
  half8_t a0[TM], b0[TN], a1[TM], b1[TN];
  // sub-steps 0..2 of the current 64-wide sub-block (sub-step 0 expanded;
  // its raw fragments in set f)
  auto sub_head = [&](auto f) {
    mfmas(a0, b0);
    expand(1, a1, b1, f);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    mfmas(a1, b1);
    expand(2, a0, b0, f);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    mfmas(a0, b0);
    expand(3, a1, b1, f);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
  };
  // sub-step 3 of the current sub-block, with the scale conversion and the
  // sub-step 0 expansion of the next sub-block (raw fragments in set g)
  auto sub_tail = [&](auto g) {
    mfmas(a1, b1);
    cvt_scales(g);
    expand(0, a0, b0, g);
    interleave_tail();
    __builtin_amdgcn_sched_barrier(0);
  };
  // Stage kt sits in ring slot S with its sub-block 0 fragments in register
  // set 0 (sub-step 0 expanded).  It first issues the DMA of stage kt + 1
  // into the other slot (every wave finished reading it before the previous
  // barrier).  The raw fragments of sub-block j + 1 are read into the other
  // register set when sub-block j starts, a whole sub-block ahead of their
  // use.  Sub-block 3's fragments were read (and consumed) before sub-block
  // 3 starts, so there every wave waits for its DMA and the barrier
  // publishes the other slot, whose sub-block 0 is then read.  A DMA past
  // the last stage repeats it into a slot that is never read again.
  auto stage_step = [&](int64_t kt, auto sc) {
    using SN = std::integral_constant<int, 1 - decltype(sc)::value>;
    issue(kt + 1 < nk ? kt + 1 : kt, SN{});
    read_frags(sc, 1, F1{});
    sub_head(F0{});
    sub_tail(F1{});
    read_frags(sc, 2, F0{});
    sub_head(F1{});
    sub_tail(F0{});
    read_frags(sc, 3, F1{});
    sub_head(F0{});
    sub_tail(F1{});
    ring_barrier();
    read_frags(SN{}, 0, F0{});
    sub_head(F1{});
    sub_tail(F0{});
  };

  if (nk > 0) {
    issue((int64_t)0, S0{});
    ring_barrier();
    read_frags(S0{}, 0, F0{});
    cvt_scales(F0{});
    expand(0, a0, b0, F0{});
    __builtin_amdgcn_sched_barrier(0);
    for (int64_t kt = 0; kt < nk; kt += 2) {
      stage_step(kt, S0{});
      if (kt + 1 < nk) stage_step(kt + 1, S1{});
    }
  }

  // ---- K-extension: stage e sits in ring slot (nk - 1 + e) % 2; every wave
  // reads its fragments of a sub-step straight from the stage (lane L at
  // block offset 16 L) while the next stage's DMA is in flight
  auto ext_step = [&](int64_t e, auto sc) __attribute__((always_inline)) {
    using SN = std::integral_constant<int, 1 - decltype(sc)::value>;
    if (e + 1 < ne) issue_ext(e + 1, SN{});
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      bf16x8_t ea[TM], eb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        ea[i] = *(const bf16x8_t*)(stage_base(sc) + ((wm * TM + i) * 4 + u) * 1024 + lane * 16);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        eb[j] = *(const bf16x8_t*)(stage_base(sc) + (EA + (wn * TN + j) * 4 + u) * 1024 + lane * 16);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ea[i], eb[j], acc[i][j], 0, 0, 0);
    }
    ring_barrier();
  };
  auto ext_loop = [&](auto first) __attribute__((always_inline)) {
    using SB = std::integral_constant<int, 1 - decltype(first)::value>;
    for (int64_t e = 0; e < ne; e += 2) {
      ext_step(e, first);
      if (e + 1 < ne) ext_step(e + 1, SB{});
    }
  };
  if (ne > 0) {
    // both slots are free once every wave is past this barrier (the main
    // loop's last DMA, into either slot, has landed and its last reads are
    // done), so the extension always starts in slot 0: one loop instance,
    // whose accumulators stay where the main loop left them
    if (nk > 0) ring_barrier();
    issue_ext(0, S0{});
    ring_barrier();
    ext_loop(S0{});
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
          __builtin_nontemporal_store(y, &C[row * p.ldc + col]);
        }
      }
    }
  }
}

}  // namespace metis
