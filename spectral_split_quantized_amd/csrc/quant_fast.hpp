// quant_fast.hpp -- the two NVFP4 quantiser sweeps (quant.hpp) for whole-tile
// bf16 operands: rows % 128 == 0, cols % 64 == 0, 16-byte aligned rows.  Same
// definitions, same residual (the shared lowrank_mfma / lowrank_subtract), a
// different schedule built for HBM streaming on gfx950:
//   - work items are (128-row panel, chunk of 64-column tiles), ordered so
//     that an XCD sweeps a block of 16 panels chunk by chunk: the rank-k
//     fragments hit in its L2, and the axis-0 outputs of neighbouring panels
//     (64 code bytes and 8 scale bytes of each column per panel) complete
//     each other's cache lines there;
//   - a workgroup walks a fixed number of tiles, fully unrolled, so every
//     wait for memory is a compile-time count; M rows are prefetched two
//     tiles ahead into three rotating register sets; the tile's vcat
//     fragments stream into a two-slot LDS ring by direct global->LDS loads;
//     the rank-k MFMA of tile t+1 is issued before tile t is reduced or
//     quantised, so the matrix pipe works under the vector work; one
//     workgroup barrier per tile;
//   - pass 2 takes 1 / (s_b s_g) from a per-tensor table of the 127 block
//     scales, and writes 16-byte code groups (lanes exchange halves with
//     v_permlane32_swap).
#pragma once

#include "quant.hpp"

namespace metis {

// Work item of a workgroup: rows r0 .. r0 + 127, the TPW column tiles from
// ct0 (n of them inside the operand).  Items are numbered block by block,
// a block being kQfPB consecutive panels (the last may have fewer) swept
// chunk by chunk, panels innermost: w = b (kQfPB C) + c Pb + (p - b kQfPB)
// for C chunks and Pb panels in block b.  Workgroup id i runs on XCD i % 8
// and XCD x takes items [x per, (x + 1) per) in id order, so an XCD works
// through whole blocks: the ucat fragments of a block's panels (loaded by
// every item) and the vcat fragments of a chunk (loaded by the block's
// items in a row) are read from HBM about once and then hit in its L2, and
// the panels that share an axis-0 output line run side by side.
constexpr int kQfPB = 16;

struct QfItem {
  int64_t r0, ct0;
  int n;
};

template <int TPW>
__device__ inline bool qf_item(const QuantParams& p, QfItem& it) {
  const int P = (int)(p.rows / kQT_R), ntc = (int)(p.cols / kQT_C);
  const int C = (ntc + TPW - 1) / TPW;
  const int W = P * C, per = (W + 7) / 8;
  const int id = blockIdx.x;
  const int w = (id & 7) * per + (id >> 3);
  if (w >= W) return false;
  const int b = w / (kQfPB * C), r = w - b * (kQfPB * C);
  const int pb = min(kQfPB, P - b * kQfPB);
  const int c = r / pb;
  it.r0 = (int64_t)(b * kQfPB + (r - c * pb)) * kQT_R;
  it.ct0 = (int64_t)c * TPW;
  it.n = __builtin_amdgcn_readfirstlane(min(ntc, c * TPW + TPW) - c * TPW);
  return true;
}

// s_waitcnt vmcnt(N) (N < 64), other counters untouched.
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// s_waitcnt vmcnt(N) lgkmcnt(0).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
}

// One 64-column tile of this lane's row: the two 16-element blocks at
// columns 16 hh .. and 32 + 16 hh .. (the layout lowrank_subtract leaves).
__device__ __forceinline__ void qf_load(const uint16_t* m, uint4 (&r)[4]) {
  r[0] = *(const uint4*)m;
  r[1] = *(const uint4*)(m + 8);
  r[2] = *(const uint4*)(m + 32);
  r[3] = *(const uint4*)(m + 40);
}

// Shared opening of both sweeps: this lane's row pointer and ucat fragments.
template <int NKK>
struct QfLane {
  int wave, lane, hh;
  int64_t row;
  const uint16_t* mrow;
  half8_t uf[NKK > 0 ? NKK : 1];
  float ps;

  __device__ __forceinline__ void init(const QuantParams& p, const QfItem& it) {
    const int tid = threadIdx.x;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    lane = tid & 63;
    hh = lane >> 5;
    row = it.r0 + wave * 32 + (lane & 31);
    mrow = (const uint16_t*)p.M + row * p.ld + 16 * hh;
    if constexpr (NKK > 0) {
      const int64_t g = (it.r0 >> 5) + wave;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) uf[kk] = *(const half8_t*)(p.ucat + ((g * NKK + kk) * 64 + lane) * 8);
      ps = p.pscale[0];
    } else {
      ps = 0.0f;
    }
  }
};

// DMAs per wave for one tile's vcat fragments (2 NKK 1-KB blocks over four
// waves, rounded up: every wave issues the same number, so the counts of
// outstanding vector-memory operations are the same in every wave and step).
template <int NKK>
constexpr int qf_ndma() {
  return NKK > 0 ? (2 * NKK + 3) / 4 : 0;
}

// The tile's vcat fragments -> buf by LDS-DMA.  A wave whose share is one
// block short repeats its previous block (same data to the same place).
template <int NKK>
__device__ __forceinline__ void qf_dma_bf(const QuantParams& p, int64_t ct, uint4* buf, int wave, int lane) {
  if constexpr (NKK > 0) {
    constexpr int BFU = NKK * 2 * 64;
    const uint4* src = (const uint4*)p.vcat + ct * BFU;
#pragma unroll
    for (int i = 0; i < qf_ndma<NKK>(); ++i) {
      const int j0 = wave + 4 * i;
      const int j = j0 < 2 * NKK ? j0 : j0 - 4;
      dma16(src + j * 64 + lane, (uint8_t*)(buf + j * 64));
    }
  }
}

__device__ __forceinline__ void qf_unpack(const uint4 (&r)[4], float (&x)[2][16]) {
  unpack_bf16x16(r[0], r[1], x[0]);
  unpack_bf16x16(r[2], r[3], x[1]);
}

// Tile t of the item; in a chunk cut short by the operand's edge the steps
// past its end take its last tile again and rewrite the same bytes, so every
// step runs the same instructions and the memory counts stay static.
__device__ __forceinline__ int64_t qf_tile(const QfItem& it, int t) { return it.ct0 + min(t, it.n - 1); }

// LDS address of a shared-memory pointer.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Maximum of v over the wave.  DPP steps within each 16-lane row (swap
// neighbours, swap pairs, mirror the half rows, mirror the rows), then the
// four row results by v_readlane: no LDS instruction, so the compiler does
// not hold it behind LDS-DMAs in flight.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row_mirror
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return max(max(r0, r1), max(r2, r3));
}

// --------------------------------------------------------------- pass 1 --

// Pipeline of both sweeps, per workgroup and tile t = 0 .. TPW - 1 (the rows
// of tile t in register set X[t % 3], its vcat fragments in LDS slot
// B[t % 2], its rank-k MFMA issued during step t - 1):
//   1. unpack X[t % 3]; load tile t+2's rows into X[(t + 2) % 3] (that set
//      held tile t - 1, already unpacked);
//   2. subtract the rank-k product of tile t;
//   3. ring barrier: tile t+1's fragments have landed (issued one step ago)
//      and every wave has read B[t % 2];
//   4. MFMA of tile t+1 from B[(t + 1) % 2]; DMA of tile t+2 into B[t % 2];
//   5. the tile's own work (max, or quantisation and stores).
// Vector-memory operations of a step, in order: 4 row loads (t + 2 < TPW),
// then the DMAs (t + 2 < TPW) and the stores of pass 2.  The barrier's wait
// counts what came after tile t+1's DMAs: the previous step's stores and this
// step's row loads.  The prologue loads the rows of tiles 0 and 1, then
// their fragments.

template <int NKK, int TPW>
__global__ __launch_bounds__(kQThreads) __attribute__((amdgpu_waves_per_eu(2, 4)))
void qf_amax_kernel(QuantParams p) {
  constexpr bool HAS_F = NKK > 0;
  constexpr int BFU = HAS_F ? NKK * 2 * 64 : 1;
  constexpr int ND = qf_ndma<NKK>();
  __shared__ uint4 Bf0[BFU];
  __shared__ uint4 Bf1[BFU];
  QfItem it;
  if (!qf_item<TPW>(p, it)) return;
  QfLane<NKK> L;
  L.init(p, it);
  uint32_t runmax = 0u;  // bits of |x|: non-negative binary32 values order as unsigned integers
  f32x16_t a0, a1;
  uint4 X[3][4];

  qf_load(L.mrow + qf_tile(it, 0) * kQT_C, X[0]);
  if constexpr (TPW > 1) qf_load(L.mrow + qf_tile(it, 1) * kQT_C, X[1]);
  if constexpr (HAS_F) {
    qf_dma_bf<NKK>(p, qf_tile(it, 0), Bf0, L.wave, L.lane);
    if constexpr (TPW > 1) qf_dma_bf<NKK>(p, qf_tile(it, 1), Bf1, L.wave, L.lane);
    wait_vm<(TPW > 1 ? ND : 0)>();  // tile 0's fragments (tile 1's may still be in flight)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    lowrank_mfma<NKK>(Bf0, L.uf, L.lane, a0, a1);
  }

#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    float x[2][16];
    qf_unpack(X[t % 3], x);
    if (t + 2 < TPW) qf_load(L.mrow + qf_tile(it, t + 2) * kQT_C, X[(t + 2) % 3]);
    if constexpr (HAS_F) {
      lowrank_subtract(a0, a1, L.ps, x);
      if (t + 1 < TPW) {
        if (t + 2 < TPW)
          wait_vm<4>();
        else
          wait_vm<0>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        lowrank_mfma<NKK>((t & 1) ? Bf0 : Bf1, L.uf, L.lane, a0, a1);
        if (t + 2 < TPW) qf_dma_bf<NKK>(p, qf_tile(it, t + 2), (t & 1) ? Bf1 : Bf0, L.wave, L.lane);
      }
    }
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const uint32_t u0 = __float_as_uint(x[b][i]) & 0x7FFFFFFFu;
        const uint32_t u1 = __float_as_uint(x[b][i + 1]) & 0x7FFFFFFFu;
        runmax = max(runmax, max(u0, u1));
      }
  }
  // NaN and infinities have the largest magnitude bit patterns
  if (runmax > 0x7F7FFFFFu) raise_status(kStatusNonFinite);
  runmax = wave_max_u32(runmax);
  // one atomic per workgroup, into the slot of its id
  __shared__ uint32_t wmax[kQThreads / 64];
  if (L.lane == 0) wmax[L.wave] = runmax;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = wmax[0];
#pragma unroll
    for (int w = 1; w < kQThreads / 64; ++w) m = max(m, wmax[w]);
    atomicMax(p.amax_slots + kAmaxSlotStride * (blockIdx.x % kAmaxSlots), m);
  }
}

// --------------------------------------------------------------- pass 2 --

// Tensor |max| bits: the maximum over pass 1's slots, read by scalar loads
// that wait for themselves (lgkmcnt).  A vector load here would be waited for
// with vmcnt(0) while LDS-DMAs are in flight (the compiler cannot order it
// against them), stalling on the whole prefetch.
__device__ __forceinline__ uint32_t qf_tensor_amax(const QuantParams& p) {
  static_assert(kAmaxSlots == 16 && kAmaxSlotStride == 32, "16 slots, 128 bytes apart");
  uint32_t v[16];
  asm volatile(
      "s_load_dword %0, %16, 0x0\n\t"
      "s_load_dword %1, %16, 0x80\n\t"
      "s_load_dword %2, %16, 0x100\n\t"
      "s_load_dword %3, %16, 0x180\n\t"
      "s_load_dword %4, %16, 0x200\n\t"
      "s_load_dword %5, %16, 0x280\n\t"
      "s_load_dword %6, %16, 0x300\n\t"
      "s_load_dword %7, %16, 0x380\n\t"
      "s_load_dword %8, %16, 0x400\n\t"
      "s_load_dword %9, %16, 0x480\n\t"
      "s_load_dword %10, %16, 0x500\n\t"
      "s_load_dword %11, %16, 0x580\n\t"
      "s_load_dword %12, %16, 0x600\n\t"
      "s_load_dword %13, %16, 0x680\n\t"
      "s_load_dword %14, %16, 0x700\n\t"
      "s_load_dword %15, %16, 0x780\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&s"(v[0]), "=&s"(v[1]), "=&s"(v[2]), "=&s"(v[3]), "=&s"(v[4]), "=&s"(v[5]), "=&s"(v[6]),
        "=&s"(v[7]), "=&s"(v[8]), "=&s"(v[9]), "=&s"(v[10]), "=&s"(v[11]), "=&s"(v[12]), "=&s"(v[13]),
        "=&s"(v[14]), "=&s"(v[15])
      : "s"(p.amax_slots));
  uint32_t m = v[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) m = max(m, v[i]);
  return m;
}

// Per-tensor reciprocals of the 127 effective block scales:
// inv[b] = RN(1 / RN(E4M3(b) s_g)), inv[0] = 0.
__device__ __forceinline__ void qf_inv_table(float s_g, float* inv) {
  const int t = threadIdx.x;
  if (t < 128) inv[t] = (t == 0 || t == 127) ? 0.0f : __fdiv_rn(1.0f, __fmul_rn(e4m3_decode_hw(t), s_g));
}

// LDS reads the compiler must not order behind the vcat DMAs.  It cannot tell
// these arrays from the DMA ring, so it would wait for every outstanding
// vector-memory operation (the row prefetch among them) before a plain read;
// each block below issues its reads and waits for them itself.
__device__ __forceinline__ void lds_read2(uint32_t a0, uint32_t a1, float& v0, float& v1) {
  asm volatile(
      "ds_read_b32 %0, %2\n\t"
      "ds_read_b32 %1, %3\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v0), "=&v"(v1)
      : "v"(a0), "v"(a1)
      : "memory");
}

// 16 binary32 values at a, a + 144, .., a + 15 * 144 (a column of a slab).
__device__ __forceinline__ void lds_col16_f32(uint32_t a, float (&v)[16]) {
  asm volatile(
      "ds_read_b32 %0, %16\n\t"
      "ds_read_b32 %1, %16 offset:144\n\t"
      "ds_read_b32 %2, %16 offset:288\n\t"
      "ds_read_b32 %3, %16 offset:432\n\t"
      "ds_read_b32 %4, %16 offset:576\n\t"
      "ds_read_b32 %5, %16 offset:720\n\t"
      "ds_read_b32 %6, %16 offset:864\n\t"
      "ds_read_b32 %7, %16 offset:1008\n\t"
      "ds_read_b32 %8, %16 offset:1152\n\t"
      "ds_read_b32 %9, %16 offset:1296\n\t"
      "ds_read_b32 %10, %16 offset:1440\n\t"
      "ds_read_b32 %11, %16 offset:1584\n\t"
      "ds_read_b32 %12, %16 offset:1728\n\t"
      "ds_read_b32 %13, %16 offset:1872\n\t"
      "ds_read_b32 %14, %16 offset:2016\n\t"
      "ds_read_b32 %15, %16 offset:2160\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]),
        "=&v"(v[7]), "=&v"(v[8]), "=&v"(v[9]), "=&v"(v[10]), "=&v"(v[11]), "=&v"(v[12]), "=&v"(v[13]),
        "=&v"(v[14]), "=&v"(v[15])
      : "v"(a)
      : "memory");
}

// 16 halves at a, a + 80, .., a + 15 * 80 (a column of a draw slab).
__device__ __forceinline__ void lds_col16_u16(uint32_t a, uint32_t (&v)[16]) {
  asm volatile(
      "ds_read_u16 %0, %16\n\t"
      "ds_read_u16 %1, %16 offset:80\n\t"
      "ds_read_u16 %2, %16 offset:160\n\t"
      "ds_read_u16 %3, %16 offset:240\n\t"
      "ds_read_u16 %4, %16 offset:320\n\t"
      "ds_read_u16 %5, %16 offset:400\n\t"
      "ds_read_u16 %6, %16 offset:480\n\t"
      "ds_read_u16 %7, %16 offset:560\n\t"
      "ds_read_u16 %8, %16 offset:640\n\t"
      "ds_read_u16 %9, %16 offset:720\n\t"
      "ds_read_u16 %10, %16 offset:800\n\t"
      "ds_read_u16 %11, %16 offset:880\n\t"
      "ds_read_u16 %12, %16 offset:960\n\t"
      "ds_read_u16 %13, %16 offset:1040\n\t"
      "ds_read_u16 %14, %16 offset:1120\n\t"
      "ds_read_u16 %15, %16 offset:1200\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]),
        "=&v"(v[7]), "=&v"(v[8]), "=&v"(v[9]), "=&v"(v[10]), "=&v"(v[11]), "=&v"(v[12]), "=&v"(v[13]),
        "=&v"(v[14]), "=&v"(v[15])
      : "v"(a)
      : "memory");
}

// Scale byte of a 16-block: the division and the E4M3 conversion.
__device__ __forceinline__ uint32_t qf_scale(const float (&x)[16], float d) {
  return e4m3_encode_hw(__fdiv_rn(__uint_as_float(abs_max16_bits(x)), d));
}

// Codes of a 16-block with y = RN(x inv) (quant_block16's definition).
template <bool SR>
__device__ __forceinline__ void qf_codes(const float (&x)[16], const uint32_t* hc, float iv, uint32_t& lo,
                                         uint32_t& hi) {
  float y[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) y[i] = __fmul_rn(x[i], iv);
  if constexpr (SR) {
    lo = e2m1_pack8_sr(y, hc);
    hi = e2m1_pack8_sr(y + 8, hc + 8);
  } else {
    lo = e2m1_pack8_rne(y);
    hi = e2m1_pack8_rne(y + 8);
  }
}

// v_permlane32_swap of the upper half of a with the lower half of b.
__device__ __forceinline__ void swap_halves(uint32_t& a, uint32_t& b) {
  const auto s = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  a = s[0];
  b = s[1];
}

// The axis-1 outputs of a workgroup's TPW tiles for this lane's row: 16 code
// bytes per tile at columns 32 hh .. of the tile, and a scale pair (2 bytes).
// With four whole tiles, lanes l and l + 32 exchange scale pairs so that each
// writes 8 contiguous bytes (l: tiles 0 and 1, l + 32: tiles 2 and 3).
template <int TPW>
__device__ __forceinline__ void qf_store_axis1(const QuantParams& p, const QfItem& it, int64_t row, int hh,
                                               const uint32_t (&o1)[TPW][4], const uint32_t (&s1)[TPW]) {
  uint8_t* crow = p.codes1 + row * (p.cols >> 1);
  uint8_t* srow = p.scales1 + row * (p.cols >> 4);
#pragma unroll
  for (int u = 0; u < TPW; ++u)
    *(uint4*)(crow + qf_tile(it, u) * 32 + 16 * hh) = make_uint4(o1[u][0], o1[u][1], o1[u][2], o1[u][3]);
  if constexpr (TPW == 4) {
    if (it.n == 4) {
      uint32_t a = s1[0] | (s1[1] << 16), b = s1[2] | (s1[3] << 16);
      swap_halves(a, b);  // l: own pairs of tiles 0, 1 in a, l + 32's in b; l + 32: l's pairs of tiles 2, 3 in a, its own in b
      const uint32_t w0 = (a & 0xFFFFu) | (b << 16), w1 = (a >> 16) | (b & 0xFFFF0000u);
      *(uint2*)(srow + it.ct0 * 4 + 8 * hh) = make_uint2(w0, w1);
      return;
    }
  }
#pragma unroll
  for (int u = 0; u < TPW; ++u) *(uint16_t*)(srow + qf_tile(it, u) * 4 + 2 * hh) = (uint16_t)s1[u];
}

constexpr int kQfRP = 36;  // row pitch (floats) of a wave's transpose slab (144 bytes)
constexpr int kQfHP = 40;  // row pitch (halves) of its draw slab (80 bytes)

// AX: bit 0 axis 0 (K = rows), bit 1 axis 1 (K = cols).
template <int NKK, bool SR, int AX, int TPW>
__global__ __launch_bounds__(kQThreads) __attribute__((amdgpu_waves_per_eu(NKK > 0 ? 2 : 3, NKK > 0 ? 2 : 4)))
void qf_quant_kernel(QuantParams p) {
  constexpr bool HAS_F = NKK > 0;
  constexpr int BFU = HAS_F ? NKK * 2 * 64 : 1;
  constexpr bool AX0 = (AX & 1) != 0, AX1 = (AX & 2) != 0;
  // stores of a step before the last (axis 1 writes everything at the end)
  constexpr int NS = AX0 ? 2 : 0;
  __shared__ uint4 Bf0[BFU];
  __shared__ uint4 Bf1[BFU];
  __shared__ __attribute__((aligned(16))) float R[AX0 ? 4 : 1][AX0 ? 32 * kQfRP : 4];
  __shared__ __attribute__((aligned(16))) uint16_t H[AX0 && SR ? 4 : 1][AX0 && SR ? 32 * kQfHP : 8];
  __shared__ float inv[128];
  QfItem it;
  if (!qf_item<TPW>(p, it)) return;
  QfLane<NKK> L;
  L.init(p, it);

  f32x16_t a0, a1;
  uint4 X[3][4];
  qf_load(L.mrow + qf_tile(it, 0) * kQT_C, X[0]);
  if constexpr (TPW > 1) qf_load(L.mrow + qf_tile(it, 1) * kQT_C, X[1]);
  if constexpr (HAS_F) {
    qf_dma_bf<NKK>(p, qf_tile(it, 0), Bf0, L.wave, L.lane);
    if constexpr (TPW > 1) qf_dma_bf<NKK>(p, qf_tile(it, 1), Bf1, L.wave, L.lane);
  }

  float s_g = 1.0f, d = 6.0f;
  {
    const float at = __uint_as_float(qf_tensor_amax(p));
    if (at > 0.0f) {
      s_g = __fdiv_rn(at, 2688.0f);
      d = __fmul_rn(6.0f, s_g);
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      if (p.sg0) p.sg0[0] = s_g;
      if (p.sg1) p.sg1[0] = s_g;
    }
  }
  qf_inv_table(s_g, inv);
  // the inverse table and tile 0's fragments are in place (tile 1's may
  // still be in flight; without factors the row loads stay in flight too)
  wait_vm_lgkm0<!HAS_F ? 63 : (TPW > 1 ? qf_ndma<NKK>() : 0)>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  if constexpr (HAS_F) lowrank_mfma<NKK>(Bf0, L.uf, L.lane, a0, a1);

  const int lr = L.lane & 31;  // row (write) or column (read) of this lane in a slab
  const uint32_t inv_a = lds_addr(inv);
  uint32_t slab_r = 0, hslab_r = 0;
  if constexpr (AX0) {
    slab_r = lds_addr(R[L.wave] + 16 * L.hh * kQfRP + lr);
    if constexpr (SR) hslab_r = lds_addr(H[L.wave] + 16 * L.hh * kQfHP + lr);
  }
  const int64_t rw0 = it.r0 + L.wave * 32;
  const uint64_t rowe = (uint64_t)L.row * (uint64_t)p.cols;
  // axis-1 codes and scale pairs of every step, stored together after the
  // last: a row's 128-byte line of codes then fills at once in L2 instead of
  // 32 bytes per step, which let partly written lines be evicted and written
  // back several times
  uint32_t o1[AX1 ? TPW : 1][4], s1[AX1 ? TPW : 1];

#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int64_t c0 = qf_tile(it, t) * kQT_C;
    float x[2][16];
    qf_unpack(X[t % 3], x);
    if (t + 2 < TPW) qf_load(L.mrow + qf_tile(it, t + 2) * kQT_C, X[(t + 2) % 3]);
    if constexpr (HAS_F) {
      lowrank_subtract(a0, a1, L.ps, x);
      if (t + 1 < TPW) {
        // tile t+1's fragments: after them came the previous step's stores
        // (none before step 1) and this step's row loads
        if (t >= 1) {
          if (t + 2 < TPW)
            wait_vm<NS + 4>();
          else
            wait_vm<NS>();
        } else {
          if (t + 2 < TPW)
            wait_vm<4>();
          else
            wait_vm<0>();
        }
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        lowrank_mfma<NKK>((t & 1) ? Bf0 : Bf1, L.uf, L.lane, a0, a1);
        if (t + 2 < TPW) qf_dma_bf<NKK>(p, qf_tile(it, t + 2), (t & 1) ? Bf1 : Bf0, L.wave, L.lane);
      }
    }

    // draws of this lane's two blocks (row-major positions; both orientations)
    uint32_t hc[2][16];
    if constexpr (SR) {
#pragma unroll
      for (int b = 0; b < 2; ++b) draws16(rowe + (uint64_t)(c0 + 32 * b + 16 * L.hh), p.tag1, p.step, p.seed, hc[b]);
    }

    // ---- axis 1: blocks at columns 16 hh and 32 + 16 hh of this lane's row
    if constexpr (AX1) {
      uint32_t sc0 = qf_scale(x[0], d), sc1 = qf_scale(x[1], d);
      float iv0, iv1;
      lds_read2(inv_a + 4 * sc0, inv_a + 4 * sc1, iv0, iv1);
      uint32_t lo0, hi0, lo1, hi1;
      qf_codes<SR>(x[0], hc[0], iv0, lo0, hi0);
      qf_codes<SR>(x[1], hc[1], iv1, lo1, hi1);
      // lanes l < 32 end with columns 0..31, lanes l + 32 with 32..63
      swap_halves(lo0, lo1);
      swap_halves(hi0, hi1);
      swap_halves(sc0, sc1);
      o1[t][0] = lo0;
      o1[t][1] = hi0;
      o1[t][2] = lo1;
      o1[t][3] = hi1;
      s1[t] = sc0 | (sc1 << 8);
      if (t == TPW - 1) qf_store_axis1<TPW>(p, it, L.row, L.hh, o1, s1);
    }

    // ---- axis 0: per 32-column half, through this wave's slabs; lane
    // (row lr, columns 16 hh ..) writes, lane (column lr, rows 16 hh ..) reads
    if constexpr (AX0) {
      uint32_t lo[2], hi[2], sc[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        float* wr = (float*)(R[L.wave] + lr * kQfRP + 16 * L.hh);
#pragma unroll
        for (int i = 0; i < 16; i += 4) *(float4*)(wr + i) = make_float4(x[b][i], x[b][i + 1], x[b][i + 2], x[b][i + 3]);
        float xc16[16];
        uint32_t hcc[16];
        if constexpr (SR) {
          uint32_t w[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) w[i] = hc[b][2 * i] | (hc[b][2 * i + 1] << 16);
          uint16_t* hw = H[L.wave] + lr * kQfHP + 16 * L.hh;
          *(uint4*)hw = make_uint4(w[0], w[1], w[2], w[3]);
          *(uint4*)(hw + 8) = make_uint4(w[4], w[5], w[6], w[7]);
          lds_col16_u16(hslab_r, hcc);
        }
        lds_col16_f32(slab_r, xc16);
        sc[b] = qf_scale(xc16, d);
        float iv, dummy;
        lds_read2(inv_a + 4 * sc[b], inv_a, iv, dummy);
        qf_codes<SR>(xc16, hcc, iv, lo[b], hi[b]);
      }
      // lane l < 32 ends with rows 0..31 of column lr of the first half
      // (its own block, then that of lane l + 32), lane l + 32 with those of
      // the second half
      swap_halves(lo[0], lo[1]);
      swap_halves(hi[0], hi[1]);
      swap_halves(sc[0], sc[1]);
      const int64_t col = c0 + 32 * L.hh + lr;
      *(uint4*)(p.codes0 + col * (p.rows >> 1) + (rw0 >> 1)) = make_uint4(lo[0], hi[0], lo[1], hi[1]);
      *(uint16_t*)(p.scales0 + col * (p.rows >> 4) + (rw0 >> 4)) = (uint16_t)(sc[0] | (sc[1] << 8));
    }
  }
}

}  // namespace metis
