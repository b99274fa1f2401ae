// rsvd.hpp -- randomized truncated SVD of one operand with the cross-step
// basis cache ("Metis: Training LLMs with FP4 Quantization", 关键设计 2:
// sparse random row sampling + Gaussian random projection; 关键设计 3: reuse
// of the factors; 关键设计 1: M = U_k S_k V_k^T + M_R).
//
// Refresh (every `refresh` steps):
//   idx   = the l_k rows with the smallest (Philox key, row) pairs, ascending
//   Y     = sqrt(r / l_k) M[idx] Omega           (l_k x n, n = k + s)
//   Q     = shifted CholeskyQR3(Y)                (fp64 Gram / Cholesky)
//   B     = Q^T sqrt(r / l_k) M[idx]              (n x cols)
//   Z, T  = Jacobi(B B^T)  (fp64, one workgroup)
//   V     = B^T Z[:, :k] T^-1/2                    (cols x k, the cached basis)
// Every step:
//   P = M V, Jacobi(P^T P) = (R, lambda), V <- V R (sign rule),
//   U = P R lambda^-1/2, S = lambda^1/2.
// Small dense algebra (n <= 96) runs in fp64 inside one workgroup so no
// device-to-host synchronisation is needed anywhere on the path.
#pragma once

#include "common.hpp"
#include "status.hpp"

namespace metis {

constexpr int kMaxN = 96;       // largest sketch width / rank handled in LDS
constexpr int kCandMax = 4096;  // candidate slots of the sampler's boundary bin
constexpr double kEigZero = 1e-12;

// The 65536-entry bf16 Gaussian quantile table (filled from the host once
// per device).
__device__ uint16_t g_omega_table[65536];

// ----------------------------------------------------------------- sampler --

__global__ void sample_keys_kernel(uint32_t* __restrict__ keys, uint32_t* __restrict__ hist,
                                   int64_t rows, uint32_t tag, uint32_t step, uint64_t seed) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows) return;
  const uint32_t k = philox_word((uint64_t)i, tag, step, seed);
  keys[i] = k;
  atomicAdd(&hist[k >> 16], 1u);
}

// meta[0] = boundary bin b*, meta[1] = rows still needed from b*, meta[2] =
// candidate count (zeroed here).
__global__ __launch_bounds__(1024) void sample_threshold_kernel(const uint32_t* __restrict__ hist,
                                                                uint32_t* __restrict__ meta,
                                                                int64_t l_k) {
  __shared__ uint32_t part[1024];
  const int tid = threadIdx.x;
  uint32_t s = 0;
  for (int b = 0; b < 64; ++b) s += hist[tid * 64 + b];
  part[tid] = s;
  __syncthreads();
  // inclusive scan (Hillis-Steele)
  for (int o = 1; o < 1024; o <<= 1) {
    const uint32_t v = tid >= o ? part[tid - o] : 0u;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  const uint32_t incl = part[tid];
  const uint32_t excl = incl - s;
  if (excl < (uint32_t)l_k && (uint32_t)l_k <= incl) {
    uint32_t c = excl;
    for (int b = 0; b < 64; ++b) {
      const uint32_t h = hist[tid * 64 + b];
      if (c + h >= (uint32_t)l_k) {
        meta[0] = (uint32_t)(tid * 64 + b);
        meta[1] = (uint32_t)l_k - c;
        meta[2] = 0;
        break;
      }
      c += h;
    }
  }
}

__global__ void sample_mark_kernel(const uint32_t* __restrict__ keys, uint32_t* __restrict__ meta,
                                   uint8_t* __restrict__ flags, uint2* __restrict__ cand,
                                   int64_t rows) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows) return;
  const uint32_t k = keys[i];
  const uint32_t b = k >> 16, bs = meta[0];
  flags[i] = b < bs ? 1 : 0;
  if (b == bs) {
    const uint32_t slot = atomicAdd(&meta[2], 1u);
    if (slot < (uint32_t)kCandMax)
      cand[slot] = make_uint2(k, (uint32_t)i);
    else
      raise_status(kStatusSample);
  }
}

__global__ __launch_bounds__(1024) void sample_resolve_kernel(const uint32_t* __restrict__ meta,
                                                              const uint2* __restrict__ cand,
                                                              uint8_t* __restrict__ flags) {
  const uint32_t n = min(meta[2], (uint32_t)kCandMax);
  const uint32_t need = meta[1];
  for (uint32_t a = threadIdx.x; a < n; a += blockDim.x) {
    const uint2 ca = cand[a];
    uint32_t rank = 0;
    for (uint32_t b = 0; b < n; ++b) {
      const uint2 cb = cand[b];
      rank += (cb.x < ca.x || (cb.x == ca.x && cb.y < ca.y)) ? 1u : 0u;
    }
    if (rank < need) flags[ca.y] = 1;
  }
}

// idx = ascending list of flagged rows (one workgroup scan over all rows).
__global__ __launch_bounds__(1024) void sample_compact_kernel(const uint8_t* __restrict__ flags,
                                                              int64_t rows, int64_t l_k,
                                                              int32_t* __restrict__ idx) {
  __shared__ uint32_t part[1024];
  const int tid = threadIdx.x;
  const int64_t chunk = ceil_div<int64_t>(rows, 1024);
  const int64_t b = tid * chunk, e = min(rows, b + chunk);
  uint32_t c = 0;
  for (int64_t i = b; i < e; ++i) c += flags[i];
  part[tid] = c;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const uint32_t v = tid >= o ? part[tid - o] : 0u;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  uint32_t pos = part[tid] - c;
  for (int64_t i = b; i < e; ++i)
    if (flags[i]) {
      if ((int64_t)pos < l_k) idx[pos] = (int32_t)i;
      ++pos;
    }
  // fewer flagged rows than l_k (a candidate overflow, reported below): the
  // remaining indices name row 0, so the sketch reads only valid rows
  for (int64_t i = (int64_t)part[1023] + tid; i < l_k; i += 1024) idx[i] = 0;
  if (tid == 1023 && (int64_t)part[1023] != l_k) raise_status(kStatusSample);
}

__global__ void iota_kernel(int32_t* idx, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) idx[i] = (int32_t)i;
}

// ------------------------------------------------------------------ Omega --

__global__ void omega_kernel(float* __restrict__ om, int64_t cols, int n, uint32_t tag,
                             uint32_t step, uint64_t seed) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // block of 8
  const int64_t total = cols * n;
  const int64_t e0 = q * 8;
  if (e0 >= total) return;
  const Philox4 b = philox_block((uint64_t)q, tag, step, seed);
#pragma unroll
  for (int o = 0; o < 8; ++o) {
    const int64_t e = e0 + o;
    if (e < total) {
      const uint32_t h = philox_half_of(b, (uint32_t)o);
      om[e] = __uint_as_float((uint32_t)g_omega_table[h] << 16);
    }
  }
}

// ------------------------------------------------------------ sketch GEMMs --

// Y[s][j] = scale * sum_c M[idx[s]][c] Om[c][j]; 32 sample rows per block.
__global__ __launch_bounds__(256) void sketch_y_kernel(const void* __restrict__ M, int dtype,
                                                       int64_t ld, const int32_t* __restrict__ idx,
                                                       int64_t ns, int64_t cols,
                                                       const float* __restrict__ om, int n,
                                                       float scale, float* __restrict__ Y) {
  __shared__ float ms[32][65];
  __shared__ float os[64][kMaxN + 1];
  const int tid = threadIdx.x;
  const int64_t s0 = (int64_t)blockIdx.x * 32;
  const int sl = tid >> 3, jg = tid & 7;
  float acc[kMaxN / 8];
#pragma unroll
  for (int t = 0; t < kMaxN / 8; ++t) acc[t] = 0.0f;
  for (int64_t c0 = 0; c0 < cols; c0 += 64) {
    for (int e = tid; e < 32 * 64; e += 256) {
      const int r = e >> 6, c = e & 63;
      const int64_t s = s0 + r;
      float v = 0.0f;
      if (s < ns && c0 + c < cols) v = load_as_float(M, dtype, (int64_t)idx[s] * ld + c0 + c);
      ms[r][c] = v;
    }
    for (int e = tid; e < 64 * n; e += 256) {
      const int c = e / n, j = e % n;
      os[c][j] = (c0 + c < cols) ? om[(c0 + c) * n + j] : 0.0f;
    }
    __syncthreads();
    for (int c = 0; c < 64; ++c) {
      const float mv = ms[sl][c];
#pragma unroll
      for (int t = 0; t < kMaxN / 8; ++t) {
        const int j = jg + 8 * t;
        if (j < n) acc[t] = fmaf(mv, os[c][j], acc[t]);
      }
    }
    __syncthreads();
  }
  const int64_t s = s0 + sl;
  if (s < ns)
#pragma unroll
    for (int t = 0; t < kMaxN / 8; ++t) {
      const int j = jg + 8 * t;
      if (j < n) Y[s * n + j] = acc[t] * scale;
    }
}

// Partial B[j][c] over a slice of sample rows: part[slice][j][c] = the sum,
// in sample-row order, of Q[s][j] M[idx[s]][c] (binary32 FMA).  kSkbCols
// columns per block, four consecutive ones per lane, loaded as one 8-byte
// (bf16) or 16-byte (fp32) vector when the rows allow it (vec), so each
// lane keeps four times the bytes in flight and each Q value read from LDS
// feeds four FMAs.  Wave w owns the jw consecutive rows j of B from w jw
// (jw: n / 4 rounded up to a multiple of 4), read from the Q tile in LDS
// four at a time (all lanes read the same address), and the M values of
// eight sample rows are loaded before their FMAs.
constexpr int kSkbCols = 256;
__device__ __forceinline__ void skb_load4(const void* M, int dtype, int64_t base, int64_t c, int64_t cols, bool vec,
                                          float (&v)[4]) {
  if (vec) {
    if (dtype == 0) {
      const uint2 w = *(const uint2*)((const uint16_t*)M + base + c);
      v[0] = __uint_as_float(w.x << 16);
      v[1] = __uint_as_float(w.x & 0xFFFF0000u);
      v[2] = __uint_as_float(w.y << 16);
      v[3] = __uint_as_float(w.y & 0xFFFF0000u);
    } else {
      const float4 f = *(const float4*)((const float*)M + base + c);
      v[0] = f.x;
      v[1] = f.y;
      v[2] = f.z;
      v[3] = f.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = load_as_float(M, dtype, base + min(c + e, cols - 1));
  }
}

__global__ __launch_bounds__(256) void sketch_b_kernel(const void* __restrict__ M, int dtype,
                                                       int64_t ld, const int32_t* __restrict__ idx,
                                                       int64_t ns, int64_t cols,
                                                       const float* __restrict__ Q, int n,
                                                       int64_t rows_per_slice,
                                                       float* __restrict__ part) {
  constexpr int QP = kMaxN;  // Q tile pitch in floats (16-byte rows)
  static_assert(QP % 4 == 0, "Q tile pitch");
  __shared__ __attribute__((aligned(16))) float qs[64][QP];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int jw = ((n + 3) / 4 + 3) & ~3;
  const int j0 = wave * jw;
  const int64_t c = (int64_t)blockIdx.x * kSkbCols + 4 * lane;  // first of this lane's four columns
  // whole, aligned four-column vectors inside the row (dtype 0: bf16, 8 bytes)
  const bool vec = (ld % 4 == 0) && (((uintptr_t)M & (dtype == 0 ? 7 : 15)) == 0) && c + 3 < cols;
  const int64_t cl = c < cols ? c : cols - 1;
  const int64_t sb = (int64_t)blockIdx.y * rows_per_slice;
  const int64_t se = min(ns, sb + rows_per_slice);
  float acc[4][kMaxN / 4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int t = 0; t < kMaxN / 4; ++t) acc[e][t] = 0.0f;
  for (int64_t s0 = sb; s0 < se; s0 += 64) {
    __syncthreads();
    for (int e = tid; e < 64 * QP; e += 256) {
      const int r = e / QP, j = e - r * QP;
      qs[r][j] = (j < n && s0 + r < se) ? Q[(s0 + r) * n + j] : 0.0f;
    }
    __syncthreads();
    const int lim = (int)min((int64_t)64, se - s0);
    for (int r0 = 0; r0 < lim; r0 += 8) {
      float mv[8][4];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (r0 + u < lim) {
          skb_load4(M, dtype, (int64_t)idx[s0 + r0 + u] * ld, cl, cols, vec, mv[u]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) mv[u][e] = 0.0f;
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (r0 + u >= lim) break;
        const float4* q4 = (const float4*)&qs[r0 + u][j0];
#pragma unroll
        for (int t4 = 0; t4 < kMaxN / 16; ++t4) {
          if (4 * t4 < jw) {
            const float4 q = q4[t4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              acc[e][4 * t4 + 0] = fmaf(q.x, mv[u][e], acc[e][4 * t4 + 0]);
              acc[e][4 * t4 + 1] = fmaf(q.y, mv[u][e], acc[e][4 * t4 + 1]);
              acc[e][4 * t4 + 2] = fmaf(q.z, mv[u][e], acc[e][4 * t4 + 2]);
              acc[e][4 * t4 + 3] = fmaf(q.w, mv[u][e], acc[e][4 * t4 + 3]);
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kMaxN / 4; ++t) {
    const int j = j0 + t;
    if (t < jw && j < n) {
      float* const prow = part + ((int64_t)blockIdx.y * n + j) * cols;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (c + e < cols) prow[c + e] = acc[e][t];
    }
  }
}

// B[j][c] = scale * sum over slices (fixed order -> deterministic).
__global__ void reduce_slices_kernel(const float* __restrict__ part, int slices, int64_t count,
                                     float scale, float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  float s = 0.0f;
  for (int k = 0; k < slices; ++k) s += part[(int64_t)k * count + i];
  out[i] = s * scale;
}

// --------------------------------------------------------------- fp64 Grams --

// Partial Gram of an nr x n matrix X (element (r, j) at X[r*rs + j*cs]),
// n <= 16 T: part[block][a][b] = sum over this block's rows (in row order)
// of X[r][a] X[r][b], in fp64 (each product of two binary32 values is exact).
// Thread (ti, tj) of a 16 x 16 grid owns entries a = ti + 16 u, b = tj + 16 v.
template <int T>
__global__ __launch_bounds__(256) void gram_partial_kernel(const float* __restrict__ X, int64_t nr, int n,
                                                           int64_t rs, int64_t cs, int64_t rows_per_block,
                                                           double* __restrict__ part) {
  constexpr int W = 16 * T;
  __shared__ float xs[32][W + 1];
  const int tid = threadIdx.x;
  const int ti = tid & 15, tj = tid >> 4;
  const int64_t rb = (int64_t)blockIdx.x * rows_per_block;
  const int64_t re = min(nr, rb + rows_per_block);
  double acc[T][T];
#pragma unroll
  for (int u = 0; u < T; ++u)
#pragma unroll
    for (int v = 0; v < T; ++v) acc[u][v] = 0.0;
  for (int64_t r0 = rb; r0 < re; r0 += 32) {
    __syncthreads();
    if (cs == 1) {  // rows contiguous: walk the columns fastest
      for (int e = tid; e < 32 * n; e += 256) {
        const int r = e / n, j = e - r * n;
        xs[r][j] = (r0 + r < re) ? X[(r0 + r) * rs + j] : 0.0f;
      }
    } else {        // columns contiguous: walk the rows fastest
      for (int e = tid; e < 32 * n; e += 256) {
        const int r = e & 31, j = e >> 5;
        xs[r][j] = (r0 + r < re) ? X[(r0 + r) * rs + (int64_t)j * cs] : 0.0f;
      }
    }
    __syncthreads();
#pragma unroll 4
    for (int r = 0; r < 32; ++r) {
      double xa[T], xb[T];
#pragma unroll
      for (int u = 0; u < T; ++u) xa[u] = (double)xs[r][ti + 16 * u];
#pragma unroll
      for (int v = 0; v < T; ++v) xb[v] = (double)xs[r][tj + 16 * v];
#pragma unroll
      for (int u = 0; u < T; ++u)
#pragma unroll
        for (int v = 0; v < T; ++v) acc[u][v] += xa[u] * xb[v];
    }
  }
  const int nn = n * n;
#pragma unroll
  for (int u = 0; u < T; ++u)
#pragma unroll
    for (int v = 0; v < T; ++v) {
      const int a = ti + 16 * u, b = tj + 16 * v;
      if (a < n && b < n) part[(int64_t)blockIdx.x * nn + a * n + b] = acc[u][v];
    }
}

// The projection's split reduction fused with the Gram partials: rows
// [rb, re) of P = scale * sum_s part[s][r][j] (j < n; the splits added in
// order from zero, then scaled, as project_reduce_kernel does) are written
// to P and, 32 rows at a time, accumulated as gram_partial_kernel does
// (same thread ownership, same row order), so P and the partials are the
// same bits as the two kernels in sequence.  The next 32 rows' split sums
// are formed in registers while the current rows are accumulated.
template <int T>
__global__ __launch_bounds__(256) void gram_rows_kernel(const float* __restrict__ part, int64_t splits, int pw,
                                                        float scale, float* __restrict__ P, int64_t nr, int n,
                                                        int64_t rows_per_block, double* __restrict__ gpart) {
  constexpr int W = 16 * T;
  constexpr int PER = (32 * W + 255) / 256;  // row-chunk elements per thread
  __shared__ float xs[2][32][W + 1];
  const int tid = threadIdx.x;
  const int ti = tid & 15, tj = tid >> 4;
  const int64_t rb = (int64_t)blockIdx.x * rows_per_block;
  const int64_t re = min(nr, rb + rows_per_block);
  double acc[T][T];
#pragma unroll
  for (int u = 0; u < T; ++u)
#pragma unroll
    for (int v = 0; v < T; ++v) acc[u][v] = 0.0;
  float val[PER];
  // The split loop is outermost so that a thread's PER loads of one split
  // (two splits per iteration) are in flight together; each element still
  // adds its splits in order from zero.
  auto fetch = [&](int64_t r0) {
    int64_t off[PER];
    bool ok[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid + 256 * u;
      const int r = e / n, j = e - r * n;
      ok[u] = e < 32 * n && r0 + r < re;
      off[u] = ok[u] ? (r0 + r) * pw + j : 0;
      val[u] = 0.0f;
    }
    const int64_t sstride = nr * pw;
#pragma unroll 2
    for (int64_t sp = 0; sp < splits; ++sp) {
      const float* src = part + sp * sstride;
      float x[PER];
#pragma unroll
      for (int u = 0; u < PER; ++u) x[u] = src[off[u]];  // off = 0 (in bounds) where !ok
#pragma unroll
      for (int u = 0; u < PER; ++u)
        if (ok[u]) val[u] += x[u];
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      if (ok[u]) {
        const int e = tid + 256 * u;
        const int r = e / n, j = e - r * n;
        val[u] = val[u] * scale;
        P[(r0 + r) * n + j] = val[u];
      }
    }
  };
  auto stash = [&](int b) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid + 256 * u;
      if (e < 32 * n) {
        const int r = e / n, j = e - r * n;
        xs[b][r][j] = val[u];
      }
    }
  };
  if (rb < re) {
    fetch(rb);
    stash(0);
  }
  __syncthreads();
  int b = 0;
  for (int64_t r0 = rb; r0 < re; r0 += 32) {
    const bool more = r0 + 32 < re;
    if (more) fetch(r0 + 32);
#pragma unroll 4
    for (int r = 0; r < 32; ++r) {
      double xa[T], xb[T];
#pragma unroll
      for (int u = 0; u < T; ++u) xa[u] = (double)xs[b][r][ti + 16 * u];
#pragma unroll
      for (int v = 0; v < T; ++v) xb[v] = (double)xs[b][r][tj + 16 * v];
#pragma unroll
      for (int u = 0; u < T; ++u)
#pragma unroll
        for (int v = 0; v < T; ++v) acc[u][v] += xa[u] * xb[v];
    }
    if (more) stash(b ^ 1);
    __syncthreads();
    b ^= 1;
  }
  const int nn = n * n;
#pragma unroll
  for (int u = 0; u < T; ++u)
#pragma unroll
    for (int v = 0; v < T; ++v) {
      const int a = ti + 16 * u, c = tj + 16 * v;
      if (a < n && c < n) gpart[(int64_t)blockIdx.x * nn + a * n + c] = acc[u][v];
    }
}

// G[e] = sum of the blocks' partials, in a fixed order: 64 entries per
// workgroup, wave q adds the partials b = q, q + 4, ... in order, then the
// four sums are added pairwise.  A lane fetches 32 of its partials before
// adding them (the additions keep their order), so a wave pays one memory
// round trip per 32 partials rather than one per partial.
__global__ __launch_bounds__(256) void reduce_gram_kernel(const double* __restrict__ part, int blocks, int nn,
                                                          double* __restrict__ G) {
  constexpr int kBatch = 32;
  __shared__ double red[4][64];
  const int el = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + el;
  double s = 0.0;
  if (e < nn)
    for (int b0 = q; b0 < blocks; b0 += 4 * kBatch) {
      double v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int b = b0 + 4 * u;
        v[u] = b < blocks ? part[(int64_t)b * nn + e] : 0.0;
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (b0 + 4 * u < blocks) s += v[u];
    }
  red[q][el] = s;
  __syncthreads();
  if (q == 0 && e < nn) G[e] = (red[0][el] + red[1][el]) + (red[2][el] + red[3][el]);
}

// ------------------------------------------------------ Cholesky (one WG) --

// Rinv = R^-1 with R^T R = G + shift I.  pass 0: shift = c u32 tr(G);
// passes 1, 2: no shift unless the factorisation breaks down, then the
// guard shift c u64 tr(G).  c = 11 (p n + n (n + 1)).
// Right-looking Cholesky (column j: pivot square root, column scaling,
// rank-1 update of the trailing lower triangle, all threads sharing each
// phase), then X = L^-1 by right-looking forward elimination of L X = I.
// LDS holds L and X at NM x (NM + 1) doubles (n <= NM).
template <int NM>
__global__ __launch_bounds__(256) void cholinv_kernel(const double* __restrict__ G, int n,
                                                      int64_t p, int pass,
                                                      double* __restrict__ Rinv) {
  __shared__ double L[NM][NM + 1];
  __shared__ double X[NM][NM + 1];
  __shared__ double red[4];
  __shared__ int fail;
  const int tid = threadIdx.x;
  double t = 0.0;
  for (int i = tid; i < n; i += 256) t += G[i * n + i];
  t = wave_sum_d(t);
  if ((tid & 63) == 0) red[tid >> 6] = t;
  __syncthreads();
  const double tr = red[0] + red[1] + red[2] + red[3];
  const double c = 11.0 * ((double)p * n + (double)n * (n + 1));
  const int attempts = pass == 0 ? 1 : 2;
  for (int att = 0; att < attempts; ++att) {
    double shift = 0.0;
    if (pass == 0) shift = c * ldexp(1.0, -24) * tr;
    else if (att == 1) shift = c * ldexp(1.0, -53) * tr;
    __syncthreads();
    for (int e = tid; e < n * n; e += 256) {
      const int a = e / n, b = e - a * n;
      L[a][b] = G[e] + (a == b ? shift : 0.0);
    }
    if (tid == 0) fail = 0;
    __syncthreads();
    for (int j = 0; j < n; ++j) {
      // pivot (every thread reads it; thread 0 records a breakdown)
      double d = L[j][j];
      if (!(d > 0.0)) {
        if (tid == 0) fail = 1;
        d = 1.0;
      }
      const double piv = sqrt(d);
      // column j below the pivot
      for (int i = j + 1 + tid; i < n; i += 256) L[i][j] /= piv;
      __syncthreads();
      if (tid == 0) L[j][j] = piv;
      // trailing lower triangle: L[i][k] -= L[i][j] L[k][j], j < k <= i;
      // thread (tid / 16, tid % 16) strides rows and columns by 16
      for (int i = j + 1 + (tid >> 4); i < n; i += 16) {
        const double lij = L[i][j];
        for (int k = j + 1 + (tid & 15); k <= i; k += 16) L[i][k] -= lij * L[k][j];
      }
      __syncthreads();
    }
    if (!fail) break;
  }
  if (fail && tid == 0) raise_status(kStatusCholesky);
  // X = L^-1: start from I, eliminate column by column
  for (int e = tid; e < n * n; e += 256) {
    const int a = e / n, b = e - a * n;
    X[a][b] = a == b ? 1.0 : 0.0;
  }
  __syncthreads();
  for (int k = 0; k < n; ++k) {
    // row k: X[k][:] /= L[k][k] (only columns <= k are nonzero)
    for (int b = tid; b <= k; b += 256) X[k][b] /= L[k][k];
    __syncthreads();
    // rows below: X[i][b] -= L[i][k] X[k][b], thread (tid / 16, tid % 16)
    // striding rows and columns by 16
    for (int i = k + 1 + (tid >> 4); i < n; i += 16) {
      const double lik = L[i][k];
      for (int b = tid & 15; b <= k; b += 16) X[i][b] -= lik * X[k][b];
    }
    __syncthreads();
  }
  // R^-1 = (L^-1)^T
  for (int e = tid; e < n * n; e += 256) {
    const int a = e / n, b = e - a * n;
    Rinv[e] = X[b][a];
  }
}

// Qout[s] = Y[s] Rinv (fp64 accumulation over a = 0 .. j in order),
// kApplyRows rows per block (n <= NM); the block's rows of Y are staged in
// LDS next to Rinv, so the inner products read only LDS.
constexpr int kApplyRows = 16;
template <int NM>
__global__ __launch_bounds__(256) void apply_rinv_kernel(const float* __restrict__ Y, int64_t ns,
                                                         int n, const double* __restrict__ Rinv,
                                                         float* __restrict__ Qout) {
  __shared__ double ri[NM][NM + 1];
  __shared__ float ys[kApplyRows][NM + 1];
  const int tid = threadIdx.x;
  const int64_t s0 = (int64_t)blockIdx.x * kApplyRows;
  for (int e = tid; e < n * n; e += blockDim.x) ri[e / n][e % n] = Rinv[e];
  for (int e = tid; e < kApplyRows * n; e += blockDim.x) {
    const int r = e / n, a = e - r * n;
    ys[r][a] = s0 + r < ns ? Y[(s0 + r) * n + a] : 0.0f;
  }
  __syncthreads();
  for (int e = tid; e < kApplyRows * n; e += blockDim.x) {
    const int r = e / n, j = e - r * n;
    const int64_t s = s0 + r;
    if (s >= ns) continue;
    double acc = 0.0;
    for (int a = 0; a <= j; ++a) acc += (double)ys[r][a] * ri[a][j];
    Qout[s * n + j] = (float)acc;
  }
}

// --------------------------------------------------------- Jacobi (one WG) --

// Pair kp of round r in the circle method over np players (np even; player
// np-1 stays, the others rotate), as (p, q) with p < q.
__device__ __forceinline__ int jacobi_pair(int kp, int r, int np) {
  const int m = np - 1;
  int a, b;
  if (kp == 0) {
    a = m;
    b = r;
  } else {
    a = r + kp;
    if (a >= m) a -= m;
    b = r - kp;
    if (b < 0) b += m;
  }
  return min(a, b) | (max(a, b) << 8);
}

// 1 / x and 1 / sqrt(x) (x > 0, normal) from the hardware estimates with one
// Newton step each: a few units in the last place, enough for rotations
// (the rotation below stays orthogonal to that accuracy) and far shorter
// than the correctly rounded division, square root and hypot, which made
// the rotation the latency of every Jacobi round.
__device__ __forceinline__ double rcp_nr(double x) {
  const double r = __builtin_amdgcn_rcp(x);
  return fma(r, fma(-x, r, 1.0), r);
}
__device__ __forceinline__ double rsq_nr(double x) {
  const double y = __builtin_amdgcn_rsq(x);
  const double e = fma(-x * y, y, 1.0);  // 1 - x y^2
  return fma(0.5 * y, e, y);
}

// Symmetric 2x2 Schur rotation (Golub & Van Loan, section 8.5) that zeroes
// a_pq: [c s; -s c]^T [app apq; apq aqq] [c s; -s c] is diagonal, with
// tau = (aqq - app) / (2 apq), t = sign(tau) / (|tau| + sqrt(1 + tau^2)),
// c = 1 / sqrt(1 + t^2), s = t c.
__device__ __forceinline__ void jacobi_rot(double app, double aqq, double apq, double& c, double& s) {
  c = 1.0;
  s = 0.0;
  if (apq == 0.0) return;
  const double tau = (aqq - app) * rcp_nr(2.0 * apq);
  const double at = fabs(tau);
  double t;
  if (at > 1e150) {
    t = 0.5 * rcp_nr(tau);  // tau^2 would overflow: t -> 1 / (2 tau)
  } else {
    const double q = fma(tau, tau, 1.0);
    const double h = q * rsq_nr(q);  // sqrt(1 + tau^2)
    t = copysign(rcp_nr(at + h), tau);
  }
  c = rsq_nr(fma(t, t, 1.0));
  s = t * c;
}

// Cyclic Jacobi with the symmetric Schur rotation in the parallel circle
// order; stops when off(A) <= 1e-12 ||A||_F (or 30 sweeps).  By Weyl's
// bound the diagonal is then within 1e-12 ||A||_F of the eigenvalues, which
// for the Gram matrices here (||A||_F <= 1e5 lambda_min / 1e-7 or so) keeps
// the singular values to ~1e-6 relative; the last, quadratically converging
// sweep to 1e-15 would only refine rounding.  Output:
// eigenvalues descending (ties by index) and eigenvectors (column-major in
// Z: Z[a * n + i] = component a of vector i) signed so the largest-magnitude
// component is positive (lowest index on ties).
//
// One round applies its np/2 disjoint rotations as J^T A J on 2x2 blocks:
// block (P, Q), P <= Q, of pairs P and Q is owned by one thread for the
// whole run.  A is kept as its upper triangle (entry (r, c) at
// A[min][max]); the eigenvector matrix is kept transposed (VT[p][i] =
// V[i][p]) so the column updates read consecutive addresses.  After the
// blocks, wave 0 forms the next round's rotations while the other waves
// apply this round's to V: two barriers per round.  clear (n words, may be
// null) is zeroed for the caller's next kernel.
template <int NM>
__global__ __launch_bounds__(1024) void jacobi_kernel(const double* __restrict__ Ain, int n,
                                                      double* __restrict__ w_out,
                                                      double* __restrict__ Z,
                                                      unsigned long long* __restrict__ clear) {
  static_assert(NM % 2 == 0 && NM <= kMaxN, "even, at most kMaxN");
  constexpr int kHalf = NM / 2;
  constexpr int kBlk = kHalf * (kHalf + 1) / 2;
  constexpr int kPer = (kBlk + 1023) / 1024;  // blocks per thread
  __shared__ double A[NM][NM + 1];
  __shared__ double VT[NM][NM + 1];
  __shared__ double2 rot[2][kHalf];  // (c, s) of pair P
  __shared__ int2 rpq[2][kHalf];     // (p, q), p < q
  __shared__ double red[16];
  __shared__ int go;
  const int tid = threadIdx.x;
  const int np = (n + 1) & ~1;  // even, padded with a zero row/column
  const int half = np / 2;
  const int nblk = half * (half + 1) / 2;
  if (clear && tid < n) clear[tid] = 0ull;
  for (int e = tid; e < np * np; e += 1024) {
    const int a = e / np, b = e % np;
    if (a <= b) A[a][b] = (a < n && b < n) ? 0.5 * (Ain[a * n + b] + Ain[b * n + a]) : 0.0;
    VT[a][b] = (a == b) ? 1.0 : 0.0;
  }
  // this thread's blocks (P, Q): the e-th pair with P <= Q in row order
  int bP[kPer], bQ[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    int rem = tid + 1024 * u, P = 0;
    while (P < half && rem >= half - P) {
      rem -= half - P;
      ++P;
    }
    bP[u] = P;
    bQ[u] = P + rem;
  }
  __syncthreads();
  double loc = 0.0;
  for (int e = tid; e < np * np; e += 1024) {
    const int a = e / np, b = e % np;
    if (a <= b) {
      const double v = A[a][b];
      loc += (a == b ? 1.0 : 2.0) * v * v;
    }
  }
  loc = wave_sum_d(loc);
  if ((tid & 63) == 0) red[tid >> 6] = loc;
  if (tid < half) {
    const int pr = jacobi_pair(tid, 0, np);
    const int p = pr & 255, q = pr >> 8;
    double c, sn;
    jacobi_rot(A[p][p], A[q][q], A[p][q], c, sn);
    rpq[0][tid] = make_int2(p, q);
    rot[0][tid] = make_double2(c, sn);
  }
  __syncthreads();
  double norm2 = 0.0;
  for (int i = 0; i < 16; ++i) norm2 += red[i];
  const double tol2 = 1e-24 * norm2;
  // V update by waves 1..15: slot e = tid - 64 + 960 j is (pair e / np, row
  // e % np), lanes over consecutive rows
  constexpr int kVPer = (kHalf * NM + 959) / 960;
  int vk[kVPer], vi[kVPer];
#pragma unroll
  for (int j = 0; j < kVPer; ++j) {
    const int e = tid - 64 + 960 * j;
    vk[j] = e >= 0 && e < half * np ? e / np : -1;
    vi[j] = e >= 0 && e < half * np ? e - (e / np) * np : 0;
  }
  int par = 0;
  for (int sweep = 0; sweep < 30; ++sweep) {
    double o = 0.0;
    for (int e = tid; e < np * np; e += 1024) {
      const int a = e / np, b = e % np;
      if (a < b) o += 2.0 * A[a][b] * A[a][b];
    }
    o = wave_sum_d(o);
    __syncthreads();
    if ((tid & 63) == 0) red[tid >> 6] = o;
    __syncthreads();
    if (tid == 0) {
      double off2 = 0.0;
      for (int i = 0; i < 16; ++i) off2 += red[i];
      go = off2 > tol2;
    }
    __syncthreads();
    if (!go) break;
    for (int round = 0; round < np - 1; ++round) {
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        if (tid + 1024 * u >= nblk) break;
        const int P = bP[u], Q = bQ[u];
        const int2 r1 = rpq[par][P], r2 = rpq[par][Q];
        const double2 g1 = rot[par][P], g2 = rot[par][Q];
        const int p1 = r1.x, q1 = r1.y, p2 = r2.x, q2 = r2.y;
        const double c1 = g1.x, s1 = g1.y, c2 = g2.x, s2 = g2.y;
        // rows {p1, q1} x columns {p2, q2}, each at its upper-triangle place
        // (in a diagonal block, P == Q, entry (q, p) is entry (p, q): it is
        // read twice and written twice, the later value being the same
        // quantity up to rounding, and near zero)
        double* const ea = p1 < p2 ? &A[p1][p2] : &A[p2][p1];
        double* const eb = p1 < q2 ? &A[p1][q2] : &A[q2][p1];
        double* const ec = q1 < p2 ? &A[q1][p2] : &A[p2][q1];
        double* const ed = q1 < q2 ? &A[q1][q2] : &A[q2][q1];
        const double a = *ea, b = *eb, c = *ec, d = *ed;
        // rows (J^T from the left), then columns (J from the right)
        const double ra = c1 * a - s1 * c, rc = s1 * a + c1 * c;
        const double rb = c1 * b - s1 * d, rd = s1 * b + c1 * d;
        *ea = c2 * ra - s2 * rb;
        *eb = s2 * ra + c2 * rb;
        *ec = c2 * rc - s2 * rd;
        *ed = s2 * rc + c2 * rd;
      }
      __syncthreads();
      if (tid < 64) {
        if (tid < half) {
          const int nr = round + 1 < np - 1 ? round + 1 : 0;
          const int pr = jacobi_pair(tid, nr, np);
          const int p = pr & 255, q = pr >> 8;
          double c, sn;
          jacobi_rot(A[p][p], A[q][q], A[p][q], c, sn);
          rpq[par ^ 1][tid] = make_int2(p, q);
          rot[par ^ 1][tid] = make_double2(c, sn);
        }
      } else {
#pragma unroll
        for (int j = 0; j < kVPer; ++j) {
          if (vk[j] < 0) break;
          const int2 r = rpq[par][vk[j]];
          const double2 g = rot[par][vk[j]];
          const int i = vi[j];
          const double vp = VT[r.x][i], vq = VT[r.y][i];
          VT[r.x][i] = g.x * vp - g.y * vq;
          VT[r.y][i] = g.y * vp + g.x * vq;
        }
      }
      __syncthreads();
      par ^= 1;
    }
  }
  __syncthreads();
  // sort (descending, ties by index) and sign
  for (int i = tid; i < n; i += blockDim.x) {
    const double wi = A[i][i];
    int rank = 0;
    for (int j = 0; j < n; ++j) {
      const double wj = A[j][j];
      rank += (wj > wi || (wj == wi && j < i)) ? 1 : 0;
    }
    int am = 0;
    double best = -1.0;
    for (int a = 0; a < n; ++a) {
      const double v = fabs(VT[i][a]);
      if (v > best) {
        best = v;
        am = a;
      }
    }
    const double sg = VT[i][am] < 0.0 ? -1.0 : 1.0;
    w_out[rank] = wi;
    for (int a = 0; a < n; ++a) Z[a * n + rank] = sg * VT[i][a];
  }
}

// V[c][i] = sum_p B[p][c] Z[p][i] / sqrt(theta_i) for i < k; zero columns
// with theta_i <= 1e-12 theta_0.
__global__ void sketch_v_kernel(const float* __restrict__ B, int64_t cols, int n, int k,
                                const double* __restrict__ Z, const double* __restrict__ theta,
                                float* __restrict__ V) {
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= cols * k) return;
  const int64_t c = id / k;
  const int i = (int)(id % k);
  const double t0 = theta[0], ti = theta[i];
  float out = 0.0f;
  if (t0 > 0.0 && ti > kEigZero * t0) {
    double s = 0.0;
    for (int p = 0; p < n; ++p) s += (double)B[(int64_t)p * cols + c] * Z[p * n + i];
    out = (float)(s / sqrt(ti));
  }
  V[c * k + i] = out;
}

// ------------------------------------------------- projection and rediag --

// P[i][j] = sum_c M[i][c] V[c][j]; 64 rows per block, fp32 accumulation.
__global__ __launch_bounds__(256) void project_kernel(const void* __restrict__ M, int dtype,
                                                      int64_t ld, int64_t rows, int64_t cols,
                                                      const float* __restrict__ V, int k,
                                                      float* __restrict__ P) {
  __shared__ float ms[64][65];
  __shared__ float vs[64][kMaxN + 1];
  const int tid = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.x * 64;
  const int rl = tid >> 2, jg = tid & 3;
  float acc[kMaxN / 4];
#pragma unroll
  for (int t = 0; t < kMaxN / 4; ++t) acc[t] = 0.0f;
  for (int64_t c0 = 0; c0 < cols; c0 += 64) {
    __syncthreads();
    for (int e = tid; e < 64 * 64; e += 256) {
      const int r = e >> 6, c = e & 63;
      float v = 0.0f;
      if (r0 + r < rows && c0 + c < cols) v = load_as_float(M, dtype, (r0 + r) * ld + c0 + c);
      ms[r][c] = v;
    }
    for (int e = tid; e < 64 * k; e += 256) {
      const int c = e / k, j = e % k;
      vs[c][j] = (c0 + c < cols) ? V[(c0 + c) * k + j] : 0.0f;
    }
    __syncthreads();
    for (int c = 0; c < 64; ++c) {
      const float mv = ms[rl][c];
#pragma unroll
      for (int t = 0; t < kMaxN / 4; ++t) {
        const int j = jg + 4 * t;
        if (j < k) acc[t] = fmaf(mv, vs[c][j], acc[t]);
      }
    }
  }
  const int64_t r = r0 + rl;
  if (r < rows)
#pragma unroll
    for (int t = 0; t < kMaxN / 4; ++t) {
      const int j = jg + 4 * t;
      if (j < k) P[r * k + j] = acc[t];
    }
}

// ------------------------------------------- MFMA projection P = M V (bf16 M)
//
// M is exact in bf16; V (binary32) is carried as three bf16 terms
// v = t0 + t1 + t2 (+ O(2^-24 |v|)), so P = sum_t M T_t is the fp32-accurate
// product on bf16 MFMA with fp32 accumulation.  The reduction axis (cols of
// M) is walked in blocks of 64; inside a block, lane half h of a wave owns K
// indices 32h + 8j + i (j = MFMA step 0..3, i = 0..7) for both operands, so
// each lane reads 64 contiguous bytes of its row of M.  V's fragments are
// pre-arranged in exactly the order the waves read them from LDS.

// uint4 slots of one K block of B fragments: NTERM terms x NSUB 32-column
// tiles x 4 MFMA steps x 64 lanes.
template <int NTERM, int NSUB>
constexpr int proj_frag_u4() { return NTERM * NSUB * 4 * 64; }

// B (K x width, binary32, row-major with leading dimension ldb) as NTERM bf16
// terms in fragment order: bfrag[((kb*NTERM + t)*NSUB + n)*4 + j][lane] (uint4
// of 8 bf16) holds column n*32 + lane%32 at K = kb*64 + 32*(lane/32) + 8*j + i.
template <int NTERM, int NSUB>
__global__ void proj_prep_kernel(const float* __restrict__ B, int64_t K, int width, int64_t ldb,
                                 int64_t nkb, uint16_t* __restrict__ bfrag) {
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // one element
  const int64_t total = nkb * NSUB * 4 * 64 * 8;
  if (id >= total) return;
  const int i = (int)(id & 7);
  const int lane = (int)((id >> 3) & 63);
  const int j = (int)((id >> 9) & 3);
  const int64_t rest = id >> 11;
  const int n = (int)(rest % NSUB);
  const int64_t kb = rest / NSUB;
  const int col = n * 32 + (lane & 31);
  const int64_t kk = kb * 64 + 32 * (lane >> 5) + 8 * j + i;
  float v = (col < width && kk < K) ? B[kk * ldb + col] : 0.0f;
#pragma unroll
  for (int t = 0; t < NTERM; ++t) {
    const __bf16 b = (__bf16)v;
    v = v - (float)b;
    const int64_t slot = (((kb * NTERM + t) * NSUB + n) * 4 + j) * 64 + lane;
    bfrag[slot * 8 + i] = __builtin_bit_cast(uint16_t, b);
  }
}

// part[s][r][NSUB*32] = sum over the K blocks of split s of A[src(r)] B, with
// src(r) = idx[r] (gathered rows) or r; A is bf16 with leading dimension ld.
// 128 output rows per workgroup, one 32-row slab per wave.  The K blocks are
// software-pipelined: while block kb is multiplied, block kb+1's B fragments
// land in the other LDS buffer by LDS-DMA and its A rows in registers.  The
// two buffers are distinct arrays and the loop is unrolled by two, so every
// LDS access names its buffer statically.
template <int NTERM, int NSUB>
__global__ __launch_bounds__(256) void project_mfma_kernel(const uint16_t* __restrict__ A, int64_t ld,
                                                           int64_t rows, const int32_t* __restrict__ idx,
                                                           const uint16_t* __restrict__ bfrag,
                                                           int64_t nkb, int64_t kb_per_split,
                                                           float* __restrict__ part) {
  constexpr int FU = proj_frag_u4<NTERM, NSUB>();
  __shared__ uint4 vs0[FU];
  __shared__ uint4 vs1[FU];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t r0 = (int64_t)blockIdx.x * 128;
  const int64_t s = blockIdx.y;
  const int64_t kb0 = s * kb_per_split;
  const int64_t kb1 = min(nkb, kb0 + kb_per_split);
  const int64_t row = r0 + wave * 32 + (lane & 31);
  const bool rv = row < rows;
  const int64_t src = rv ? (idx ? (int64_t)idx[row] : row) : 0;
  const uint16_t* mrow = A + src * ld + 32 * (lane >> 5);
  f32x16_t acc[NSUB];
#pragma unroll
  for (int n = 0; n < NSUB; ++n) acc[n] = f32x16_t{};

  auto issue = [&](int64_t kb, uint4* buf, uint4 (&a)[4]) {
    const uint4* srcf = (const uint4*)bfrag + kb * FU;
    for (int i = wave; i < FU / 64; i += 4) dma16(srcf + i * 64 + lane, (uint8_t*)(buf + i * 64));
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = rv ? *(const uint4*)(mrow + kb * 64 + 8 * j) : make_uint4(0, 0, 0, 0);
  };
  auto body = [&](const uint4* buf, const uint4 (&a)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8_t af = __builtin_bit_cast(bf16x8_t, a[j]);
#pragma unroll
      for (int t = 0; t < NTERM; ++t)
#pragma unroll
        for (int n = 0; n < NSUB; ++n) {
          const bf16x8_t bfr = __builtin_bit_cast(bf16x8_t, buf[((t * NSUB + n) * 4 + j) * 64 + lane]);
          acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bfr, acc[n], 0, 0, 0);
        }
    }
  };

  uint4 aA[4], aB[4];
  if (kb0 < kb1) issue(kb0, vs0, aA);
  for (int64_t kb = kb0; kb < kb1; kb += 2) {
    ring_barrier();  // block kb has landed in vs0; every wave is done with vs1
    if (kb + 1 < kb1) issue(kb + 1, vs1, aB);
    body(vs0, aA);
    if (kb + 1 >= kb1) break;
    ring_barrier();  // block kb+1 has landed in vs1; every wave is done with vs0
    if (kb + 2 < kb1) issue(kb + 2, vs0, aA);
    body(vs1, aB);
  }
  const int col = lane & 31;
  constexpr int W = NSUB * 32;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int64_t ro = r0 + wave * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
    if (ro < rows) {
      float* dst = part + (s * rows + ro) * W;
#pragma unroll
      for (int n = 0; n < NSUB; ++n) dst[n * 32 + col] = acc[n][v];
    }
  }
}

// out[row][j] = scale * sum_s part[s][row][j], j < width (fixed order).
__global__ void project_reduce_kernel(const float* __restrict__ part, int64_t splits, int64_t rows,
                                      int pw, int width, float scale, float* __restrict__ out) {
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= rows * width) return;
  const int64_t r = id / width;
  const int j = (int)(id % width);
  float acc = 0.0f;
  for (int64_t s = 0; s < splits; ++s) acc += part[(s * rows + r) * pw + j];
  out[id] = acc * scale;
}

// Sign key of a factor entry v in row r (r < 2^31): the bits of |v| on top,
// then the row complemented (a lower row ranks higher) and whether v < 0.
// The largest key of a column is its largest-magnitude entry (lowest row on
// ties), and its low bit is that entry's sign.
__device__ __forceinline__ unsigned long long sign_key(float v, int64_t r) {
  return ((unsigned long long)(__float_as_uint(v) & 0x7FFFFFFFu) << 32) |
         ((unsigned long long)(0x7FFFFFFFu - (uint32_t)r) << 1) | (v < 0.0f ? 1ull : 0ull);
}

// rs[p][j] = R[p][j] for j < k (D = I) or R[p][j] sign_j / sqrt(lambda_j)
// (0 below the eigenvalue threshold), zero from k to the end of the last
// 4-column group; ins[rl][p] = In[r0 + rl][p] (0 past row n).  Both tiles are
// contiguous in memory (R is k x k, the 64 input rows are 64 k words); each
// thread loads its share into registers before any LDS write, so a workgroup
// pays one memory round trip per tile instead of one per element.
// The workgroup is 256 threads.
template <int NM, bool SCALE>
__device__ __forceinline__ void rot_stage(double (*rs)[NM + 4], float (*ins)[NM + 1], const float* __restrict__ In,
                                          int64_t n, int64_t r0, int k, const double* __restrict__ R,
                                          const double* __restrict__ lam, const float* sg) {
  constexpr int kRP = (NM * NM + 255) / 256;  // R entries per thread
  constexpr int kIP = (64 * NM + 255) / 256;  // input entries per thread
  const int tid = threadIdx.x;
  const int kk = k * k;
  const int64_t avail = n - r0 < 64 ? n - r0 : 64;
  const int ne = (int)avail * k;
  const float* src = In + r0 * k;
  double rv[kRP];
  double lv[SCALE ? kRP : 1];
  float iv[kIP];
#pragma unroll
  for (int i = 0; i < kRP; ++i) {
    const int e = tid + 256 * i;
    rv[i] = e < kk ? R[e] : 0.0;
    if (SCALE) lv[i] = e < kk ? lam[e % k] : 0.0;
  }
#pragma unroll
  for (int i = 0; i < kIP; ++i) {
    const int e = tid + 256 * i;
    iv[i] = e < ne ? src[e] : 0.0f;
  }
  const double l0 = SCALE ? lam[0] : 0.0;
#pragma unroll
  for (int i = 0; i < kRP; ++i) {
    const int e = tid + 256 * i;
    if (e < kk) {
      const int p = e / k, j = e - p * k;
      double v = rv[i];
      if (SCALE) {
        const double lj = lv[i];
        v = (l0 > 0.0 && lj > kEigZero * l0) ? v * (double)sg[j] / sqrt(lj) : 0.0;
      }
      rs[p][j] = v;
    }
  }
  const int kg = (k + 3) >> 2;
  for (int e = tid; e < k * kg * 4; e += 256) {
    const int p = e / (kg * 4), j = e - p * kg * 4;
    if (j >= k) rs[p][j] = 0.0;
  }
#pragma unroll
  for (int i = 0; i < kIP; ++i) {
    const int e = tid + 256 * i;
    if (e < 64 * k) {
      const int rl = e / k, p = e - rl * k;
      ins[rl][p] = iv[i];
    }
  }
}

// Four consecutive columns 4 jg .. 4 jg + 3 of row rl of ins . rs, binary64.
template <int NM>
__device__ __forceinline__ void rot_row(const double (*rs)[NM + 4], const float (*ins)[NM + 1], int rl, int jg,
                                        int k, float (&o)[4]) {
  double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
  for (int p = 0; p < k; ++p) {
    const double x = (double)ins[rl][p];
    const double2 q0 = *(const double2*)&rs[p][4 * jg];
    const double2 q1 = *(const double2*)&rs[p][4 * jg + 2];
    a0 += x * q0.x;
    a1 += x * q0.y;
    a2 += x * q1.x;
    a3 += x * q1.y;
  }
  o[0] = (float)a0;
  o[1] = (float)a1;
  o[2] = (float)a2;
  o[3] = (float)a3;
}

// First half of the rediagonalisation's tail: Vn = V_old R (n = cols rows of
// binary32, R binary64 k x k, binary64 accumulation), 64 rows per workgroup.
// Thread t keeps the column group jg = t % kg of the rows t / kg + i (256 /
// kg), so it max-reduces one sign key per column; the workgroup's keys go to
// key[j] (zeroed beforehand) by one atomic each.  With amax given, the
// largest |Vn| goes there too (the factor's tensor amax: |V| = |Vn|) and a
// non-finite entry raises the status word.
template <int NM>
__global__ __launch_bounds__(256) void rot_v_kernel(const float* __restrict__ Vold, int64_t n, int k,
                                                    const double* __restrict__ R, float* __restrict__ Vn,
                                                    unsigned long long* __restrict__ key,
                                                    uint32_t* __restrict__ amax) {
  __shared__ __align__(16) double rs[NM][NM + 4];
  __shared__ float ins[64][NM + 1];
  __shared__ unsigned long long ks[NM];
  __shared__ uint32_t am;
  const int tid = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.x * 64;
  rot_stage<NM, false>(rs, ins, Vold, n, r0, k, R, nullptr, nullptr);
  if (tid < k) ks[tid] = 0ull;
  if (tid == 0) am = 0u;
  __syncthreads();
  const int kg = (k + 3) >> 2;
  const int tr = 256 / kg;
  const int jg = tid % kg, rl0 = tid / kg;
  unsigned long long best[4] = {0ull, 0ull, 0ull, 0ull};
  float mx = 0.0f;
  bool bad = false;
  if (rl0 < tr) {
    for (int rl = rl0; rl < 64; rl += tr) {
      const int64_t r = r0 + rl;
      if (r >= n) break;
      float o[4];
      rot_row<NM>(rs, ins, rl, jg, k, o);
      float* out = Vn + r * k + 4 * jg;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (4 * jg + c >= k) break;
        out[c] = o[c];
        const unsigned long long kk = sign_key(o[c], r);
        best[c] = kk > best[c] ? kk : best[c];
        const float a = fabsf(o[c]);
        bad |= !(a <= 3.402823466e38f);
        mx = fmaxf(mx, a);
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (4 * jg + c < k) atomicMax(&ks[4 * jg + c], best[c]);
  }
  if (amax) {
    mx = wave_max(mx);
    if ((tid & 63) == 0) atomicMax(&am, __float_as_uint(mx));
    if (bad) raise_status(kStatusNonFinite);
  }
  __syncthreads();
  if (tid < k) atomicMax(&key[tid], ks[tid]);
  if (amax && tid == 0) atomicMax(amax, am);
}

// Second half: workgroups [0, nbu) form U = P R diag(sign_j lambda_j^-1/2)
// (64 rows each, binary64 accumulation; 0 below the eigenvalue threshold),
// the others V = Vn diag(sign) (64 rows each); workgroup 0 also writes
// S = sqrt(lambda) (0 below the threshold).  sign_j is the low bit of key[j].
// With amax given, the largest |U| goes there and a non-finite U entry
// raises the status word.
template <int NM>
__global__ __launch_bounds__(256) void rot_u_kernel(const float* __restrict__ P, int64_t rows, int k,
                                                    const double* __restrict__ R, const double* __restrict__ lam,
                                                    const unsigned long long* __restrict__ key,
                                                    const float* __restrict__ Vn, int64_t cols,
                                                    float* __restrict__ U, float* __restrict__ V,
                                                    float* __restrict__ S, uint32_t* __restrict__ amax, int nbu) {
  __shared__ __align__(16) double rs[NM][NM + 4];
  __shared__ float ins[64][NM + 1];
  __shared__ float sg[NM];
  __shared__ uint32_t am;
  const int tid = threadIdx.x;
  if (tid < k) sg[tid] = (key[tid] & 1ull) ? -1.0f : 1.0f;
  if (tid == 0) am = 0u;
  if ((int)blockIdx.x >= nbu) {
    __syncthreads();
    const int64_t r0 = (int64_t)((int)blockIdx.x - nbu) * 64;
    const int64_t r1 = r0 + 64 < cols ? r0 + 64 : cols;
    const int nloc = (int)(r1 - r0) * k;
    const float* src = Vn + r0 * k;
    float* dst = V + r0 * k;
    constexpr int kIP = (64 * NM + 255) / 256;
    float vv[kIP];
#pragma unroll
    for (int i = 0; i < kIP; ++i) {
      const int e = tid + 256 * i;
      vv[i] = e < nloc ? src[e] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < kIP; ++i) {
      const int e = tid + 256 * i;
      if (e < nloc) dst[e] = vv[i] * sg[e % k];
    }
    return;
  }
  const int64_t r0 = (int64_t)blockIdx.x * 64;
  if (blockIdx.x == 0 && tid < k) {
    const double l0 = lam[0], lj = lam[tid];
    S[tid] = (l0 > 0.0 && lj > kEigZero * l0) ? (float)sqrt(lj) : 0.0f;
  }
  __syncthreads();
  rot_stage<NM, true>(rs, ins, P, rows, r0, k, R, lam, sg);
  __syncthreads();
  const int kg = (k + 3) >> 2;
  float mx = 0.0f;
  bool bad = false;
  for (int item = tid; item < 64 * kg; item += 256) {
    const int rl = item / kg, jg = item - rl * kg;
    const int64_t r = r0 + rl;
    if (r >= rows) continue;
    float o[4];
    rot_row<NM>(rs, ins, rl, jg, k, o);
    float* out = U + r * k + 4 * jg;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (4 * jg + c >= k) break;
      out[c] = o[c];
      const float a = fabsf(o[c]);
      bad |= !(a <= 3.402823466e38f);
      mx = fmaxf(mx, a);
    }
  }
  if (amax) {
    mx = wave_max(mx);
    if ((tid & 63) == 0) atomicMax(&am, __float_as_uint(mx));
    if (bad) raise_status(kStatusNonFinite);
    __syncthreads();
    if (tid == 0) atomicMax(amax, am);
  }
}

}  // namespace metis
