// metis.hip -- host side of libmetis: the C ABI declared in include/metis.h.
//
// Argument validation is synchronous; all work is enqueued on the caller's
// stream; scratch memory is carved from the caller's workspace.  The only
// device state the library owns is a per-device numeric status word and the
// Gaussian quantile table, both static __device__ arrays.

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/metis.h"
#include "common.hpp"
#include "gemm.hpp"
#include "gemm_launch.hpp"
#include "quant.hpp"
#include "quant_fast.hpp"
#include "rsvd.hpp"
#include "mxfp4.hpp"
#include "mxfp4_gemm.hpp"

using namespace metis;

// Scratch of the allocation-free quantiser entry point (metis_quantize_static):
// one array per GPU, held until the process ends.  Host code never names it
// directly: the device address of each GPU's copy comes from
// hipGetSymbolAddress at set-up (g_scratch_ptr below), and only that address
// is passed to kernels.
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {

thread_local std::string g_last_error;

metis_status fail(metis_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

#define HIP_TRY(expr)                                                                     \
  do {                                                                                    \
    hipError_t e__ = (expr);                                                              \
    if (e__ != hipSuccess) return fail(METIS_E_HIP, "%s: %s", #expr, hipGetErrorString(e__)); \
  } while (0)

#define LAUNCH_CHECK()                                                                    \
  do {                                                                                    \
    hipError_t e__ = hipGetLastError();                                                   \
    if (e__ != hipSuccess) return fail(METIS_E_HIP, "kernel launch: %s", hipGetErrorString(e__)); \
  } while (0)

// ---------------------------------------------- benchmark instrumentation

// When enabled, a pair of HIP events is recorded on the launching stream
// around each main split-GEMM kernel (kind 0), each quantiser sweep (kind
// 1: amax pass, kind 2: quantise pass), each MXFP4 GEMM kernel (kind 3), the
// sketch of a refresh step (kind 4) and metis_decompose's projection and
// rediagonalisation (kind 5).  Events are created once, when timing is
// enabled; recording them allocates nothing.
struct TimingRec {
  hipEvent_t a, b;
  int64_t kind, d0, d1, d2, d3;
};
std::mutex g_tmu;
std::vector<TimingRec> g_trecs;
size_t g_tused = 0;
bool g_timing = false;
uint32_t g_tkinds = ~0u;  // kinds recorded while timing is enabled

TimingRec* timing_begin(hipStream_t st, int64_t kind, int64_t d0, int64_t d1, int64_t d2, int64_t d3) {
  if (!g_timing || kind < 0 || kind > 31 || !((g_tkinds >> kind) & 1u)) return nullptr;
  std::lock_guard<std::mutex> lk(g_tmu);
  if (g_tused >= g_trecs.size()) return nullptr;
  TimingRec* r = &g_trecs[g_tused++];
  r->kind = kind;
  r->d0 = d0;
  r->d1 = d1;
  r->d2 = d2;
  r->d3 = d3;
  if (hipEventRecord(r->a, st) != hipSuccess) return nullptr;  // record is skipped
  return r;
}

void timing_end(TimingRec* r, hipStream_t st) {
  if (r) (void)hipEventRecord(r->b, st);  // a failed record reads back as -1 ms
}

// ------------------------------------------------------- Omega quantile table

// Phi^{-1}(p) for 0 < p < 0.5 by Newton's method on Phi(x) = erfc(-x/sqrt2)/2,
// started from the rational approximation of Abramowitz & Stegun 26.2.23.
double norm_quantile_lower(double p) {
  const double t = sqrt(-2.0 * log(p));
  double x = -(t - (2.515517 + 0.802853 * t + 0.010328 * t * t) /
                       (1.0 + 1.432788 * t + 0.189269 * t * t + 0.001308 * t * t * t));
  for (int it = 0; it < 8; ++it) {
    const double f = 0.5 * erfc(-x / sqrt(2.0)) - p;
    const double d = exp(-0.5 * x * x) / sqrt(2.0 * M_PI);
    const double step = f / d;
    x -= step;
    if (fabs(step) <= 1e-17 * fabs(x)) break;
  }
  return x;
}

uint16_t bf16_bits_rne(double x) {
  if (x == 0.0) return 0;
  int e;
  const double m = frexp(x, &e);          // x = m 2^e, 0.5 <= |m| < 1
  const double q = nearbyint(m * 256.0);  // 8 significant bits, ties to even
  const float f = (float)ldexp(q, e - 8); // exact
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

const uint16_t* host_omega_table() {
  static uint16_t table[65536];
  static std::once_flag once;
  std::call_once(once, [] {
    for (int t = 0; t < 32768; ++t) {
      const double x = norm_quantile_lower((t + 0.5) / 65536.0);
      const uint16_t b = bf16_bits_rne(x);
      table[t] = b;
      table[65535 - t] = b ^ 0x8000u;  // Phi^-1(1 - p) = -Phi^-1(p)
    }
  });
  return table;
}

std::mutex g_dev_mu;
bool g_dev_ready[64] = {false};
void* g_scratch_ptr[64] = {nullptr};

// Once per device, with that device current: the Gaussian quantile table, the
// numeric status word and the address of the static scratch array.
metis_status ensure_device_tables() {
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) return fail(METIS_E_UNSUPPORTED, "device index %d", dev);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (!g_dev_ready[dev]) {
    HIP_TRY(hipMemcpyToSymbol(HIP_SYMBOL(g_omega_table), host_omega_table(), 65536 * 2));
    const int zero = 0;
    HIP_TRY(hipMemcpyToSymbol(HIP_SYMBOL(g_metis_status), &zero, sizeof(int)));
    void* p = nullptr;
    HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(METIS_E_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
    g_dev_ready[dev] = true;
  }
  return METIS_OK;
}

// This device's static scratch (after ensure_device_tables).
void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  return g_scratch_ptr[dev];
}

// ------------------------------------------------------------- workspace --

struct Carver {
  char* base;
  size_t off = 0;
  size_t cap;
  explicit Carver(void* b, size_t c) : base((char*)b), cap(c) {}
  template <typename T>
  T* take(size_t count) {
    off = (off + 255) & ~(size_t)255;
    T* p = base ? (T*)(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
  size_t used() const { return (off + 255) & ~(size_t)255; }
};

inline int round_up(int a, int b) { return (a + b - 1) / b * b; }
inline int64_t round_up64(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

inline unsigned grid1(int64_t n, int block) { return (unsigned)((n + block - 1) / block); }

bool dtype_ok(int32_t dt) { return dt == METIS_BF16 || dt == METIS_F32; }

// --------------------------------------------------------- decomposition --

struct DecompWs {
  uint32_t *keys, *hist, *meta;
  uint2* cand;
  uint8_t* flags;
  int32_t* idx;
  float *om, *y, *q, *bpart, *b, *p, *vn, *ppart, *spart;
  unsigned long long* key;  // per-column sign keys of the rediagonalisation
  uint16_t *vfrag, *ofrag;
  int64_t proj_nkb, proj_kbps, proj_splits, sk_kbps, sk_splits;
  double *gpart, *g, *rinv, *z, *theta, *ptp, *rot, *lam;
  int gblocks, slices;
  int64_t rows_per_gblock, rows_per_slice;
};

// Compute units of the target (MI355X: 8 XCDs of 32).  Launch plans that
// size a grid to one round of resident workgroups use it; on another chip
// they stay correct, only less even.
constexpr int64_t kCUs = 256;

// Split-K plan of an MFMA product with nr output rows over nkb 64-wide K
// blocks, for workgroups of 128 rows: with `wave` > 0, at most that many
// workgroups when the rows alone do not fill them (one full round of
// resident workgroups, so no second, mostly idle round); else about 1024.
// Returns the split count.
int64_t split_plan(int64_t nr, int64_t nkb, int64_t* kbps, int64_t wave = 0) {
  if (nkb <= 0 || nr <= 0) {  // no K blocks (cols < 64): the MFMA product is not used
    *kbps = 0;
    return 0;
  }
  const int64_t row_blocks = (nr + 127) / 128;
  int64_t splits = wave > 0 ? wave / row_blocks : (1024 + row_blocks - 1) / row_blocks;
  if (splits > nkb) splits = nkb;
  if (splits < 1) splits = 1;
  *kbps = (nkb + splits - 1) / splits;
  return (nkb + *kbps - 1) / *kbps;
}

// out (nr x width, row-major) = scale * A[src rows] B on MFMA with B as NTERM
// bf16 terms (width <= 96; A bf16, 16-byte aligned rows).
template <int NTERM, int NSUB>
metis_status mfma_product_n(const uint16_t* A, int64_t ld, int64_t nr, const int32_t* idx,
                            const float* B, int64_t K, int width, int64_t ldb, int64_t nkb,
                            int64_t kbps, int64_t splits, float scale, uint16_t* frag, float* part,
                            float* out, hipStream_t st, bool reduce) {
  hipLaunchKernelGGL((proj_prep_kernel<NTERM, NSUB>), dim3(grid1(nkb * NSUB * 2048, 256)), dim3(256), 0,
                     st, B, K, width, ldb, nkb, frag);
  LAUNCH_CHECK();
  hipLaunchKernelGGL((project_mfma_kernel<NTERM, NSUB>),
                     dim3((unsigned)ceil_div<int64_t>(nr, 128), (unsigned)splits), dim3(256), 0, st, A, ld,
                     nr, idx, frag, nkb, kbps, part);
  LAUNCH_CHECK();
  if (reduce) {
    hipLaunchKernelGGL(project_reduce_kernel, dim3(grid1(nr * width, 256)), dim3(256), 0, st, part, splits,
                       nr, NSUB * 32, width, scale, out);
    LAUNCH_CHECK();
  }
  return METIS_OK;
}

// Row pitch of the split partials of mfma_product for an output width.
inline int mfma_part_pitch(int width) { return width <= 32 ? 32 : (width <= 64 ? 64 : 96); }

template <int NTERM>
metis_status mfma_product(const uint16_t* A, int64_t ld, int64_t nr, const int32_t* idx, const float* B,
                          int64_t K, int width, int64_t ldb, int64_t nkb, int64_t kbps, int64_t splits,
                          float scale, uint16_t* frag, float* part, float* out, hipStream_t st,
                          bool reduce = true) {
  if (width <= 32)
    return mfma_product_n<NTERM, 1>(A, ld, nr, idx, B, K, width, ldb, nkb, kbps, splits, scale, frag,
                                    part, out, st, reduce);
  if (width <= 64)
    return mfma_product_n<NTERM, 2>(A, ld, nr, idx, B, K, width, ldb, nkb, kbps, splits, scale, frag,
                                    part, out, st, reduce);
  return mfma_product_n<NTERM, 3>(A, ld, nr, idx, B, K, width, ldb, nkb, kbps, splits, scale, frag, part,
                                  out, st, reduce);
}

DecompWs carve_decompose(Carver& cv, int64_t rows, int64_t cols, int k, int n, int64_t lr,
                         bool sample) {
  DecompWs w{};
  if (sample) {
    w.keys = cv.take<uint32_t>(rows);
    w.hist = cv.take<uint32_t>(65536);
    w.meta = cv.take<uint32_t>(16);
    w.cand = cv.take<uint2>(kCandMax);
    w.flags = cv.take<uint8_t>(rows);
  }
  w.idx = cv.take<int32_t>(lr);
  w.om = cv.take<float>(cols * n);
  w.y = cv.take<float>(lr * n);
  w.q = cv.take<float>(lr * n);
  const int64_t gmax = rows > lr ? rows : lr;
  const int64_t gsrc = gmax > cols ? gmax : cols;
  // Gram partials: a workgroup per 64 rows, at most 512
  w.gblocks = (int)((gsrc + 63) / 64 < 512 ? (gsrc + 63) / 64 : 512);
  if (w.gblocks < 1) w.gblocks = 1;
  w.gpart = cv.take<double>((size_t)w.gblocks * kMaxN * kMaxN);
  w.g = cv.take<double>(kMaxN * kMaxN);
  w.rinv = cv.take<double>(kMaxN * kMaxN);
  // sketch product B = Q^T M_s split over sample-row slices; a small sample
  // takes enough slices of >= 16 rows for about 512 workgroups, since each
  // workgroup walks its rows one dependent batch of loads after another
  int64_t slices = lr >= 4096 ? 16 : (lr >= 512 ? 4 : 1);
  const int64_t cblocks = (cols + kSkbCols - 1) / kSkbCols, fill = (512 + cblocks - 1) / cblocks;
  const int64_t cap = lr / 16 > 1 ? lr / 16 : 1;
  if (slices < fill) slices = fill < cap ? fill : cap;
  if (slices < 1) slices = 1;
  w.slices = (int)slices;
  w.rows_per_slice = (lr + w.slices - 1) / w.slices;
  w.bpart = cv.take<float>((size_t)w.slices * n * cols);
  w.b = cv.take<float>((size_t)n * cols);
  w.z = cv.take<double>(kMaxN * kMaxN);
  w.theta = cv.take<double>(kMaxN);
  w.p = cv.take<float>(rows * k);
  w.ptp = cv.take<double>(kMaxN * kMaxN);
  w.rot = cv.take<double>(kMaxN * kMaxN);
  w.lam = cv.take<double>(kMaxN);
  w.vn = cv.take<float>(cols * k);
  w.key = cv.take<unsigned long long>(kMaxN);
  // MFMA products (bf16 operands, cols % 64 == 0): split-K plans for the
  // projection P = M V (rows x k) and the sketch Y = M_s Omega (lr x n)
  w.proj_nkb = cols / 64;
  // the projection kernel keeps 3 workgroups per CU (48 KB of LDS each)
  w.proj_splits = split_plan(rows, w.proj_nkb, &w.proj_kbps, 3 * kCUs);
  w.sk_splits = split_plan(lr, w.proj_nkb, &w.sk_kbps);
  w.vfrag = cv.take<uint16_t>((size_t)w.proj_nkb * proj_frag_u4<3, 3>() * 8);
  w.ofrag = cv.take<uint16_t>((size_t)w.proj_nkb * proj_frag_u4<1, 3>() * 8);
  w.ppart = cv.take<float>((size_t)w.proj_splits * rows * 96);
  w.spart = cv.take<float>((size_t)w.sk_splits * lr * 96);
  return w;
}

// The Jacobi eigensolver with LDS sized to n (callers check the launch);
// clear (n words, may be null) is zeroed on the way.  With n <= 64 (the
// rediagonalisation at k = 61) it takes 67 KB of LDS, which fits beside one
// workgroup of the residual sweeps (78 KB).
void launch_jacobi(const double* g, int n, double* w, double* z, unsigned long long* clear, hipStream_t st) {
  if (n <= 32)
    hipLaunchKernelGGL(jacobi_kernel<32>, dim3(1), dim3(1024), 0, st, g, n, w, z, clear);
  else if (n <= 64)
    hipLaunchKernelGGL(jacobi_kernel<64>, dim3(1), dim3(1024), 0, st, g, n, w, z, clear);
  else if (n <= 72)
    hipLaunchKernelGGL(jacobi_kernel<72>, dim3(1), dim3(1024), 0, st, g, n, w, z, clear);
  else
    hipLaunchKernelGGL(jacobi_kernel<kMaxN>, dim3(1), dim3(1024), 0, st, g, n, w, z, clear);
}

// The rediagonalisation's two tail kernels with LDS sized to k.
template <int NM>
void launch_rot(DecompWs& w, const metis_factors* f, int64_t rows, int64_t cols, int k, uint32_t* amax_u,
                uint32_t* amax_v, hipStream_t st) {
  hipLaunchKernelGGL(rot_v_kernel<NM>, dim3((unsigned)ceil_div<int64_t>(cols, 64)), dim3(256), 0, st, f->V, cols,
                     k, w.rot, w.vn, w.key, amax_v);
  const int nbu = (int)ceil_div<int64_t>(rows, 64);
  const int nbv = (int)ceil_div<int64_t>(cols, 64);
  hipLaunchKernelGGL(rot_u_kernel<NM>, dim3((unsigned)(nbu + nbv)), dim3(256), 0, st, w.p, rows, k, w.rot, w.lam,
                     w.key, w.vn, cols, f->U, f->V, f->S, amax_u, nbu);
}

metis_status launch_gram(const float* X, int64_t nr, int n, int64_t rs, int64_t cs, int maxblocks,
                         double* part, double* G, hipStream_t st) {
  int64_t per = (nr + maxblocks - 1) / maxblocks;
  per = (per + 31) / 32 * 32;
  if (per < 64) per = 64;
  const int blocks = (int)((nr + per - 1) / per);
  const dim3 grid(blocks > 0 ? blocks : 1);
  switch ((n + 15) / 16) {
    case 1: hipLaunchKernelGGL(gram_partial_kernel<1>, grid, dim3(256), 0, st, X, nr, n, rs, cs, per, part); break;
    case 2: hipLaunchKernelGGL(gram_partial_kernel<2>, grid, dim3(256), 0, st, X, nr, n, rs, cs, per, part); break;
    case 3: hipLaunchKernelGGL(gram_partial_kernel<3>, grid, dim3(256), 0, st, X, nr, n, rs, cs, per, part); break;
    case 4: hipLaunchKernelGGL(gram_partial_kernel<4>, grid, dim3(256), 0, st, X, nr, n, rs, cs, per, part); break;
    case 5: hipLaunchKernelGGL(gram_partial_kernel<5>, grid, dim3(256), 0, st, X, nr, n, rs, cs, per, part); break;
    default: hipLaunchKernelGGL(gram_partial_kernel<6>, grid, dim3(256), 0, st, X, nr, n, rs, cs, per, part); break;
  }
  LAUNCH_CHECK();
  hipLaunchKernelGGL(reduce_gram_kernel, dim3(grid1(n * n, 64)), dim3(256), 0, st, part,
                     blocks > 0 ? blocks : 1, n * n, G);
  LAUNCH_CHECK();
  return METIS_OK;
}

// P (nr x n) from the split partials of an MFMA product (pitch pw) and G =
// P^T P, with the row blocks of launch_gram: the same bits as the split
// reduction followed by launch_gram on P.
metis_status launch_gram_from_parts(const float* part, int64_t splits, int pw, float scale, float* P, int64_t nr,
                                    int n, int maxblocks, double* gpart, double* G, hipStream_t st) {
  int64_t per = (nr + maxblocks - 1) / maxblocks;
  per = (per + 31) / 32 * 32;
  if (per < 64) per = 64;
  const int blocks = (int)((nr + per - 1) / per);
  const dim3 grid(blocks > 0 ? blocks : 1);
  switch ((n + 15) / 16) {
    case 1: hipLaunchKernelGGL(gram_rows_kernel<1>, grid, dim3(256), 0, st, part, splits, pw, scale, P, nr, n, per, gpart); break;
    case 2: hipLaunchKernelGGL(gram_rows_kernel<2>, grid, dim3(256), 0, st, part, splits, pw, scale, P, nr, n, per, gpart); break;
    case 3: hipLaunchKernelGGL(gram_rows_kernel<3>, grid, dim3(256), 0, st, part, splits, pw, scale, P, nr, n, per, gpart); break;
    case 4: hipLaunchKernelGGL(gram_rows_kernel<4>, grid, dim3(256), 0, st, part, splits, pw, scale, P, nr, n, per, gpart); break;
    case 5: hipLaunchKernelGGL(gram_rows_kernel<5>, grid, dim3(256), 0, st, part, splits, pw, scale, P, nr, n, per, gpart); break;
    default: hipLaunchKernelGGL(gram_rows_kernel<6>, grid, dim3(256), 0, st, part, splits, pw, scale, P, nr, n, per, gpart); break;
  }
  LAUNCH_CHECK();
  hipLaunchKernelGGL(reduce_gram_kernel, dim3(grid1(n * n, 64)), dim3(256), 0, st, gpart, (int)grid.x, n * n, G);
  LAUNCH_CHECK();
  return METIS_OK;
}

metis_status validate_config(const metis_config* cfg) {
  if (!cfg) return fail(METIS_E_INVALID, "cfg is NULL");
  if (cfg->k < 1 || cfg->k > kMaxN) return fail(METIS_E_INVALID, "k=%d outside [1, %d]", cfg->k, kMaxN);
  if (cfg->s < 0) return fail(METIS_E_INVALID, "s=%d negative", cfg->s);
  if (cfg->k + cfg->s > kMaxN)
    return fail(METIS_E_UNSUPPORTED, "k + s = %d exceeds %d", cfg->k + cfg->s, kMaxN);
  if (cfg->refresh < 1) return fail(METIS_E_INVALID, "refresh=%d < 1", cfg->refresh);
  if (cfg->rounding != METIS_RNE && cfg->rounding != METIS_SR)
    return fail(METIS_E_INVALID, "rounding=%d", cfg->rounding);
  return METIS_OK;
}

// ------------------------------------------------------------ quantiser --

constexpr int64_t kAmaxWords = (int64_t)kAmaxSlotStride * (1 + kAmaxSlots);

struct QuantWs {
  uint32_t* amax;  // words 0..2: residual, U, V; from word kAmaxSlotStride: the residual's slots
  float* pscale;
  _Float16* ucat;
  _Float16* vcat;
};

QuantWs carve_quantize(Carver& cv, int64_t rows, int64_t cols, int k) {
  QuantWs w{};
  w.amax = cv.take<uint32_t>(kAmaxWords);
  w.pscale = cv.take<float>(1);
  if (k > 0) {
    const int kc = 3 * round_up(k, 16);
    w.ucat = cv.take<_Float16>((size_t)((rows + 31) & ~(int64_t)31) * kc);
    w.vcat = cv.take<_Float16>((size_t)((cols + 63) & ~(int64_t)63) * kc);
  }
  return w;
}

template <int NKK>
metis_status launch_quant_pair(const QuantParams& qp, dim3 grid, int64_t rows, int64_t cols,
                               hipStream_t st) {
  const int64_t kc = NKK * 16;
  TimingRec* t1 = timing_begin(st, 1, rows, cols, qp.axes, kc);
  hipLaunchKernelGGL((quant_amax_kernel<NKK>), grid, dim3(kQThreads), 0, st, qp);
  LAUNCH_CHECK();
  timing_end(t1, st);
  TimingRec* t2 = timing_begin(st, 2, rows, cols, qp.axes, kc);
  if (qp.sr)
    hipLaunchKernelGGL((quant_kernel<NKK, true>), grid, dim3(kQThreads), 0, st, qp);
  else
    hipLaunchKernelGGL((quant_kernel<NKK, false>), grid, dim3(kQThreads), 0, st, qp);
  LAUNCH_CHECK();
  timing_end(t2, st);
  return METIS_OK;
}

template <int NKK, int TPW>
metis_status launch_quant_fast(const QuantParams& qp, unsigned nwg, int64_t rows, int64_t cols, hipStream_t st) {
  const int64_t kc = NKK * 16;
  const dim3 g(nwg), b(kQThreads);
  TimingRec* t1 = timing_begin(st, 1, rows, cols, qp.axes, kc);
  hipLaunchKernelGGL((qf_amax_kernel<NKK, TPW>), g, b, 0, st, qp);
  LAUNCH_CHECK();
  timing_end(t1, st);
  TimingRec* t2 = timing_begin(st, 2, rows, cols, qp.axes, kc);
#define QF_LAUNCH(SR_, AX_) hipLaunchKernelGGL((qf_quant_kernel<NKK, SR_, AX_, TPW>), g, b, 0, st, qp)
  switch (qp.axes | (qp.sr ? 4 : 0)) {
    case 1: QF_LAUNCH(false, 1); break;
    case 2: QF_LAUNCH(false, 2); break;
    case 3: QF_LAUNCH(false, 3); break;
    case 5: QF_LAUNCH(true, 1); break;
    case 6: QF_LAUNCH(true, 2); break;
    default: QF_LAUNCH(true, 3); break;
  }
#undef QF_LAUNCH
  LAUNCH_CHECK();
  timing_end(t2, st);
  return METIS_OK;
}

// The whole-tile sweeps (quant_fast.hpp) take bf16 operands of whole 128 x 64
// tiles with 16-byte aligned rows and outputs, both orientations, and no
// residual export.
bool quant_fast_ok(const QuantParams& qp) {
  auto al = [](const void* p, uintptr_t a) { return p == nullptr || ((uintptr_t)p % a) == 0; };
  return qp.amax_slots && qp.dtype == METIS_BF16 && qp.rows % kQT_R == 0 && qp.cols % kQT_C == 0 && qp.ld % 8 == 0 &&
         al(qp.M, 16) && qp.resid == nullptr && qp.shared_draws && qp.axes >= 1 && qp.axes <= 3 && al(qp.codes0, 16) &&
         al(qp.codes1, 16) && al(qp.scales0, 2) && al(qp.scales1, 2) && qp.rows / kQT_R <= INT32_MAX &&
         qp.cols / kQT_C <= INT32_MAX / 2;
}

template <int TPW>
metis_status launch_quant_fast_w(const QuantParams& qp, bool has_f, int64_t rows, int64_t cols, hipStream_t st,
                                 bool* done) {
  const int64_t P = rows / kQT_R, ntc = cols / kQT_C;
  const int64_t W = P * ceil_div<int64_t>(ntc, TPW);
  const int64_t nwg = 8 * ceil_div<int64_t>(W, 8);
  *done = false;
  if (nwg > INT32_MAX) return METIS_OK;
  *done = true;
  if (!has_f) return launch_quant_fast<0, TPW>(qp, (unsigned)nwg, rows, cols, st);
  switch (qp.kc / 16) {
    case 3: return launch_quant_fast<3, TPW>(qp, (unsigned)nwg, rows, cols, st);
    case 6: return launch_quant_fast<6, TPW>(qp, (unsigned)nwg, rows, cols, st);
    case 9: return launch_quant_fast<9, TPW>(qp, (unsigned)nwg, rows, cols, st);
    case 12: return launch_quant_fast<12, TPW>(qp, (unsigned)nwg, rows, cols, st);
    default: *done = false; return METIS_OK;
  }
}

metis_status run_quant(const QuantParams& qp0, bool has_f, int64_t rows, int64_t cols,
                       hipStream_t st) {
  QuantParams qp = qp0;
  if (quant_fast_ok(qp)) {
    // four tiles (256 columns: whole 128-byte lines of axis-1 codes) per
    // workgroup when that still gives ~2 workgroups per CU, else one
    const int64_t tiles = (rows / kQT_R) * (cols / kQT_C);
    bool done = false;
    metis_status s = tiles >= 4 * 512 && cols >= 4 * kQT_C ? launch_quant_fast_w<4>(qp, has_f, rows, cols, st, &done)
                                                            : launch_quant_fast_w<1>(qp, has_f, rows, cols, st, &done);
    if (done || s != METIS_OK) return s;
  }
  const int64_t panels = ceil_div<int64_t>(rows, kQT_R);
  const int64_t ntc = ceil_div<int64_t>(cols, kQT_C);
  int64_t tpw = panels * ntc / 2048;
  if (tpw < 1) tpw = 1;
  if (tpw > 16) tpw = 16;
  qp.tiles_per_wg = (int)tpw;
  const dim3 grid((unsigned)panels, (unsigned)ceil_div<int64_t>(ntc, tpw));
  if (panels > INT32_MAX || grid.y > 65535u) return fail(METIS_E_UNSUPPORTED, "operand too large");
  if (!has_f) return launch_quant_pair<0>(qp, grid, rows, cols, st);
  switch (qp.kc / 16) {
    case 3: return launch_quant_pair<3>(qp, grid, rows, cols, st);
    case 6: return launch_quant_pair<6>(qp, grid, rows, cols, st);
    case 9: return launch_quant_pair<9>(qp, grid, rows, cols, st);
    case 12: return launch_quant_pair<12>(qp, grid, rows, cols, st);
    default: return fail(METIS_E_UNSUPPORTED, "rank above 64 in the quantiser");
  }
}

bool q4_ok(const metis_q4& q, int64_t n_outer, int64_t k_len) {
  return q.codes && q.scales && q.tensor_scale && q.n_outer == n_outer && q.k_len == k_len &&
         (k_len % 16) == 0;
}

// ----------------------------------------------------------------- GEMMs --

template <int BM, int BN, int WM, int WN>
metis_status launch_gemm_cfg(const GemmParams& gp, int splits, hipStream_t st) {
  const int64_t tiles = ceil_div<int64_t>(gp.M, BM) * ceil_div<int64_t>(gp.N, BN);
  if (tiles <= 0) return METIS_OK;
  const size_t lds = gemm_lds_bytes<BM, BN, WM, WN>();
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [&] {
    attr_err = hipFuncSetAttribute((const void*)gemm_fp4_kernel<BM, BN, WM, WN>,
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  });
  if (attr_err != hipSuccess) return fail(METIS_E_HIP, "hipFuncSetAttribute: %s", hipGetErrorString(attr_err));
  hipLaunchKernelGGL((gemm_fp4_kernel<BM, BN, WM, WN>), dim3((unsigned)tiles, (unsigned)splits),
                     dim3(WM * WN * 64), lds, st, gp);
  LAUNCH_CHECK();
  return METIS_OK;
}

// The register-dequant kernel needs whole 256-wide K stages and 16-byte
// aligned code, scale and extension rows.
bool gemm_reg_ok(const GemmParams& gp) {
  return gp.K % 256 == 0 && ((uintptr_t)gp.a_codes & 15) == 0 && ((uintptr_t)gp.b_codes & 15) == 0 &&
         ((uintptr_t)gp.a_scales & 15) == 0 && ((uintptr_t)gp.b_scales & 15) == 0 &&
         ((uintptr_t)gp.a_ext & 15) == 0 && ((uintptr_t)gp.b_ext & 15) == 0;
}

enum GemmShape { kGemmBig, kGemmMid, kGemmTall, kGemmWide, kGemmSmall };

GemmShape gemm_shape(int64_t M, int64_t N) {
  if (N <= 64 && M > 64) return kGemmTall;
  if (M <= 64 && N > 64) return kGemmWide;
  if (M <= 64 && N <= 64) return kGemmSmall;
  const int64_t t256 = ceil_div<int64_t>(M, 256) * ceil_div<int64_t>(N, 256);
  return t256 >= 256 ? kGemmBig : kGemmMid;
}

// C = alpha A B^T (+ K-extension), one workgroup per output tile.
metis_status launch_gemm(const GemmParams& gp, hipStream_t st) {
  if (gp.M <= 0 || gp.N <= 0) return METIS_OK;
  switch (gemm_shape(gp.M, gp.N)) {
    case kGemmBig:
      if (gemm_reg_ok(gp)) {
        const hipError_t e = launch_gemm_big(gp, 1, st);
        return e == hipSuccess ? METIS_OK : fail(METIS_E_HIP, "gemm launch: %s", hipGetErrorString(e));
      }
      return launch_gemm_cfg<256, 256, 4, 2>(gp, 1, st);
    case kGemmMid: return launch_gemm_cfg<128, 128, 2, 2>(gp, 1, st);
    case kGemmTall: return launch_gemm_cfg<256, 64, 8, 1>(gp, 1, st);
    case kGemmWide: return launch_gemm_cfg<64, 256, 1, 8>(gp, 1, st);
    default: return launch_gemm_cfg<64, 64, 2, 2>(gp, 1, st);
  }
}

struct SideQ {
  const metis_q4* res;  // residual in the product's K orientation
  const metis_q4* out;  // factor along the output rows (left) / cols (right)
  const metis_q4* kf;   // factor along K
  const float* S;
  int k;
};

struct SplitWs {
  float *pa, *p1, *p2, *t2, *ones;  // thin-product partial sums; T2 summed
  uint4 *bf_E, *bf_F;             // thin operands as fp16 MFMA fragments
  uint16_t *a_ext, *b_ext;
  int64_t kext;
  int ksR, ksL, sa, s1, s2;
};

// K splits of a thin product with m rows: about 512 workgroups, at least two
// K steps each.
int thin_splits(int64_t m, int64_t K) {
  const int64_t wg = ceil_div<int64_t>(m, kThinRows);
  const int64_t nks = ceil_div<int64_t>(K, 64);
  int64_t s = ceil_div<int64_t>(512, wg);
  const int64_t smax = std::max<int64_t>(1, nks / 2);
  if (s > smax) s = smax;
  if (s > 64) s = 64;
  return (int)std::max<int64_t>(1, s);
}

SplitWs carve_split(Carver& cv, int64_t M, int64_t N, int64_t K, int kL, int kR) {
  SplitWs w{};
  w.ksR = round_up(kR, 16);
  w.ksL = round_up(kL, 16);
  w.kext = round_up(2 * w.ksR + 2 * w.ksL, 64);
  w.ones = cv.take<float>(4);
  const size_t frag = (size_t)ceil_div<int64_t>(K, 64) * 512;
  if (kR > 0) {
    w.sa = thin_splits(M, K);
    w.pa = cv.take<float>((size_t)w.sa * M * 64);
    w.bf_E = cv.take<uint4>(frag);
  }
  if (kL > 0) {
    w.s1 = thin_splits(N, K);
    w.p1 = cv.take<float>((size_t)w.s1 * N * 64);
    w.bf_F = cv.take<uint4>(frag);
  }
  if (kL > 0 && kR > 0) {
    w.s2 = thin_splits(kL, K);
    w.p2 = cv.take<float>((size_t)w.s2 * kL * 64);
    w.t2 = cv.take<float>((size_t)kL * 64);
  }
  if (w.kext > 0) {
    w.a_ext = cv.take<uint16_t>((size_t)round_up64(M, 32) * w.kext);
    w.b_ext = cv.take<uint16_t>((size_t)round_up64(N, 32) * w.kext);
  }
  return w;
}

// The K-extension of a split product: P_raw = L_R E, T1^T = R_R F^T and
// T2 = F E on the thin-product kernel (the three in one launch, after one
// launch that dequantises E and F into MFMA fragments), then the bf16 hi/lo
// operands a_ext / b_ext of the extra K columns (with S, Lambda and the
// tensor scales folded in), both in one launch.
metis_status split_ext(const SideQ& L, const SideQ& R, int64_t M, int64_t N, int64_t K, const SplitWs& w,
                       hipStream_t st) {
  if (L.k == 0 && R.k == 0) return METIS_OK;
  if (L.k == 0 || R.k == 0) {  // the ones stand in for the scales of the side without factors
    hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(64), 0, st, (uint32_t*)w.ones, 0x3F800000u,
                       (int64_t)4);
    LAUNCH_CHECK();
  }
  const int64_t nks = ceil_div<int64_t>(K, 64);
  {  // fragments of E (R's factor) and F (L's factor)
    ThinB b[2] = {};
    int nbf = 0;
    if (R.k > 0) b[nbf++] = ThinB{R.kf->codes, R.kf->scales, R.k, w.bf_E};
    if (L.k > 0) b[nbf++] = ThinB{L.kf->codes, L.kf->scales, L.k, w.bf_F};
    hipLaunchKernelGGL(thin_bfrag_kernel, dim3(grid1(nks * 512 * nbf, 256)), dim3(256), 0, st, b[0], b[1], K);
    LAUNCH_CHECK();
  }
  {  // P_raw = L_R E (M x kR), T1^T = R_R F^T (N x kL), T2 = F E (kL x kR)
    ThinBatch tb{};
    int n = 0;
    auto add = [&](const metis_q4& A, int64_t m, const uint4* bfrag, int splits, float* part) {
      tb.p[n] = ThinParams{A.codes, A.scales, bfrag, m, K, ceil_div<int64_t>(nks, splits), part};
      tb.gx[n] = ceil_div<int64_t>(m, kThinRows);
      tb.first[n + 1] = tb.first[n] + tb.gx[n] * splits;
      ++n;
    };
    if (R.k > 0) add(*L.res, M, w.bf_E, w.sa, w.pa);
    if (L.k > 0) add(*R.res, N, w.bf_F, w.s1, w.p1);
    if (L.k > 0 && R.k > 0) add(*L.kf, L.k, w.bf_E, w.s2, w.p2);
    for (int i = n; i < 3; ++i) tb.first[i + 1] = tb.first[i];
    if (tb.first[3] > INT32_MAX) return fail(METIS_E_UNSUPPORTED, "thin products too large");
    if (K % 32 == 0) hipLaunchKernelGGL(gemm_thin_kernel<true>, dim3((unsigned)tb.first[3]), dim3(256), 0, st, tb);
    else hipLaunchKernelGGL(gemm_thin_kernel<false>, dim3((unsigned)tb.first[3]), dim3(256), 0, st, tb);
    LAUNCH_CHECK();
  }
  if (L.k > 0 && R.k > 0) {  // T2 summed over its splits
    const int64_t n2 = (int64_t)L.k * 64;
    hipLaunchKernelGGL(sum_parts_kernel, dim3(grid1(n2 / 8, 256)), dim3(256), 0, st, w.p2, w.s2, n2, w.t2);
    LAUNCH_CHECK();
  }
  const int64_t kext = w.kext;
  ExtParams e{};
  e.rows = M;
  e.cols = N;
  e.kR = R.k;
  e.kL = L.k;
  e.ksR = w.ksR;
  e.ksL = w.ksL;
  e.kext = kext;
  e.praw = w.pa;
  e.t1 = w.p1;
  e.t2 = w.t2;
  e.sa = w.sa;
  e.s1 = w.s1;
  e.S_R = R.k > 0 ? R.S : w.ones;
  e.S_L = L.k > 0 ? L.S : w.ones;
  e.s_LR = L.res->tensor_scale;
  e.s_RR = R.res->tensor_scale;
  e.s_E = R.k > 0 ? R.kf->tensor_scale : w.ones;
  e.s_F = L.k > 0 ? L.kf->tensor_scale : w.ones;
  e.H = SplitSide{L.k > 0 ? L.out->codes : nullptr, L.k > 0 ? L.out->scales : nullptr,
                  L.k > 0 ? L.out->tensor_scale : w.ones, L.k, M};
  e.J = SplitSide{R.k > 0 ? R.out->codes : nullptr, R.k > 0 ? R.out->scales : nullptr,
                  R.k > 0 ? R.out->tensor_scale : w.ones, R.k, N};
  e.a_ext = w.a_ext;
  e.b_ext = w.b_ext;
  // A_ext: at most 512 looping workgroups (with B_ext's static LDS a CU
  // holds four of the launch's workgroups)
  const int64_t nba = std::min<int64_t>(grid1(round_up64(M, 32) * (kext / 8), 256), 512);
  const int64_t nbb = ceil_div<int64_t>(round_up64(N, 32), 64);
  if (nba + nbb > INT32_MAX) return fail(METIS_E_UNSUPPORTED, "K-extension too large");
  hipLaunchKernelGGL(ext_prep_kernel, dim3((unsigned)(nba + nbb)), dim3(256), 0, st, e, nba);
  LAUNCH_CHECK();
  return METIS_OK;
}

// Phases of a split product: the K-extension (written into the workspace)
// and the main GEMM that reads it.  Both phases carve the workspace alike,
// so they can be issued by separate calls.
enum SplitPhase { kPhaseExt = 1, kPhaseMain = 2, kPhaseAll = 3 };

// out (M x N) = L-hat R-hat with L = H S_L F^T + L_R, R^T = E S_R J^T + R_R^T
// along K.
metis_status split_product(const SideQ& L, const SideQ& R, int64_t M, int64_t N, int64_t K,
                           float* C, int64_t ldc, void* ws, size_t ws_bytes, hipStream_t st,
                           int phase = kPhaseAll) {
  if (L.k > 64 || R.k > 64) return fail(METIS_E_UNSUPPORTED, "split product rank above 64");
  Carver cv(ws, ws_bytes);
  SplitWs w = carve_split(cv, M, N, K, L.k, R.k);
  if (cv.used() > ws_bytes) return fail(METIS_E_WORKSPACE, "workspace %zu < %zu", ws_bytes, cv.used());
  const int64_t kext = (L.k > 0 || R.k > 0) ? w.kext : 0;
  metis_status s;
  if (phase & kPhaseExt) {
    if ((s = split_ext(L, R, M, N, K, w, st)) != METIS_OK) return s;
  }
  if (!(phase & kPhaseMain)) return METIS_OK;
  GemmParams g{M, N, K, L.res->codes, L.res->scales, R.res->codes, R.res->scales,
               L.res->tensor_scale, R.res->tensor_scale, kext, w.a_ext, w.b_ext, C, ldc};
  TimingRec* tr = timing_begin(st, 0, M, N, K, kext);
  s = launch_gemm(g, st);
  timing_end(tr, st);
  return s;
}

size_t split_ws_size(int64_t M, int64_t N, int64_t K, int kL, int kR) {
  Carver cv(nullptr, 0);
  carve_split(cv, M, N, K, kL, kR);
  return cv.used();
}

bool qop_has(const metis_qoperand* q, int axis) {
  const metis_q4& r = axis == 0 ? q->R_ax0 : q->R_ax1;
  const int64_t n_outer = axis == 0 ? q->cols : q->rows;
  const int64_t k_len = axis == 0 ? q->rows : q->cols;
  return q4_ok(r, n_outer, k_len);
}

bool qop_factors_ok(const metis_qoperand* q) {
  if (q->k == 0) return true;
  if (q->k < 0 || q->k > kMaxN || !q->S) return false;
  return q4_ok(q->U, q->k, q->rows) && q4_ok(q->V, q->k, q->cols);
}

// One decomposition call, checked and with its workspace carved.
struct DecompCall {
  const void* M;
  int32_t dtype;
  int64_t rows, cols, ld;
  const metis_config* cfg;
  bool sample;
  uint32_t tag;
  int64_t step;
  metis_factors* f;
  int k, n;
  int64_t lr;
  bool refresh;
  DecompWs w;
};

metis_status decompose_check(const void* M, int32_t dtype, int64_t rows, int64_t cols, int64_t ld,
                             const metis_config* cfg, int32_t sample_rows, uint32_t tag, int64_t step,
                             metis_factors* f, DecompCall* c) {
  metis_status s = validate_config(cfg);
  if (s != METIS_OK) return s;
  if (!M || !f || !f->U || !f->S || !f->V) return fail(METIS_E_INVALID, "NULL pointer argument");
  if (!dtype_ok(dtype)) return fail(METIS_E_INVALID, "dtype=%d", dtype);
  if (rows <= 0 || cols <= 0 || ld < cols) return fail(METIS_E_INVALID, "bad shape %lldx%lld ld=%lld",
                                                      (long long)rows, (long long)cols, (long long)ld);
  // rows and cols below 2^30: the rediagonalisation's sign keys hold a row
  // index in 31 bits and its tail launches one workgroup per 64 rows of U
  // and of V
  if (rows > (1LL << 30) || cols > (1LL << 30))
    return fail(METIS_E_UNSUPPORTED, "rows or cols above 2^30");
  // the sampler resolves its boundary histogram bin among at most kCandMax
  // candidate rows; 2^27 rows put 2048 rows in a bin on average
  if (sample_rows && rows > (int64_t)kCandMax * 65536 / 2)
    return fail(METIS_E_UNSUPPORTED, "row sample of %lld rows: at most %lld", (long long)rows,
                (long long)kCandMax * 65536 / 2);
  if (f->rows != rows || f->cols != cols || f->k != cfg->k)
    return fail(METIS_E_INVALID, "factors describe %lldx%lld k=%d, operand %lldx%lld k=%d",
                (long long)f->rows, (long long)f->cols, f->k, (long long)rows, (long long)cols, cfg->k);
  const int n = cfg->k + cfg->s;
  const bool sample = sample_rows != 0;
  const int64_t lr = sample ? cfg->l_k : rows;
  if (sample && (cfg->l_k <= 0 || cfg->l_k > rows))
    return fail(METIS_E_INVALID, "l_k=%lld outside (0, rows=%lld]", (long long)cfg->l_k, (long long)rows);
  if (n > lr || n > cols)
    return fail(METIS_E_INVALID, "k + s = %d exceeds min(l_k or rows, cols)", n);
  if (step < 0 || step > UINT32_MAX) return fail(METIS_E_INVALID, "step=%lld", (long long)step);
  *c = DecompCall{M, dtype, rows, cols, ld, cfg, sample, tag, step, f, cfg->k, n, lr,
                  f->refreshed_at < 0 || step - f->refreshed_at >= cfg->refresh, DecompWs{}};
  return METIS_OK;
}

// One CholeskyQR pass after its Gram: Rinv from the Cholesky factor, then
// dst = src Rinv, with LDS sized to the sketch width n.
template <int NM>
void cholqr_pass(const double* g, int n, int64_t lr, int pass, double* rinv, const float* src, float* dst,
                 hipStream_t st) {
  hipLaunchKernelGGL(cholinv_kernel<NM>, dim3(1), dim3(256), 0, st, g, n, lr, pass, rinv);
  hipLaunchKernelGGL(apply_rinv_kernel<NM>, dim3(grid1(lr, kApplyRows)), dim3(256), 0, st, src, lr, n, rinv, dst);
}

void launch_cholqr_pass(const double* g, int n, int64_t lr, int pass, double* rinv, const float* src, float* dst,
                        hipStream_t st) {
  if (n <= 32) cholqr_pass<32>(g, n, lr, pass, rinv, src, dst, st);
  else if (n <= 64) cholqr_pass<64>(g, n, lr, pass, rinv, src, dst, st);
  else if (n <= 72) cholqr_pass<72>(g, n, lr, pass, rinv, src, dst, st);
  else cholqr_pass<kMaxN>(g, n, lr, pass, rinv, src, dst, st);
}

// The sketch on refresh steps (V from the range of a row sample of M), then
// the projection P = M V and its Gram matrix G = P^T P.
metis_status decompose_project(DecompCall& c, hipStream_t st, TimingRec** t_proj = nullptr) {
  metis_status s;
  const void* M = c.M;
  const int32_t dtype = c.dtype;
  const int64_t rows = c.rows, cols = c.cols, ld = c.ld;
  const metis_config* cfg = c.cfg;
  const bool sample = c.sample;
  const uint32_t tag = c.tag;
  metis_factors* f = c.f;
  const int k = c.k, n = c.n;
  const int64_t lr = c.lr;
  DecompWs& w = c.w;
  const uint32_t ustep = (uint32_t)c.step;
  // bf16 rows on 16-byte boundaries with whole 64-column K blocks take MFMA
  const bool mfma_ok = dtype == METIS_BF16 && cols % 64 == 0 && ld % 8 == 0 && ((uintptr_t)M & 15) == 0;

  if (c.refresh) {
    TimingRec* t_sk = timing_begin(st, 4, rows, cols, n, lr);
    const float scale = sample ? (float)sqrt((double)rows / (double)lr) : 1.0f;
    if (sample) {
      const uint32_t tag_s = tag_with_role(tag, kRoleSample);
      hipLaunchKernelGGL(fill_u32_kernel, dim3(grid1(65536, 256)), dim3(256), 0, st, w.hist, 0u,
                         (int64_t)65536);
      LAUNCH_CHECK();
      hipLaunchKernelGGL(sample_keys_kernel, dim3(grid1(rows, 256)), dim3(256), 0, st, w.keys, w.hist,
                         rows, tag_s, ustep, cfg->seed);
      LAUNCH_CHECK();
      hipLaunchKernelGGL(sample_threshold_kernel, dim3(1), dim3(1024), 0, st, w.hist, w.meta, lr);
      LAUNCH_CHECK();
      hipLaunchKernelGGL(sample_mark_kernel, dim3(grid1(rows, 256)), dim3(256), 0, st, w.keys, w.meta,
                         w.flags, w.cand, rows);
      LAUNCH_CHECK();
      hipLaunchKernelGGL(sample_resolve_kernel, dim3(1), dim3(1024), 0, st, w.meta, w.cand, w.flags);
      LAUNCH_CHECK();
      hipLaunchKernelGGL(sample_compact_kernel, dim3(1), dim3(1024), 0, st, w.flags, rows, lr, w.idx);
      LAUNCH_CHECK();
    } else {
      hipLaunchKernelGGL(iota_kernel, dim3(grid1(rows, 256)), dim3(256), 0, st, w.idx, rows);
      LAUNCH_CHECK();
    }
    hipLaunchKernelGGL(omega_kernel, dim3(grid1(ceil_div<int64_t>(cols * n, 8), 256)), dim3(256), 0,
                       st, w.om, cols, n, tag_with_role(tag, kRoleOmega), ustep, cfg->seed);
    LAUNCH_CHECK();
    if (mfma_ok) {
      // Omega's entries are bf16 values: one term is exact
      if ((s = mfma_product<1>((const uint16_t*)M, ld, lr, w.idx, w.om, cols, n, n, w.proj_nkb, w.sk_kbps,
                               w.sk_splits, scale, w.ofrag, w.spart, w.y, st)) != METIS_OK)
        return s;
    } else {
      hipLaunchKernelGGL(sketch_y_kernel, dim3(grid1(lr, 32)), dim3(256), 0, st, M, dtype, ld, w.idx,
                         lr, cols, w.om, n, scale, w.y);
      LAUNCH_CHECK();
    }
    float* src = w.y;
    float* dst = w.q;
    for (int pass = 0; pass < 3; ++pass) {
      if ((s = launch_gram(src, lr, n, n, 1, w.gblocks, w.gpart, w.g, st)) != METIS_OK) return s;
      launch_cholqr_pass(w.g, n, lr, pass, w.rinv, src, dst, st);
      LAUNCH_CHECK();
      float* t = src;  // next pass reads what was just written
      src = dst;
      dst = t;
    }
    const float* Q = src;
    hipLaunchKernelGGL(sketch_b_kernel, dim3(grid1(cols, kSkbCols), w.slices), dim3(256), 0, st, M, dtype, ld,
                       w.idx, lr, cols, Q, n, w.rows_per_slice, w.bpart);
    LAUNCH_CHECK();
    hipLaunchKernelGGL(reduce_slices_kernel, dim3(grid1((int64_t)n * cols, 256)), dim3(256), 0, st,
                       w.bpart, w.slices, (int64_t)n * cols, scale, w.b);
    LAUNCH_CHECK();
    if ((s = launch_gram(w.b, cols, n, 1, cols, w.gblocks, w.gpart, w.g, st)) != METIS_OK) return s;
    launch_jacobi(w.g, n, w.theta, w.z, nullptr, st);
    LAUNCH_CHECK();
    hipLaunchKernelGGL(sketch_v_kernel, dim3(grid1(cols * k, 256)), dim3(256), 0, st, w.b, cols, n, k,
                       w.z, w.theta, f->V);
    LAUNCH_CHECK();
    timing_end(t_sk, st);
  }

  // projection and rediagonalisation (every step); V as three bf16 terms
  if (t_proj) *t_proj = timing_begin(st, 5, rows, cols, k, c.refresh ? 1 : 0);
  if (mfma_ok) {
    // the split reduction into P happens inside the Gram kernel
    if ((s = mfma_product<3>((const uint16_t*)M, ld, rows, nullptr, f->V, cols, k, k, w.proj_nkb, w.proj_kbps,
                             w.proj_splits, 1.0f, w.vfrag, w.ppart, w.p, st, false)) != METIS_OK)
      return s;
    return launch_gram_from_parts(w.ppart, w.proj_splits, mfma_part_pitch(k), 1.0f, w.p, rows, k, w.gblocks,
                                  w.gpart, w.ptp, st);
  }
  hipLaunchKernelGGL(project_kernel, dim3(grid1(rows, 64)), dim3(256), 0, st, M, dtype, ld, rows, cols, f->V, k,
                     w.p);
  LAUNCH_CHECK();
  if ((s = launch_gram(w.p, rows, k, k, 1, w.gblocks, w.gpart, w.ptp, st)) != METIS_OK) return s;
  return METIS_OK;
}

// Rediagonalisation: eig(G) = R Lambda R^T, V <- V R, U = P R Lambda^-1/2,
// S = Lambda^1/2, columns signed so that the largest-magnitude entry of each
// V column (lowest row on ties) is positive, in descending order.  With
// amax_u / amax_v given (zeroed words), the tensor amax of the new U and V
// lands there, so quantising the factors needs no amax sweep of its own.
metis_status decompose_rediag(DecompCall& c, hipStream_t st, uint32_t* amax_u = nullptr,
                              uint32_t* amax_v = nullptr) {
  const int64_t rows = c.rows, cols = c.cols;
  const int k = c.k;
  metis_factors* f = c.f;
  DecompWs& w = c.w;
  launch_jacobi(w.ptp, k, w.lam, w.rot, w.key, st);
  LAUNCH_CHECK();
  if (k <= 32)
    launch_rot<32>(w, f, rows, cols, k, amax_u, amax_v, st);
  else if (k <= 64)
    launch_rot<64>(w, f, rows, cols, k, amax_u, amax_v, st);
  else if (k <= 72)
    launch_rot<72>(w, f, rows, cols, k, amax_u, amax_v, st);
  else
    launch_rot<kMaxN>(w, f, rows, cols, k, amax_u, amax_v, st);
  LAUNCH_CHECK();
  return METIS_OK;
}

// Arguments of one quantisation, checked.
metis_status quantize_check(const void* M, int32_t dtype, int64_t rows, int64_t cols, int64_t ld,
                            const metis_factors* f, const metis_config* cfg, int64_t step, int32_t axes,
                            const metis_qoperand* out) {
  if (!M || !out || !cfg) return fail(METIS_E_INVALID, "NULL pointer argument");
  if (!dtype_ok(dtype)) return fail(METIS_E_INVALID, "dtype=%d", dtype);
  if (rows <= 0 || cols <= 0 || ld < cols) return fail(METIS_E_INVALID, "bad shape");
  if (cfg->rounding != METIS_RNE && cfg->rounding != METIS_SR)
    return fail(METIS_E_INVALID, "rounding=%d", cfg->rounding);
  if (axes <= 0 || axes > 3) return fail(METIS_E_INVALID, "axes=%d", axes);
  if (step < 0 || step > UINT32_MAX) return fail(METIS_E_INVALID, "step=%lld", (long long)step);
  if ((axes & METIS_AXIS0) && rows % 16) return fail(METIS_E_INVALID, "rows %% 16 != 0 for axis 0");
  if ((axes & METIS_AXIS1) && cols % 16) return fail(METIS_E_INVALID, "cols %% 16 != 0 for axis 1");
  if (out->rows != rows || out->cols != cols) return fail(METIS_E_INVALID, "out describes another shape");
  if ((axes & METIS_AXIS0) && !q4_ok(out->R_ax0, cols, rows))
    return fail(METIS_E_INVALID, "R_ax0 must be cols x rows/2 codes");
  if ((axes & METIS_AXIS1) && !q4_ok(out->R_ax1, rows, cols))
    return fail(METIS_E_INVALID, "R_ax1 must be rows x cols/2 codes");
  const int k = f ? f->k : 0;
  if (f) {
    if (!f->U || !f->S || !f->V || f->rows != rows || f->cols != cols || k < 1 || k > kMaxN)
      return fail(METIS_E_INVALID, "factors do not match the operand");
    if (rows % 16 || cols % 16) return fail(METIS_E_INVALID, "factor blocks need rows, cols %% 16 == 0");
    if (out->k != k || !q4_ok(out->U, k, rows) || !q4_ok(out->V, k, cols))
      return fail(METIS_E_INVALID, "out->U / out->V must be k x rows/2 and k x cols/2");
  } else if (out->k != 0) {
    return fail(METIS_E_INVALID, "out->k must be 0 for direct quantisation");
  }
  return METIS_OK;
}

// Quantiser parameters of the residual (or direct) sweeps.
QuantParams resid_params(const void* M, int32_t dtype, int64_t rows, int64_t cols, int64_t ld,
                         const metis_config* cfg, uint32_t tag, int64_t step, int32_t axes,
                         metis_qoperand* out, float* residual_out, const QuantWs& w) {
  QuantParams qp{};
  qp.M = M;
  qp.dtype = dtype;
  qp.rows = rows;
  qp.cols = cols;
  qp.ld = ld;
  qp.amax = w.amax;
  qp.amax_slots = w.amax + kAmaxSlotStride;
  qp.axes = axes;
  qp.sr = cfg->rounding == METIS_SR;
  qp.seed = cfg->seed;
  // both orientations round each element with its draw at its row-major
  // position in M
  qp.tag0 = qp.tag1 = tag_with_role(tag, kRoleResid);
  qp.shared_draws = 1;
  qp.step = (uint32_t)step;
  qp.resid = residual_out;
  if (axes & METIS_AXIS0) {
    qp.codes0 = out->R_ax0.codes;
    qp.scales0 = out->R_ax0.scales;
    qp.sg0 = out->R_ax0.tensor_scale;
  }
  if (axes & METIS_AXIS1) {
    qp.codes1 = out->R_ax1.codes;
    qp.scales1 = out->R_ax1.scales;
    qp.sg1 = out->R_ax1.tensor_scale;
  }
  return qp;
}

// NVFP4 codes of the factors U (rows x k) and V (cols x k), blocked along
// their rows; out->S = f->S.
metis_status quantize_factors(const metis_factors* f, int64_t rows, int64_t cols, const metis_config* cfg,
                              uint32_t tag, int64_t step, metis_qoperand* out, const QuantWs& w,
                              hipStream_t st, bool amax_ready = false) {
  const int k = f->k;
  QuantParams qp{};
  qp.sr = cfg->rounding == METIS_SR;
  {
    // factors: U (rows x k) and V (cols x k), blocked along their rows, both
    // in one launch per sweep
    QuantParams fqs[2];
    for (int which = 0; which < 2; ++which) {
      QuantParams& fq = fqs[which];
      fq = QuantParams{};
      const int64_t fr = which == 0 ? rows : cols;
      const metis_q4& o = which == 0 ? out->U : out->V;
      fq.M = which == 0 ? (const void*)f->U : (const void*)f->V;
      fq.dtype = METIS_F32;
      fq.rows = fr;
      fq.cols = k;
      fq.ld = k;
      fq.amax = w.amax + 1 + which;
      fq.axes = METIS_AXIS0;
      fq.sr = qp.sr;
      fq.seed = cfg->seed;
      fq.tag0 = tag_with_role(tag, which == 0 ? kRoleU : kRoleV);
      fq.step = (uint32_t)step;
      fq.codes0 = o.codes;
      fq.scales0 = o.scales;
      fq.sg0 = o.tensor_scale;
      fq.tiles_per_wg = 1;
    }
    const int64_t pu = ceil_div<int64_t>(rows, kQT_R), pv = ceil_div<int64_t>(cols, kQT_R);
    const dim3 grid((unsigned)(pu + pv), (unsigned)ceil_div<int64_t>(k, kQT_C));
    if (pu + pv > INT32_MAX) return fail(METIS_E_UNSUPPORTED, "operand too large");
    if (!amax_ready) {  // else the rediagonalisation left the amax of U and V in w.amax[1], [2]
      TimingRec* t1 = timing_begin(st, 1, rows + cols, k, METIS_AXIS0, 0);
      hipLaunchKernelGGL(quant_amax_pair_kernel, grid, dim3(kQThreads), 0, st, fqs[0], fqs[1], (int)pu);
      LAUNCH_CHECK();
      timing_end(t1, st);
    }
    TimingRec* t2 = timing_begin(st, 2, rows + cols, k, METIS_AXIS0, 0);
    if (qp.sr)
      hipLaunchKernelGGL(quant_pair_kernel<true>, grid, dim3(kQThreads), 0, st, fqs[0], fqs[1], (int)pu);
    else
      hipLaunchKernelGGL(quant_pair_kernel<false>, grid, dim3(kQThreads), 0, st, fqs[0], fqs[1], (int)pu);
    LAUNCH_CHECK();
    timing_end(t2, st);
    if (out->S && out->S != f->S) {
      hipLaunchKernelGGL(copy_f32_kernel, dim3(1), dim3(128), 0, st, f->S, out->S, (int64_t)k);
      LAUNCH_CHECK();
    } else {
      out->S = f->S;
    }
  }
  return METIS_OK;
}

// Reusable events for the fork/join of metis_prepare_operand (an event may
// be recorded again once the waits on its previous record are enqueued).
std::mutex g_evmu;
std::vector<hipEvent_t> g_evpool;

metis_status take_event(hipEvent_t* e) {
  {
    std::lock_guard<std::mutex> lk(g_evmu);
    if (!g_evpool.empty()) {
      *e = g_evpool.back();
      g_evpool.pop_back();
      return METIS_OK;
    }
  }
  const hipError_t err = hipEventCreateWithFlags(e, hipEventDisableTiming);
  return err == hipSuccess ? METIS_OK : fail(METIS_E_HIP, "hipEventCreate: %s", hipGetErrorString(err));
}

void give_event(hipEvent_t e) {
  std::lock_guard<std::mutex> lk(g_evmu);
  g_evpool.push_back(e);
}

// `waiter` waits for everything issued to `from` so far.
metis_status stream_after(hipStream_t waiter, hipStream_t from, hipEvent_t e) {
  hipError_t err = hipEventRecord(e, from);
  if (err == hipSuccess) err = hipStreamWaitEvent(waiter, e, 0);
  return err == hipSuccess ? METIS_OK : fail(METIS_E_HIP, "stream order: %s", hipGetErrorString(err));
}

}  // namespace

// =================================================================== ABI ===

// Y = X-hat W-hat, whole or one phase (the main phase reads the K-extension
// an earlier extension phase wrote into the same workspace).
metis_status gemm_fwd_call(const metis_qoperand* X, const metis_qoperand* W, float* Y, int64_t ldy, void* ws,
                           size_t ws_bytes, void* stream, int phase) {
  if (!X || !W || ((phase & kPhaseMain) && !Y)) return fail(METIS_E_INVALID, "NULL pointer argument");
  if (X->cols != W->rows) return fail(METIS_E_INVALID, "inner dimensions differ (%lld vs %lld)",
                                      (long long)X->cols, (long long)W->rows);
  if ((phase & kPhaseMain) && ldy < W->cols) return fail(METIS_E_INVALID, "ldy < n");
  if (!qop_has(X, 1)) return fail(METIS_E_INVALID, "X lacks its residual along m (R_ax1)");
  if (!qop_has(W, 0)) return fail(METIS_E_INVALID, "W lacks its residual along m (R_ax0)");
  if (!qop_factors_ok(X) || !qop_factors_ok(W)) return fail(METIS_E_INVALID, "bad factor descriptors");
  const SideQ L{&X->R_ax1, &X->U, &X->V, X->S, X->k};
  const SideQ R{&W->R_ax0, &W->V, &W->U, W->S, W->k};
  return split_product(L, R, X->rows, W->cols, X->cols, Y, ldy, ws, ws_bytes, (hipStream_t)stream, phase);
}

// Workspace bytes of the dX product; the dW product's region follows it.
size_t bwd_dx_region(const metis_qoperand* D, const metis_qoperand* W) {
  return round_up64((int64_t)split_ws_size(D->rows, W->rows, D->cols, D->k, W->k), 256);
}

// dX = D-hat W-hat^T and dW = X-hat^T D-hat, whole or one phase.
metis_status gemm_bwd_call(const metis_qoperand* D, const metis_qoperand* W, const metis_qoperand* X, bool do_dx,
                           float* dX, int64_t lddx, bool do_dw, float* dW, int64_t lddw, void* ws,
                           size_t ws_bytes, void* stream, int phase) {
  if (!D || !W || !X) return fail(METIS_E_INVALID, "NULL pointer argument");
  if (D->cols != W->cols || D->rows != X->rows || X->cols != W->rows)
    return fail(METIS_E_INVALID, "shapes of D, W, X do not form a linear layer");
  if (!qop_factors_ok(D) || !qop_factors_ok(W) || !qop_factors_ok(X))
    return fail(METIS_E_INVALID, "bad factor descriptors");
  hipStream_t st = (hipStream_t)stream;
  const bool main = (phase & kPhaseMain) != 0;
  const size_t off = bwd_dx_region(D, W);
  metis_status s;
  if (do_dx) {
    if (main && lddx < W->rows) return fail(METIS_E_INVALID, "lddx < m");
    if (!qop_has(D, 1) || !qop_has(W, 1)) return fail(METIS_E_INVALID, "dX needs D and W along n (R_ax1)");
    const SideQ L{&D->R_ax1, &D->U, &D->V, D->S, D->k};
    const SideQ R{&W->R_ax1, &W->U, &W->V, W->S, W->k};
    if ((s = split_product(L, R, D->rows, W->rows, D->cols, dX, lddx, ws, ws_bytes, st, phase)) != METIS_OK)
      return s;
  }
  if (do_dw) {
    if (main && lddw < D->cols) return fail(METIS_E_INVALID, "lddw < n");
    if (!qop_has(X, 0) || !qop_has(D, 0)) return fail(METIS_E_INVALID, "dW needs X and D along l (R_ax0)");
    if (ws_bytes < off) return fail(METIS_E_WORKSPACE, "workspace %zu < %zu", ws_bytes, off);
    const SideQ L{&X->R_ax0, &X->V, &X->U, X->S, X->k};
    const SideQ R{&D->R_ax0, &D->V, &D->U, D->S, D->k};
    if ((s = split_product(L, R, X->cols, D->cols, X->rows, dW, lddw, (uint8_t*)ws + off, ws_bytes - off, st,
                           phase)) != METIS_OK)
      return s;
  }
  return METIS_OK;
}

extern "C" {

int32_t metis_abi_version(void) { return METIS_ABI_VERSION; }

const char* metis_last_error(void) { return g_last_error.c_str(); }

metis_status metis_init_device(void) { return ensure_device_tables(); }

void metis_omega_table(uint16_t* out65536) {
  if (out65536) memcpy(out65536, host_omega_table(), 65536 * sizeof(uint16_t));
}

void metis_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  const Philox4 b = philox4x32_10(ctr[0], ctr[1], ctr[2], ctr[3], key[0], key[1]);
  for (int i = 0; i < 4; ++i) out[i] = b.v[i];
}

size_t metis_decompose_workspace(int64_t rows, int64_t cols, const metis_config* cfg,
                                 int32_t sample_rows) {
  if (!cfg || rows <= 0 || cols <= 0 || cfg->k < 1) return 0;
  const int n = cfg->k + cfg->s;
  const int64_t lr = sample_rows ? cfg->l_k : rows;
  Carver cv(nullptr, 0);
  carve_decompose(cv, rows, cols, cfg->k, n, lr, sample_rows != 0);
  return cv.used();
}

size_t metis_quantize_workspace(int64_t rows, int64_t cols, int32_t k) {
  Carver cv(nullptr, 0);
  carve_quantize(cv, rows, cols, k);
  return cv.used();
}

size_t metis_gemm_fwd_workspace(const metis_qoperand* X, const metis_qoperand* W) {
  if (!X || !W) return 0;
  return split_ws_size(X->rows, W->cols, X->cols, X->k, W->k);
}

size_t metis_gemm_bwd_workspace(const metis_qoperand* D, const metis_qoperand* W,
                                const metis_qoperand* X) {
  if (!D || !W || !X) return 0;
  return bwd_dx_region(D, W) + split_ws_size(X->cols, D->cols, X->rows, X->k, D->k);
}

metis_status metis_decompose(const void* M, int32_t dtype, int64_t rows, int64_t cols, int64_t ld,
                             const metis_config* cfg, int32_t sample_rows, uint32_t tag,
                             int64_t step, metis_factors* f, void* ws, size_t ws_bytes,
                             void* stream) {
  DecompCall c;
  metis_status s = decompose_check(M, dtype, rows, cols, ld, cfg, sample_rows, tag, step, f, &c);
  if (s != METIS_OK) return s;
  Carver cv(ws, ws_bytes);
  c.w = carve_decompose(cv, rows, cols, c.k, c.n, c.lr, c.sample);
  if (!ws || cv.used() > ws_bytes)
    return fail(METIS_E_WORKSPACE, "workspace %zu < %zu", ws_bytes, cv.used());
  if ((s = ensure_device_tables()) != METIS_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  TimingRec* t_proj = nullptr;
  if ((s = decompose_project(c, st, &t_proj)) != METIS_OK) return s;
  if ((s = decompose_rediag(c, st)) != METIS_OK) return s;
  timing_end(t_proj, st);
  if (c.refresh) f->refreshed_at = step;
  return METIS_OK;
}

}  // extern "C"

namespace {

// metis_quantize after its checks, with the workspace carved.
metis_status quantize_body(const void* M, int32_t dtype, int64_t rows, int64_t cols, int64_t ld,
                           const metis_factors* f, const metis_config* cfg, uint32_t tag, int64_t step,
                           int32_t axes, metis_qoperand* out, float* residual_out, const QuantWs& w,
                           hipStream_t st) {
  metis_status s;
  const int k = f ? f->k : 0;
  QuantParams qp = resid_params(M, dtype, rows, cols, ld, cfg, tag, step, axes, out, residual_out, w);
  if (!f) {
    hipLaunchKernelGGL(fill_u32_kernel, dim3(grid1(kAmaxWords, 256)), dim3(256), 0, st, w.amax, 0u, kAmaxWords);
    LAUNCH_CHECK();
  } else {
    // fragments of U S and V, pre-scale from S[0], amax words cleared
    const int kp = round_up(k, 16);
    const ResidPrep rp{f->U, f->S, f->V, nullptr, rows, cols, k, kp, w.pscale, w.ucat, w.vcat, w.amax,
                       (int)kAmaxWords};
    hipLaunchKernelGGL(resid_prep_kernel, dim3(grid1(resid_prep_threads(rows, cols, kp), 256)), dim3(256), 0, st,
                       rp);
    LAUNCH_CHECK();
    qp.ucat = w.ucat;
    qp.vcat = w.vcat;
    qp.kc = 3 * kp;
    qp.pscale = w.pscale;
  }
  if ((s = run_quant(qp, f != nullptr, rows, cols, st)) != METIS_OK) return s;
  if (f) return quantize_factors(f, rows, cols, cfg, tag, step, out, w, st);
  return METIS_OK;
}

}  // namespace

extern "C" {

metis_status metis_quantize(const void* M, int32_t dtype, int64_t rows, int64_t cols, int64_t ld,
                            const metis_factors* f, const metis_config* cfg, uint32_t tag,
                            int64_t step, int32_t axes, metis_qoperand* out, float* residual_out,
                            void* ws, size_t ws_bytes, void* stream) {
  metis_status s = quantize_check(M, dtype, rows, cols, ld, f, cfg, step, axes, out);
  if (s != METIS_OK) return s;
  const int k = f ? f->k : 0;
  Carver cv(ws, ws_bytes);
  QuantWs w = carve_quantize(cv, rows, cols, k);
  if (!ws || cv.used() > ws_bytes) return fail(METIS_E_WORKSPACE, "workspace %zu < %zu", ws_bytes, cv.used());
  if ((s = ensure_device_tables()) != METIS_OK) return s;
  return quantize_body(M, dtype, rows, cols, ld, f, cfg, tag, step, axes, out, residual_out, w,
                       (hipStream_t)stream);
}

size_t metis_quantize_static_capacity(void) { return kStaticScratchBytes; }

metis_status metis_quantize_static(const void* M, int32_t dtype, int64_t rows, int64_t cols, int64_t ld,
                                   const metis_factors* f, const metis_config* cfg, uint32_t tag, int64_t step,
                                   int32_t axes, metis_qoperand* out, float* residual_out, void* stream) {
  metis_status s = quantize_check(M, dtype, rows, cols, ld, f, cfg, step, axes, out);
  if (s != METIS_OK) return s;
  const int k = f ? f->k : 0;
  Carver probe(nullptr, 0);
  carve_quantize(probe, rows, cols, k);
  if (probe.used() > kStaticScratchBytes)
    return fail(METIS_E_UNSUPPORTED,
                "quantize_static: this operand (%lld x %lld, k = %d) needs %zu bytes of scratch; the static "
                "scratch holds %zu (use metis_quantize with a workspace)",
                (long long)rows, (long long)cols, k, probe.used(), kStaticScratchBytes);
  if ((s = ensure_device_tables()) != METIS_OK) return s;
  void* base = device_scratch();
  if (!base) return fail(METIS_E_HIP, "quantize_static: no scratch address for the current device");
  Carver cv(base, kStaticScratchBytes);
  QuantWs w = carve_quantize(cv, rows, cols, k);
  return quantize_body(M, dtype, rows, cols, ld, f, cfg, tag, step, axes, out, residual_out, w,
                       (hipStream_t)stream);
}

size_t metis_prepare_operand_workspace(int64_t rows, int64_t cols, const metis_config* cfg,
                                       int32_t sample_rows) {
  if (!cfg || rows <= 0 || cols <= 0 || cfg->k < 1 || cfg->k > kMaxN || cfg->s < 0) return 0;
  const int n = cfg->k + cfg->s;
  const int64_t lr = sample_rows ? cfg->l_k : rows;
  Carver cv(nullptr, 0);
  carve_decompose(cv, rows, cols, cfg->k, n, lr, sample_rows != 0);
  carve_quantize(cv, rows, cols, cfg->k);
  return cv.used();
}

metis_status metis_prepare_operand(const void* M, int32_t dtype, int64_t rows, int64_t cols, int64_t ld,
                                   const metis_config* cfg, int32_t sample_rows, uint32_t tag, int64_t step,
                                   metis_factors* f, int32_t axes, metis_qoperand* out, float* residual_out,
                                   void* ws, size_t ws_bytes, void* stream, void* side_stream) {
  DecompCall c;
  metis_status s = decompose_check(M, dtype, rows, cols, ld, cfg, sample_rows, tag, step, f, &c);
  if (s != METIS_OK) return s;
  if ((s = quantize_check(M, dtype, rows, cols, ld, f, cfg, step, axes, out)) != METIS_OK) return s;
  const int k = c.k;
  Carver cv(ws, ws_bytes);
  c.w = carve_decompose(cv, rows, cols, k, c.n, c.lr, c.sample);
  QuantWs qw = carve_quantize(cv, rows, cols, k);
  if (!ws || cv.used() > ws_bytes)
    return fail(METIS_E_WORKSPACE, "workspace %zu < %zu", ws_bytes, cv.used());
  if ((s = ensure_device_tables()) != METIS_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  hipStream_t st2 = side_stream ? (hipStream_t)side_stream : st;
  const bool fork = st2 != st;

  // P = M V_old and G = P^T P (the sketch first on refresh steps)
  if ((s = decompose_project(c, st)) != METIS_OK) return s;
  // the residual's rank-k product from P and V_old, before V is rotated
  // (pre-scale from the Gram diagonal), with the amax words cleared
  const int kp = round_up(k, 16);
  const ResidPrep rp{c.w.p, nullptr, f->V, c.w.ptp, rows, cols, k, kp, qw.pscale, qw.ucat, qw.vcat, qw.amax,
                     (int)kAmaxWords};
  hipLaunchKernelGGL(resid_prep_kernel, dim3(grid1(resid_prep_threads(rows, cols, kp), 256)), dim3(256), 0, st,
                     rp);
  LAUNCH_CHECK();
  QuantParams qp = resid_params(M, dtype, rows, cols, ld, cfg, tag, step, axes, out, residual_out, qw);
  qp.ucat = qw.ucat;
  qp.vcat = qw.vcat;
  qp.kc = 3 * kp;
  qp.pscale = qw.pscale;

  hipEvent_t e_fork = nullptr, e_join = nullptr;
  if (fork) {
    if ((s = take_event(&e_fork)) != METIS_OK) return s;
    if ((s = take_event(&e_join)) != METIS_OK) {
      give_event(e_fork);
      return s;
    }
    if ((s = stream_after(st2, st, e_fork)) != METIS_OK) {
      give_event(e_fork);
      give_event(e_join);
      return s;
    }
  }
  // rediagonalisation on the side stream (with the factors' amax into the
  // words zeroed above), residual sweeps on the main stream
  s = decompose_rediag(c, st2, qw.amax + 1, qw.amax + 2);
  if (s == METIS_OK) s = run_quant(qp, true, rows, cols, st);
  if (fork) {
    const metis_status sj = stream_after(st, st2, e_join);
    if (s == METIS_OK) s = sj;
    give_event(e_fork);
    give_event(e_join);
  }
  if (s != METIS_OK) return s;
  if ((s = quantize_factors(f, rows, cols, cfg, tag, step, out, qw, st, true)) != METIS_OK) return s;
  if (c.refresh) f->refreshed_at = step;
  return METIS_OK;
}

metis_status metis_gemm_fwd(const metis_qoperand* X, const metis_qoperand* W, float* Y, int64_t ldy,
                            void* ws, size_t ws_bytes, void* stream) {
  return gemm_fwd_call(X, W, Y, ldy, ws, ws_bytes, stream, kPhaseAll);
}

metis_status metis_gemm_fwd_prepare(const metis_qoperand* X, const metis_qoperand* W, void* ws,
                                    size_t ws_bytes, void* stream) {
  return gemm_fwd_call(X, W, nullptr, 0, ws, ws_bytes, stream, kPhaseExt);
}

metis_status metis_gemm_fwd_prepared(const metis_qoperand* X, const metis_qoperand* W, float* Y, int64_t ldy,
                                     void* ws, size_t ws_bytes, void* stream) {
  return gemm_fwd_call(X, W, Y, ldy, ws, ws_bytes, stream, kPhaseMain);
}

metis_status metis_gemm_bwd(const metis_qoperand* D, const metis_qoperand* W, const metis_qoperand* X,
                            float* dX, int64_t lddx, float* dW, int64_t lddw, void* ws,
                            size_t ws_bytes, void* stream) {
  return gemm_bwd_call(D, W, X, dX != nullptr, dX, lddx, dW != nullptr, dW, lddw, ws, ws_bytes, stream,
                       kPhaseAll);
}

metis_status metis_gemm_bwd_prepare(const metis_qoperand* D, const metis_qoperand* W, const metis_qoperand* X,
                                    int32_t which, void* ws, size_t ws_bytes, void* stream) {
  if (which <= 0 || which > (METIS_GRAD_DX | METIS_GRAD_DW)) return fail(METIS_E_INVALID, "which=%d", which);
  return gemm_bwd_call(D, W, X, (which & METIS_GRAD_DX) != 0, nullptr, 0, (which & METIS_GRAD_DW) != 0, nullptr,
                       0, ws, ws_bytes, stream, kPhaseExt);
}

metis_status metis_gemm_bwd_prepared(const metis_qoperand* D, const metis_qoperand* W, const metis_qoperand* X,
                                     float* dX, int64_t lddx, float* dW, int64_t lddw, void* ws,
                                     size_t ws_bytes, void* stream) {
  return gemm_bwd_call(D, W, X, dX != nullptr, dX, lddx, dW != nullptr, dW, lddw, ws, ws_bytes, stream,
                       kPhaseMain);
}

metis_status metis_timing_kinds(int32_t mask) {
  std::lock_guard<std::mutex> lk(g_tmu);
  g_tkinds = (uint32_t)mask;
  return METIS_OK;
}

metis_status metis_timing_enable(int32_t capacity) {
  std::lock_guard<std::mutex> lk(g_tmu);
  for (auto& r : g_trecs) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_trecs.clear();
  g_tused = 0;
  g_timing = capacity > 0;
  if (!g_timing) return METIS_OK;
  g_trecs.resize((size_t)capacity);
  for (auto& r : g_trecs) {
    HIP_TRY(hipEventCreate(&r.a));
    HIP_TRY(hipEventCreate(&r.b));
  }
  return METIS_OK;
}

int32_t metis_timing_read(float* ms, int64_t* shape, int32_t max_records) {
  std::lock_guard<std::mutex> lk(g_tmu);
  int32_t n = 0;
  for (size_t i = 0; i < g_tused && n < max_records; ++i, ++n) {
    TimingRec& r = g_trecs[i];
    float t = -1.0f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) t = -1.0f;
    ms[n] = t;
    shape[5 * n + 0] = r.kind;
    shape[5 * n + 1] = r.d0;
    shape[5 * n + 2] = r.d1;
    shape[5 * n + 3] = r.d2;
    shape[5 * n + 4] = r.d3;
  }
  g_tused = 0;
  return n;
}

metis_status metis_status_sync(void* stream) {
  HIP_TRY(hipStreamSynchronize((hipStream_t)stream));
  int v = 0;
  HIP_TRY(hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_metis_status), sizeof(int)));
  if (v != 0) {
    const int zero = 0;
    HIP_TRY(hipMemcpyToSymbol(HIP_SYMBOL(g_metis_status), &zero, sizeof(int)));
    return fail(METIS_E_NUMERIC, "device numeric status 0x%x (1: non-finite input, 2: Cholesky, 4: sampler)", v);
  }
  return METIS_OK;
}

// ------------------------------------------------------------- MXFP4 --

metis_status metis_mxfp4_quantize(const void* M, int32_t dtype, int64_t rows, int64_t cols, int64_t ld,
                                  int32_t axis, int32_t rounding, uint64_t seed, uint32_t tag, int64_t step,
                                  uint8_t* codes, uint8_t* scales, void* stream) {
  if (!M || !codes || !scales) return fail(METIS_E_INVALID, "mxfp4_quantize: null pointer");
  if (dtype != METIS_BF16 && dtype != METIS_F32) return fail(METIS_E_INVALID, "mxfp4_quantize: dtype %d", dtype);
  if (rows <= 0 || cols <= 0 || ld < cols) return fail(METIS_E_INVALID, "mxfp4_quantize: shape %lld x %lld, ld %lld",
                                                     (long long)rows, (long long)cols, (long long)ld);
  if (axis != 0 && axis != 1) return fail(METIS_E_INVALID, "mxfp4_quantize: axis %d", axis);
  if (rounding != METIS_RNE && rounding != METIS_SR) return fail(METIS_E_INVALID, "mxfp4_quantize: rounding %d", rounding);
  if (step < 0) return fail(METIS_E_INVALID, "mxfp4_quantize: step %lld", (long long)step);
  const int64_t k_len = axis ? cols : rows;
  if (k_len % 32) return fail(METIS_E_INVALID, "mxfp4_quantize: K = %lld is not a multiple of 32", (long long)k_len);
  if ((uintptr_t)codes & 15) return fail(METIS_E_INVALID, "mxfp4_quantize: codes not 16-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  MxQuantParams q{M, dtype, rows, cols, ld, codes, scales, rounding == METIS_SR, seed, tag, (uint32_t)step};
  if (axis == 1) {
    hipLaunchKernelGGL(mx_quant_rows_kernel, dim3(grid1(rows * (cols >> 5), 256)), dim3(256), 0, st, q);
  } else {
    if ((rows >> 5) > 65535) return fail(METIS_E_UNSUPPORTED, "mxfp4_quantize: %lld rows", (long long)rows);
    hipLaunchKernelGGL(mx_quant_cols_kernel, dim3(grid1(cols, 256), (unsigned)(rows >> 5)), dim3(256), 0, st, q);
  }
  LAUNCH_CHECK();
  return METIS_OK;
}

metis_status metis_mxfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                              const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, float* C, int64_t ldc,
                              void* stream) {
  if (M < 0 || N < 0 || K <= 0) return fail(METIS_E_INVALID, "mxfp4_gemm: shape %lld x %lld x %lld",
                                            (long long)M, (long long)N, (long long)K);
  if (M == 0 || N == 0) return METIS_OK;
  if (!a_codes || !a_scales || !b_codes || !b_scales || !C) return fail(METIS_E_INVALID, "mxfp4_gemm: null pointer");
  if (K % 1024) return fail(METIS_E_UNSUPPORTED, "mxfp4_gemm: K = %lld is not a multiple of 1024", (long long)K);
  if (M % 8 || N % 8) return fail(METIS_E_UNSUPPORTED, "mxfp4_gemm: M and N must be multiples of 8");
  if (K / 2 * 8 > INT32_MAX) return fail(METIS_E_UNSUPPORTED, "mxfp4_gemm: K = %lld too large", (long long)K);
  if (ldc < N) return fail(METIS_E_INVALID, "mxfp4_gemm: ldc %lld < N %lld", (long long)ldc, (long long)N);
  if (((uintptr_t)a_codes | (uintptr_t)a_scales | (uintptr_t)b_codes | (uintptr_t)b_scales) & 15)
    return fail(METIS_E_INVALID, "mxfp4_gemm: code and scale arrays must be 16-byte aligned");
  MxGemmParams g{M, N, K, a_codes, a_scales, b_codes, b_scales, C, ldc};
  hipStream_t st = (hipStream_t)stream;
  TimingRec* tr = timing_begin(st, 3, M, N, K, 0);
  const hipError_t e = launch_mx_gemm(g, st);
  if (e != hipSuccess) return fail(METIS_E_HIP, "mxfp4_gemm launch: %s", hipGetErrorString(e));
  timing_end(tr, st);
  return METIS_OK;
}

}  // extern "C"
