/*
 * metis.h -- C ABI of the MI355X (gfx950) Metis spectral-split NVFP4 GEMM.
 *
 * The method is described on the web page "Metis: Training LLMs with FP4
 * Quantization" (ICLR 2026 reading notes):
 *   - section 关键设计 1: every GEMM operand M (weight W, activation X, output
 *     gradient D) is split as M = U_k S_k V_k^T + M_R; the factors and the
 *     residual are quantised, the singular values stay in high precision, and
 *     the forward GEMM is
 *       Y = (Q(A_k) L_k Q(B_k^T) + Q(X_R)) (Q(U_k) S_k Q(V_k^T) + Q(W_R));
 *   - section 关键设计 2: the dominant subspace is estimated from a sparse
 *     random row sample and a Gaussian random projection (randomized SVD);
 *   - section 关键设计 3: the factors are reused across steps (refresh every 8);
 *   - section 研究背景与动机: NVFP4 = E2M1 values in blocks of 16 with one FP8
 *     (here E4M3) scale per block; section 损失函数/训练策略: W4A4G4 with
 *     stochastic rounding, rank 1.5%.
 *
 * Conventions shared by every entry point
 *   Memory.  Every pointer argument except the metis_* descriptor structs and
 *     the host-only self-test helpers is DEVICE memory owned by the caller.
 *     The library allocates no device memory in these calls; scratch space is
 *     the caller's workspace (size from the *_workspace functions, 256-byte
 *     aligned).  Buffers must stay valid until the enqueued work completes.
 *   Streams.  `stream` is a hipStream_t passed as void* (NULL = the null
 *     stream).  Calls only enqueue work and return; they are safe to call from
 *     several threads on distinct streams with distinct workspaces.
 *   Layouts.  Matrices are row-major with a leading dimension `ld` (elements).
 *     A quantised orientation (metis_q4) stores codes[n_outer][k_len/2] with the
 *     even K index in the low nibble, scales[n_outer][k_len/16] as E4M3 bytes,
 *     and one binary32 tensor scale.  "K axis" is the reduction axis of the GEMM
 *     the orientation feeds.
 *   Errors.  Argument errors are reported synchronously with METIS_E_INVALID
 *     (nothing is enqueued) and a message from metis_last_error().  Numeric
 *     failure inside a kernel (non-finite input, a Cholesky breakdown that the
 *     shift cannot repair) sets a per-device flag that metis_status_sync()
 *     returns as METIS_E_NUMERIC; outputs are then unspecified.
 *   Determinism.  Identical inputs, seed, tag and step give bit-identical
 *     outputs: reductions that feed quantisation use max, never sums in
 *     varying order.
 */
#ifndef METIS_H
#define METIS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define METIS_ABI_VERSION 1

typedef enum {
  METIS_OK = 0,
  METIS_E_INVALID = -1,     /* bad argument or shape; nothing was enqueued */
  METIS_E_UNSUPPORTED = -2, /* valid but not implemented (e.g. k + s > 96) */
  METIS_E_HIP = -3,         /* a HIP runtime call failed */
  METIS_E_NUMERIC = -4,     /* device-side numeric failure (status_sync only) */
  METIS_E_WORKSPACE = -5    /* workspace too small */
} metis_status;

typedef enum { METIS_BF16 = 0, METIS_F32 = 1 } metis_dtype;
typedef enum { METIS_RNE = 0, METIS_SR = 1 } metis_rounding;

/* Operand roles used in the Philox tag: tag = layer << 16 | operand << 12.
 * The library fills bits 8..11 (the draw's role) itself. */
enum { METIS_OPERAND_W = 1, METIS_OPERAND_X = 2, METIS_OPERAND_D = 3 };

/* Hyper-parameters (Metis notes page, 关键设计 2/3 and 损失函数/训练策略). */
typedef struct {
  int32_t k;        /* rank kept in high precision (1..96) */
  int32_t s;        /* sketch oversampling; the sketch has k + s columns */
  int64_t l_k;      /* sampled rows for operands with sample_rows != 0 */
  int32_t refresh;  /* factor-cache period in steps (>= 1) */
  int32_t rounding; /* metis_rounding */
  uint64_t seed;    /* Philox4x32-10 key */
} metis_config;

/* Factors of one operand (rows x cols).  U: rows x k, S: k (descending),
 * V: cols x k, all binary32 row-major device buffers owned by the caller.
 * V doubles as the factor cache: it holds the basis between calls.
 * refreshed_at is host state: -1 means "no basis yet". */
typedef struct {
  float *U;
  float *S;
  float *V;
  int64_t rows, cols;
  int32_t k;
  int64_t refreshed_at;
} metis_factors;

/* One quantised orientation (device buffers owned by the caller). */
typedef struct {
  uint8_t *codes;       /* n_outer * k_len / 2 bytes */
  uint8_t *scales;      /* n_outer * k_len / 16 bytes */
  float *tensor_scale;  /* 1 binary32 */
  int64_t n_outer;
  int64_t k_len;        /* multiple of 16 */
} metis_q4;

/* A quantised operand M (rows x cols): Q(U) (blocked along rows of U, so
 * n_outer = k, k_len = rows), S (binary32, not quantised), Q(V) (n_outer = k,
 * k_len = cols), and the residual along K = rows (R_ax0: n_outer = cols,
 * k_len = rows) and/or K = cols (R_ax1: n_outer = rows, k_len = cols).
 * k == 0 is direct NVFP4 (U, V, S unused).
 * S: k binary32 values in device memory.  metis_quantize and
 * metis_prepare_operand copy the factors' S into it when it is non-NULL on
 * entry, so the operand keeps the singular values its codes were made with
 * while later calls update the same factors; when it is NULL they set it to
 * f->S, the live factor buffer, which the next decomposition of those factors
 * overwrites. */
typedef struct {
  int64_t rows, cols;
  int32_t k;
  float *S;
  metis_q4 U, V, R_ax0, R_ax1;
} metis_qoperand;

enum { METIS_AXIS0 = 1, METIS_AXIS1 = 2 }; /* bitmask for metis_quantize */

int32_t metis_abi_version(void);
const char *metis_last_error(void);

/* metis_init_device -- set up the library on the current device: its copy of
 * the Gaussian quantile table that Omega is drawn from, the numeric status
 * word that metis_status_sync reads, and the address of the static scratch
 * array of metis_quantize_static.  Every other call does this itself on its
 * first use of a device; it copies to device symbols synchronously, so a
 * caller that captures library calls into a HIP graph calls this first, on
 * each device, outside the capture.  Repeated calls return METIS_OK at once.
 * Errors: METIS_E_HIP (no device, or a failed copy), METIS_E_UNSUPPORTED
 * (device index >= 64). */
metis_status metis_init_device(void);

/* Workspace sizes in bytes (0 never means "no workspace needed"; always
 * pass at least the returned size). */
size_t metis_decompose_workspace(int64_t rows, int64_t cols, const metis_config *cfg,
                                 int32_t sample_rows);
size_t metis_quantize_workspace(int64_t rows, int64_t cols, int32_t k);
size_t metis_gemm_fwd_workspace(const metis_qoperand *X, const metis_qoperand *W);
size_t metis_gemm_bwd_workspace(const metis_qoperand *D, const metis_qoperand *W,
                                const metis_qoperand *X);
size_t metis_prepare_operand_workspace(int64_t rows, int64_t cols, const metis_config *cfg,
                                       int32_t sample_rows);

/* metis_decompose -- spectral split of one operand (关键设计 1-3).
 * M: rows x cols (dtype metis_dtype, leading dimension ld >= cols).
 * If f->refreshed_at < 0 or step - f->refreshed_at >= cfg->refresh, a new
 * basis is sketched: sample l_k rows (sample_rows != 0; weights use all rows),
 * Y = M_s Omega (Omega: cols x (k+s) quantile-exact bf16 Gaussian), shifted
 * CholeskyQR3 of Y, B = Q^T M_s, Jacobi on B B^T, V = B^T Z Theta^-1/2.
 * f->refreshed_at is then set to step (host side, before the call returns).
 * Every call then projects P = M V, rediagonalises P^T P by Jacobi and writes
 * U = P R Lambda^-1/2, S = Lambda^1/2, V <- V R, so U S V^T = M V_old V_old^T.
 * Requires 1 <= k, k + s <= 96 and k + s <= min(l_k (or rows), cols); with
 * sample_rows != 0, rows <= 2^27 (METIS_E_UNSUPPORTED otherwise: the row
 * sampler resolves the boundary of its key histogram among at most 4096 rows).
 * tag: layer << 16 | operand << 12 (Omega and the row sample take roles 4, 5). */
metis_status metis_decompose(const void *M, int32_t dtype, int64_t rows, int64_t cols, int64_t ld,
                             const metis_config *cfg, int32_t sample_rows, uint32_t tag,
                             int64_t step, metis_factors *f, void *ws, size_t ws_bytes,
                             void *stream);

/* metis_quantize -- NVFP4 fake quantisation of an operand (关键设计 1).
 * With f == NULL the tensor M itself is quantised (direct NVFP4); otherwise
 * the factors are quantised (U and V blocked along their rows) and the
 * residual M_R = M - U diag(S) V^T is formed on the fly (never stored) and
 * quantised along each requested axis (axes: METIS_AXIS0 | METIS_AXIS1).
 * Quantiser: tensor amax A_T, s_g = A_T/2688, block scale = E4M3(RNE, satfinite)
 * of a_b/(6 s_g), y = |x| * (1/(s_b s_g)), E2M1 by RNE or Philox stochastic
 * rounding (16-bit uniform per element).  out->S is set to f->S.
 * residual_out: optional rows x cols binary32 (ld = cols) copy of the exact
 * binary32 residual the quantiser consumed (for verification; NULL normally).
 * Requires K (rows for AXIS0, cols for AXIS1) to be a multiple of 16.
 * out->S: see metis_qoperand (snapshot copy when non-NULL). */
metis_status metis_quantize(const void *M, int32_t dtype, int64_t rows, int64_t cols, int64_t ld,
                            const metis_factors *f, const metis_config *cfg, uint32_t tag,
                            int64_t step, int32_t axes, metis_qoperand *out, float *residual_out,
                            void *ws, size_t ws_bytes, void *stream);

/* metis_quantize_static -- metis_quantize without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Arguments, outputs
 * and errors are those of metis_quantize.  The call allocates nothing: its
 * scratch (the tensor amax words and the fp16 operands of the rank-k
 * product) lives in one static device array of the library per GPU,
 * metis_quantize_static_capacity() bytes (16 MiB), held until the process
 * ends.  An operand whose scratch exceeds it (with factors about
 * (rows + cols) * 6 * round_up(k, 16) bytes) returns METIS_E_UNSUPPORTED with
 * nothing enqueued.  Every call on one GPU uses that GPU's array: calls that
 * overlap in time on one GPU (other streams or threads) race, so the caller
 * orders them; the array keeps the last call's contents and each call clears
 * what it needs zeroed. */
size_t metis_quantize_static_capacity(void);
metis_status metis_quantize_static(const void *M, int32_t dtype, int64_t rows, int64_t cols, int64_t ld,
                                   const metis_factors *f, const metis_config *cfg, uint32_t tag,
                                   int64_t step, int32_t axes, metis_qoperand *out, float *residual_out,
                                   void *stream);

/* metis_prepare_operand -- metis_decompose followed by metis_quantize with
 * the new factors (关键设计 1-3), as one call.  After the projection
 * P = M V_old the residual M_R = M - P V_old^T is quantised on `stream` while
 * the rediagonalisation (Jacobi, V <- V R, U, S) runs on `side_stream`; the
 * two are equal in exact arithmetic because the rotation R is orthogonal
 * (U diag(S) V^T = P R R^T V_old^T), and in binary32 they differ by rounding
 * only.  The factors are then quantised on `stream`, which on return has
 * everything ordered after it.  side_stream may be NULL or equal to stream
 * (then everything runs on stream).  Arguments, requirements and outputs are
 * those of metis_decompose and metis_quantize (f non-NULL; out->k == cfg->k);
 * ws holds at least metis_prepare_operand_workspace(rows, cols, cfg,
 * sample_rows) bytes. */
metis_status metis_prepare_operand(const void *M, int32_t dtype, int64_t rows, int64_t cols, int64_t ld,
                                   const metis_config *cfg, int32_t sample_rows, uint32_t tag,
                                   int64_t step, metis_factors *f, int32_t axes, metis_qoperand *out,
                                   float *residual_out, void *ws, size_t ws_bytes, void *stream,
                                   void *side_stream);

/* metis_gemm_fwd -- Y = X-hat W-hat (关键设计 1, the split forward GEMM).
 * X: l x m with R_ax1 (K = m); W: m x n with R_ax0 (K = m).  Y: l x n
 * binary32, leading dimension ldy.  Evaluated as
 *   Y = Q(X_R) Q(W_R) + P' Q(V_W)^T + Q(U_X) G,
 *   P' = Q(X_R) Q(U_W) S_W,  G = S_X (Q(V_X)^T Q(W_R) + (Q(V_X)^T Q(U_W)) S_W Q(V_W)^T),
 * which equals the product of the dense dequantised operands. */
metis_status metis_gemm_fwd(const metis_qoperand *X, const metis_qoperand *W, float *Y, int64_t ldy,
                            void *ws, size_t ws_bytes, void *stream);

/* metis_gemm_bwd -- dX = D-hat W-hat^T (K = n: D needs R_ax1, W needs R_ax1)
 * and dW = X-hat^T D-hat (K = l: X needs R_ax0, D needs R_ax0), the same
 * split embedded in the backward GEMMs (W4A4G4, 整体框架).  dX: l x m,
 * dW: m x n, binary32.  Either output pointer may be NULL to skip that
 * product.  The dW product uses the part of ws after the dX product's
 * region, so ws holds metis_gemm_bwd_workspace(D, W, X) bytes even when only
 * dW is asked for. */
metis_status metis_gemm_bwd(const metis_qoperand *D, const metis_qoperand *W, const metis_qoperand *X,
                            float *dX, int64_t lddx, float *dW, int64_t lddw, void *ws,
                            size_t ws_bytes, void *stream);

/* Two-phase form of the split GEMMs.  The low-rank terms of a split product
 * (P' and G of the forward equation of 关键设计 1, and their counterparts in
 * dX and dW) ride along K as bf16 hi/lo operands; building them needs only
 * the quantised operands.  *_prepare builds them into ws on `stream` and
 * *_prepared runs the main GEMM, reading them from the same ws, so a caller
 * can build one product's terms on another stream while an earlier GEMM
 * runs.  Arguments are those of metis_gemm_fwd / metis_gemm_bwd; `which`
 * selects the backward products (METIS_GRAD_DX | METIS_GRAD_DW).  Contract:
 * the prepared call names the same operands, ws and ws_bytes as the prepare
 * call, is ordered after it (same stream or an event), and neither ws nor the
 * operands change in between; the results then equal those of
 * metis_gemm_fwd / metis_gemm_bwd bit for bit.  Argument errors return
 * synchronously as in the one-call form. */
enum { METIS_GRAD_DX = 1, METIS_GRAD_DW = 2 };
metis_status metis_gemm_fwd_prepare(const metis_qoperand *X, const metis_qoperand *W, void *ws,
                                    size_t ws_bytes, void *stream);
metis_status metis_gemm_fwd_prepared(const metis_qoperand *X, const metis_qoperand *W, float *Y, int64_t ldy,
                                     void *ws, size_t ws_bytes, void *stream);
metis_status metis_gemm_bwd_prepare(const metis_qoperand *D, const metis_qoperand *W, const metis_qoperand *X,
                                    int32_t which, void *ws, size_t ws_bytes, void *stream);
metis_status metis_gemm_bwd_prepared(const metis_qoperand *D, const metis_qoperand *W, const metis_qoperand *X,
                                     float *dX, int64_t lddx, float *dW, int64_t lddw, void *ws,
                                     size_t ws_bytes, void *stream);

/* Waits for `stream`, then returns and clears the current device's numeric
 * failure flag (METIS_OK or METIS_E_NUMERIC). */
metis_status metis_status_sync(void *stream);

/* ------------------------------------------------------------------ MXFP4
 * A separate FP4 format, for comparison with NVFP4 on the same hardware: the
 * pages name MXFP4 only as a format their NVFP4 recipes are not claimed for
 * ("Full-Stack FP4: Stable LLM Pretraining with Quantized Projections,
 * Optimizers, and Attention", 局限性).  Its definition is the OCP Microscaling
 * (MX) one: 32 consecutive elements along K share a power-of-two scale
 * X = 2^(floor(log2 amax) - 2), stored as an E8M0 byte (exponent + 127,
 * clamped to [-127, 127]; an all-zero block stores 0); each element is x / X
 * rounded to the nearest E2M1 value, ties to even mantissa, saturating at 6
 * (rounding METIS_RNE), or stochastically (METIS_SR) with the Philox draws of
 * seed, tag and step indexed by the element's position outer * K + k in the
 * output layout.  No spectral split on this path.
 *
 * metis_mxfp4_quantize: M is rows x cols, row-major with leading dimension
 * ld, bf16 or fp32 (dtype), finite (a non-finite block sets the numeric flag
 * of metis_status_sync; its codes are then unspecified).  axis names the K
 * axis: 1 along a row, 0 down a column (the output is then the quantised
 * transpose).  With outer = the other dimension and K its length: codes is
 * outer x K/2 bytes (element 2i in the low nibble of byte i), 16-byte
 * aligned; scales is outer x K/32 E8M0 bytes.  K % 32 == 0, rounding is
 * METIS_RNE or METIS_SR and step >= 0 (METIS_E_INVALID otherwise); with
 * axis 0, rows / 32 <= 65535 (METIS_E_UNSUPPORTED otherwise).  Both buffers
 * are caller-owned device memory, written on stream.
 *
 * metis_mxfp4_gemm: C = A B^T in fp32 (row-major, leading dimension ldc >= N)
 * of two MXFP4 operands in that layout, A with M rows and B with N rows of
 * K elements: codes M x K/2 and N x K/2, scales M x K/32 and N x K/32, all four
 * arrays 16-byte aligned, K % 1024 == 0, M % 8 == 0 and N % 8 == 0
 * (METIS_E_UNSUPPORTED otherwise).
 * Products are exact and accumulate in fp32 on the block-scaled FP4 matrix
 * instruction of gfx950.  M or N == 0 returns METIS_OK with nothing enqueued.
 * Argument errors return synchronously; nothing is allocated. */
metis_status metis_mxfp4_quantize(const void *M, int32_t dtype, int64_t rows, int64_t cols, int64_t ld,
                                  int32_t axis, int32_t rounding, uint64_t seed, uint32_t tag, int64_t step,
                                  uint8_t *codes, uint8_t *scales, void *stream);
metis_status metis_mxfp4_gemm(const uint8_t *a_codes, const uint8_t *a_scales, const uint8_t *b_codes,
                              const uint8_t *b_scales, int64_t M, int64_t N, int64_t K, float *C,
                              int64_t ldc, void *stream);

/* Kernel timing for benchmarks.  metis_timing_enable(capacity) creates
 * capacity pairs of HIP events (0 disables timing and releases them); while
 * enabled, each main split-GEMM kernel (kind 0; d = M, N, K, K-extension) and
 * each quantiser sweep (kind 1: amax pass, kind 2: quantise pass; d = rows,
 * cols, axes, K of the rank-k product), each MXFP4 GEMM kernel (kind 3;
 * d = M, N, K, 0), the sketch of a refresh step, from the row sample to V
 * (kind 4; d = rows, cols, k + s, l_k), and metis_decompose's projection
 * and rediagonalisation (kind 5; d = rows, cols, k, 1 on a refresh step)
 * is bracketed by events recorded on the launching stream,
 * until the capacity is used up.  metis_timing_read waits
 * for the recorded events, writes up to max_records durations (ms) and
 * 5-tuples (kind, d0, d1, d2, d3), resets the record list and returns the
 * number written. */
metis_status metis_timing_enable(int32_t capacity);
int32_t metis_timing_read(float *ms, int64_t *shape, int32_t max_records);
/* Restricts the recorded kinds to the bits of mask (bit k: kind k; all kinds
 * by default).  Each record adds two event packets to the stream, so a caller
 * timing a whole step records only the kinds it needs. */
metis_status metis_timing_kinds(int32_t mask);

/* Host-only helpers (no GPU needed) exposing the library's own definitions
 * of its random draws, for verification against an independent model.
 * metis_omega_table: the 65536 bf16 bit patterns of the Gaussian quantile
 * table, T[t] = bf16(Phi^-1((t + 0.5) / 65536)).
 * metis_philox4x32_10: one Philox4x32-10 block (Salmon et al., SC'11). */
void metis_omega_table(uint16_t *out65536);
void metis_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);

#ifdef __cplusplus
}
#endif
#endif /* METIS_H */
