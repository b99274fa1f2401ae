"""Spectral split of one operand: randomized sketch, projection + rediag,
residual and the cross-step factor cache, in float64.

Sources (Metis notes page):
  关键设计 1  M = U_k S_k V_k^T + M_R; the rank-k part keeps its singular
             values in high precision, the residual is quantised.
  关键设计 2  (i) estimate the dominant subspace from l_k << l randomly chosen
             rows (sample covariance); (ii) project the hidden dimension to
             k + s columns with a Gaussian test matrix Omega (randomized SVD).
  关键设计 3  reuse the low-rank factors across steps; refresh every 8 steps.
  损失函数/训练策略  rank k = 1.5%, refresh period 8.

Readings where the pages are silent:
  * Omega_ij = T[h] with h the 16-bit Philox draw of element i*(k+s)+j and
    T[t] = bf16-RNE(Phi^{-1}((t + 0.5) / 65536)): a quantile-exact discretised
    Gaussian whose values are exact in bf16.
  * Rows are sampled uniformly without replacement: row i gets the Philox
    word of element i as key, rows are ordered by (key, i), the first l_k are
    kept and sorted ascending.  M_s = sqrt(r / l_k) M[idx, :].  Weights are not
    sampled (l_k = r).
  * No power iteration.  Q = shifted CholeskyQR3(M_s Omega); B = Q^T M_s;
    Jacobi on B B^T gives (Theta, Z); V = B^T Z Theta^{-1/2}, first k columns;
    a column with theta_i <= 1e-12 theta_1 is set to zero.
  * Every step: P = M V; Jacobi on P^T P gives (lambda, R); V <- V R with the
    largest-magnitude entry of each column made positive, U = P R
    lambda^{-1/2}, S = sqrt(lambda) (columns with lambda_i <= 1e-12 lambda_1
    get U = 0, S = 0).  Then U S V^T = M V_old V_old^T exactly.
  * The cache holds V (after the rediag rotation) and the step of the last
    refresh; a refresh happens when the cache is empty or
    step - refreshed_at >= refresh.
"""

import math
import statistics
from dataclasses import dataclass

import numpy as np

from . import linalg, philox

EIG_ZERO = 1e-12


@dataclass
class Config:
    k: int
    s: int = 8
    l_k: int = 0
    refresh: int = 8
    rounding: str = "rne"
    seed: int = 0


def rn_bf16(x):
    """Round a Python float to the nearest bfloat16 value (ties to even)."""
    if x == 0.0 or not math.isfinite(x):
        return x
    m, e = math.frexp(x)             # x = m 2^e, 0.5 <= |m| < 1
    q = round(m * 256.0)             # 8 significant bits; round() is half-even
    return math.ldexp(q, e - 8)


_OMEGA_TABLE = None


def omega_table():
    """T[t] = bf16(Phi^{-1}((t + 0.5) / 65536)), t = 0..65535 (float64 array)."""
    global _OMEGA_TABLE
    if _OMEGA_TABLE is None:
        nd = statistics.NormalDist()
        _OMEGA_TABLE = np.array([rn_bf16(nd.inv_cdf((t + 0.5) / 65536.0))
                                 for t in range(65536)], dtype=np.float64)
    return _OMEGA_TABLE


def omega(cols, n, seed, tag, step):
    """Gaussian test matrix Omega (cols x n) for a sketch of width n = k + s."""
    e = np.arange(cols * n, dtype=np.uint64)
    h = philox.halves(e, seed, philox.with_role(tag, philox.ROLE_OMEGA), step)
    return omega_table()[h].reshape(cols, n)


def sample_indices(rows, l_k, seed, tag, step):
    """l_k distinct row indices, ascending (uniform without replacement)."""
    if not 0 < l_k <= rows:
        raise ValueError("need 0 < l_k <= rows")
    i = np.arange(rows, dtype=np.uint64)
    key = philox.words(i, seed, philox.with_role(tag, philox.ROLE_SAMPLE), step)
    order = np.lexsort((i, key))     # primary key, then row index
    return np.sort(order[:l_k]).astype(np.int64)


def rsvd_sketch(m, cfg, sample_rows, tag, step, return_theta=False):
    """Right basis V (cols x k) of the dominant subspace from a sketch
    (and the sketch eigenvalues Theta when ``return_theta``)."""
    m = np.asarray(m, dtype=np.float64)
    r, c = m.shape
    k, n = cfg.k, cfg.k + cfg.s
    if sample_rows:
        l_k = cfg.l_k
        idx = sample_indices(r, l_k, cfg.seed, tag, step)
        ms = math.sqrt(r / l_k) * m[idx, :]
    else:
        ms = m
    if n > min(ms.shape[0], c):
        raise ValueError("k + s must not exceed min(l_k, cols)")
    om = omega(c, n, cfg.seed, tag, step)
    y = ms @ om
    q, _ = linalg.cholqr3_shifted(y)
    b = q.T @ ms
    theta, z, _ = linalg.jacobi_eigh(b @ b.T)
    v = np.zeros((c, k))
    top = theta[0]
    for j in range(k):
        if top > 0 and theta[j] > EIG_ZERO * top:
            v[:, j] = (b.T @ z[:, j]) / math.sqrt(theta[j])
    return (v, theta) if return_theta else v


def project_rediag(m, v):
    """(U, S, V_new, P) from the cached basis V: P = M V, rediagonalised."""
    m = np.asarray(m, dtype=np.float64)
    p = m @ v
    lam, rot, _ = linalg.jacobi_eigh(p.T @ p)
    v_new = v @ rot
    for j in range(v_new.shape[1]):
        i = int(np.argmax(np.abs(v_new[:, j])))
        if v_new[i, j] < 0:
            v_new[:, j] = -v_new[:, j]
            rot[:, j] = -rot[:, j]
    k = v.shape[1]
    s = np.zeros(k)
    u = np.zeros((m.shape[0], k))
    top = lam[0] if k else 0.0
    for j in range(k):
        if top > 0 and lam[j] > EIG_ZERO * top:
            s[j] = math.sqrt(lam[j])
            u[:, j] = (p @ rot[:, j]) / s[j]
    return u, s, v_new, p


def residual(m, u, s, v):
    """M_R = M - U diag(S) V^T."""
    return np.asarray(m, np.float64) - (np.asarray(u, np.float64) * np.asarray(s, np.float64)) @ np.asarray(v, np.float64).T


class FactorCache:
    """Cross-step cache of one operand's basis (关键设计 3)."""

    def __init__(self):
        self.v = None
        self.refreshed_at = None

    def needs_refresh(self, step, refresh):
        return self.v is None or step - self.refreshed_at >= refresh


def decompose(m, cfg, sample_rows, tag, step, cache=None):
    """One step of the spectral split: (U, S, V) with the cache updated.

    refreshed: whether the sketch ran on this call."""
    if cache is None:
        cache = FactorCache()
    refreshed = cache.needs_refresh(step, cfg.refresh)
    if refreshed:
        cache.v = rsvd_sketch(m, cfg, sample_rows, tag, step)
        cache.refreshed_at = step
    u, s, v_new, _ = project_rediag(m, cache.v)
    cache.v = v_new
    return u, s, v_new, refreshed
