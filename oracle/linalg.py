"""Small dense linear algebra of the randomized SVD, in float64.

* ``jacobi_eigh``: cyclic Jacobi for a symmetric matrix, using the symmetric
  2x2 Schur rotation of Golub & Van Loan, "Matrix Computations", section 8.5
  (the Jacobi method), row-cyclic pair order.  Stops when off(A) <= 1e-15 *
  ||A||_F or after 30 sweeps.  Eigenpairs are sorted by decreasing eigenvalue
  (ties by index) and each eigenvector is signed so that its entry of largest
  magnitude is positive (lowest index wins a tie).  The Metis pages name a
  randomized SVD (关键设计 2) but not its eigensolver; the sort and sign rules
  are readings that make the result unique.
* ``jacobi_svd``: one-sided (Hestenes) Jacobi SVD, the brute-force reference
  for tiny inputs.
* ``cholqr3_shifted``: shifted CholeskyQR3 (Fukaya, Kannan, Nakatsukasa, Zhang
  & Yamamoto, SIAM J. Sci. Comput. 2020): one shifted Cholesky-QR pass followed
  by two more.  The Full-Stack FP4 page (section 2.1) also pairs Cholesky-QR
  with a randomized SVD.  Reading: the first shift is
  11 (p n + n (n + 1)) u ||Y||_F^2 with u = 2**-24 (the unit roundoff of the
  binary32 sketch the GPU forms).  Passes 2 and 3 are plain Cholesky-QR; only
  if their Cholesky factorisation breaks down (an exactly rank-deficient
  sketch) is the pass repeated with the same shift formula at u = 2**-53.
"""

import math

import numpy as np
import scipy.linalg

JACOBI_TOL = 1e-15
JACOBI_MAX_SWEEPS = 30


def _off(a):
    """Frobenius norm of the off-diagonal part, summed directly (subtracting
    the diagonal's share from ||A||_F would cancel catastrophically)."""
    off = a - np.diag(np.diag(a))
    return float(np.sqrt(np.sum(off * off)))


def sort_and_sign(w, v):
    """Sort eigenpairs by decreasing value (ties by index); sign each vector
    so that its largest-magnitude entry is positive (first index on ties)."""
    order = np.argsort(-w, kind="stable")
    w = w[order]
    v = v[:, order].copy()
    for j in range(v.shape[1]):
        i = int(np.argmax(np.abs(v[:, j])))
        if v[i, j] < 0:
            v[:, j] = -v[:, j]
    return w, v


def jacobi_eigh(a, tol=JACOBI_TOL, max_sweeps=JACOBI_MAX_SWEEPS):
    """Eigen-decomposition of a symmetric matrix: returns (w, V), A V = V diag(w).

    Returns also the number of sweeps taken as a third value."""
    a = np.array(a, dtype=np.float64, copy=True)
    n = a.shape[0]
    if a.shape != (n, n):
        raise ValueError("square matrix expected")
    a = 0.5 * (a + a.T)
    v = np.eye(n)
    norm = np.linalg.norm(a)
    sweeps = 0
    while sweeps < max_sweeps and _off(a) > tol * norm:
        sweeps += 1
        for p in range(n - 1):
            for q in range(p + 1, n):
                apq = a[p, q]
                if apq == 0.0:
                    continue
                diff = a[q, q] - a[p, p]
                if abs(diff) > 1e300 * abs(apq):
                    t = apq / diff           # tau overflows: t = 1 / (2 tau)
                else:
                    tau = diff / (2.0 * apq)
                    h = math.hypot(1.0, tau)
                    t = 1.0 / (tau + h) if tau >= 0 else -1.0 / (-tau + h)
                c = 1.0 / np.sqrt(1.0 + t * t)
                s = t * c
                rp = a[p, :].copy()
                rq = a[q, :].copy()
                a[p, :] = c * rp - s * rq
                a[q, :] = s * rp + c * rq
                cp = a[:, p].copy()
                cq = a[:, q].copy()
                a[:, p] = c * cp - s * cq
                a[:, q] = s * cp + c * cq
                vp = v[:, p].copy()
                vq = v[:, q].copy()
                v[:, p] = c * vp - s * vq
                v[:, q] = s * vp + c * vq
    w, v = sort_and_sign(np.diag(a).copy(), v)
    return w, v, sweeps


def jacobi_svd(a, tol=1e-15, max_sweeps=60):
    """One-sided Jacobi SVD of a (m x n, m >= n): returns U (m x n), s, V (n x n).

    Column pairs are rotated until every pair is orthogonal to ``tol``."""
    u = np.array(a, dtype=np.float64, copy=True)
    m, n = u.shape
    if m < n:
        ut, s, vt = jacobi_svd(u.T, tol, max_sweeps)
        return vt, s, ut
    v = np.eye(n)
    for _ in range(max_sweeps):
        rotated = False
        for p in range(n - 1):
            for q in range(p + 1, n):
                alpha = u[:, p] @ u[:, p]
                beta = u[:, q] @ u[:, q]
                gamma = u[:, p] @ u[:, q]
                if abs(gamma) <= tol * np.sqrt(alpha * beta) or gamma == 0.0:
                    continue
                rotated = True
                zeta = (beta - alpha) / (2.0 * gamma)
                t = np.sign(zeta) / (abs(zeta) + math.hypot(1.0, zeta)) if zeta != 0 else 1.0
                c = 1.0 / np.sqrt(1.0 + t * t)
                s = c * t
                up = u[:, p].copy()
                uq = u[:, q].copy()
                u[:, p] = c * up - s * uq
                u[:, q] = s * up + c * uq
                vp = v[:, p].copy()
                vq = v[:, q].copy()
                v[:, p] = c * vp - s * vq
                v[:, q] = s * vp + c * vq
        if not rotated:
            break
    s = np.linalg.norm(u, axis=0)
    order = np.argsort(-s, kind="stable")
    s = s[order]
    u = u[:, order]
    v = v[:, order]
    nz = s > 0
    u[:, nz] = u[:, nz] / s[nz]
    return u, s, v


def cholqr_pass(y, shift):
    """Q = Y R^{-1} with R^T R = Y^T Y + shift I (Cholesky); returns (Q, R)."""
    n = y.shape[1]
    g = y.T @ y + shift * np.eye(n)
    lower = np.linalg.cholesky(g)
    q = scipy.linalg.solve_triangular(lower, y.T, lower=True).T
    return q, lower.T


def _guarded_pass(y, c):
    try:
        return cholqr_pass(y, 0.0)
    except np.linalg.LinAlgError:
        return cholqr_pass(y, c * 2.0 ** -53 * np.sum(y * y))


def cholqr3_shifted(y):
    """Shifted CholeskyQR3 of a tall p x n matrix; returns (Q, R) with Y = Q R."""
    y = np.asarray(y, dtype=np.float64)
    p, n = y.shape
    c = 11.0 * (p * n + n * (n + 1))
    q1, r1 = cholqr_pass(y, c * 2.0 ** -24 * np.sum(y * y))
    q2, r2 = _guarded_pass(q1, c)
    q3, r3 = _guarded_pass(q2, c)
    return q3, r3 @ r2 @ r1
