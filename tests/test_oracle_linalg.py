"""Pins of the oracle's small linear algebra (oracle.linalg) against LAPACK
(numpy.linalg) and closed forms."""

import numpy as np
import pytest

from oracle import linalg


@pytest.mark.parametrize("n", [2, 5, 16, 33])
def test_jacobi_eigh_matches_lapack(n):
    rng = np.random.default_rng(n)
    a = rng.standard_normal((n, n))
    a = a @ a.T + np.diag(rng.uniform(0, 3, n))
    w, v, sweeps = linalg.jacobi_eigh(a)
    wl, vl = np.linalg.eigh(a)
    wl = wl[::-1]
    vl = vl[:, ::-1]
    assert np.allclose(w, wl, rtol=1e-13, atol=1e-13 * abs(wl).max())
    # same vectors up to sign
    for j in range(n):
        assert min(np.abs(v[:, j] - vl[:, j]).max(), np.abs(v[:, j] + vl[:, j]).max()) < 1e-9
    assert np.abs(a @ v - v * w).max() < 1e-12 * abs(w).max()
    assert np.abs(v.T @ v - np.eye(n)).max() < 1e-13
    assert sweeps <= 12


def test_jacobi_eigh_sort_and_sign_rules():
    a = np.diag([1.0, 3.0, 3.0, 2.0])
    w, v, _ = linalg.jacobi_eigh(a)
    assert list(w) == [3.0, 3.0, 2.0, 1.0]
    # ties keep index order; identity eigenvectors keep +1 sign
    assert np.array_equal(v, np.eye(4)[:, [1, 2, 3, 0]])
    rng = np.random.default_rng(0)
    a = rng.standard_normal((6, 6))
    a = a + a.T
    _, v, _ = linalg.jacobi_eigh(a)
    for j in range(6):
        i = np.argmax(np.abs(v[:, j]))
        assert v[i, j] > 0


def test_jacobi_eigh_indefinite_and_diagonal():
    a = np.array([[0.0, 2.0], [2.0, 0.0]])
    w, v, _ = linalg.jacobi_eigh(a)
    assert np.allclose(w, [2.0, -2.0], atol=1e-15)
    assert np.allclose(np.abs(v), np.sqrt(0.5), atol=1e-15)


@pytest.mark.parametrize("shape", [(12, 7), (40, 24), (9, 9), (5, 11)])
def test_jacobi_svd_matches_lapack(shape):
    rng = np.random.default_rng(sum(shape))
    a = rng.standard_normal(shape) * np.exp(rng.standard_normal(shape[1]))
    u, s, v = linalg.jacobi_svd(a)
    sl = np.linalg.svd(a, compute_uv=False)
    assert np.allclose(s[:len(sl)], sl, rtol=1e-12, atol=1e-13 * sl[0])
    assert np.abs((u * s) @ v.T - a).max() < 1e-12 * sl[0]


def test_cholqr3_well_conditioned():
    rng = np.random.default_rng(3)
    y = rng.standard_normal((200, 20)) @ np.diag(np.logspace(0, 4, 20))
    q, r = linalg.cholqr3_shifted(y)
    assert np.abs(q.T @ q - np.eye(20)).max() < 1e-13
    assert np.abs(q @ r - y).max() < 1e-11 * np.abs(y).max()
    assert np.allclose(np.tril(r, -1), 0)


def test_cholqr3_rank_deficient_keeps_the_range():
    # exactly rank 6 sketch of width 14: no breakdown, and Q's span contains Y
    rng = np.random.default_rng(4)
    y = rng.standard_normal((80, 6)) @ rng.standard_normal((6, 14))
    q, _ = linalg.cholqr3_shifted(y)
    assert np.all(np.isfinite(q))
    # range(Y) lies in span(Q), and Q has orthonormal columns (the eight
    # directions beyond the rank are normalised rounding noise)
    coef = np.linalg.lstsq(q, y, rcond=None)[0]
    assert np.linalg.norm(y - q @ coef) < 1e-13 * np.linalg.norm(y)
    assert np.abs(q.T @ q - np.eye(14)).max() < 1e-4
