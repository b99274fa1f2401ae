"""Pins of the oracle's random sources: Philox stream statistics, the Omega
quantile table and the row sampler.

Philox itself is "parity unpinned" for its exact stream (no known-answer
vectors here); these tests check the properties any correct Philox4x32-10
stream has and that the scalar and vectorised forms agree."""

import math

import numpy as np
import torch

from oracle import philox, rsvd


def test_scalar_and_vector_forms_agree():
    e = np.array([0, 1, 2, 3, 4, 5, 7, 2 ** 33 + 5, 2 ** 40 + 3], dtype=np.uint64)
    for seed, tag, step in [(0, 0, 0), (0xDEADBEEF12345678, 0x00021400, 7)]:
        vec = philox.words(e, seed, tag, step)
        sca = [philox.word_scalar(int(v), seed, tag, step) for v in e]
        assert [int(v) for v in vec] == sca


def test_uniformity_chi_square():
    w = philox.words(np.arange(1 << 18, dtype=np.uint64), 1, 0x2100, 0)
    hist = np.bincount((w >> np.uint64(24)).astype(np.int64), minlength=256)
    exp = (1 << 18) / 256
    chi2 = float(np.sum((hist - exp) ** 2 / exp))
    # 255 dof: mean 255, sd ~22.6; 6 sd bound
    assert chi2 < 255 + 6 * 22.6


def test_bit_balance_and_serial_independence():
    w = philox.words(np.arange(1 << 16, dtype=np.uint64), 3, 0x1300, 2)
    bits = ((w[:, None] >> np.arange(32, dtype=np.uint64)[None, :]) & np.uint64(1)).astype(np.float64)
    frac = bits.mean(axis=0)
    assert np.all(np.abs(frac - 0.5) < 6 * 0.5 / math.sqrt(1 << 16))
    u = (w >> np.uint64(8)).astype(np.float64) * 2.0 ** -24
    r = np.corrcoef(u[:-1], u[1:])[0, 1]
    assert abs(r) < 6 / math.sqrt(1 << 16)


def test_counter_avalanche():
    # flipping one counter bit flips about half of the 128 output bits
    rng = np.random.default_rng(0)
    flips = []
    for _ in range(200):
        c = [int(v) for v in rng.integers(0, 2 ** 32, 4, dtype=np.uint64)]
        k = [int(v) for v in rng.integers(0, 2 ** 32, 2, dtype=np.uint64)]
        b = int(rng.integers(0, 128))
        c2 = list(c)
        c2[b // 32] ^= 1 << (b % 32)
        o1, o2 = philox.block(c, k), philox.block(c2, k)
        flips.append(sum(bin(x ^ y).count("1") for x, y in zip(o1, o2)))
    assert abs(np.mean(flips) - 64) < 2.0


def test_uniform_is_exact_binary32():
    h = philox.halves(np.arange(4096, dtype=np.uint64), 9, 0, 0)
    u = philox.uniform_from_halves(h)
    assert np.all(u.astype(np.float32).astype(np.float64) == u)
    assert u.min() >= 0 and u.max() < 1


def test_halves_scalar_vector_and_uniformity():
    e = np.array([0, 1, 2, 7, 8, 9, 15, 2 ** 35 + 11], dtype=np.uint64)
    vec = philox.halves(e, 77, 0x21400, 3)
    assert [int(v) for v in vec] == [philox.half_scalar(int(x), 77, 0x21400, 3) for x in e]
    h = philox.halves(np.arange(1 << 18, dtype=np.uint64), 2, 0x100, 0)
    hist = np.bincount(h >> 8, minlength=256)
    exp = (1 << 18) / 256
    assert float(np.sum((hist - exp) ** 2 / exp)) < 255 + 6 * 22.6
    # the two halves of one word are not the same draw
    assert np.mean(h[0::2] == h[1::2]) < 0.01


# ------------------------------------------------------------- Omega table --

def test_rn_bf16_matches_torch_on_binary32_values():
    # torch's float32 -> bfloat16 cast rounds to nearest even; for values
    # exact in binary32 the double-rounding question does not arise
    rng = np.random.default_rng(4)
    x = (rng.standard_normal(20000) * 4).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    ours = np.array([rsvd.rn_bf16(float(v)) for v in x])
    assert np.array_equal(ours, ref)


def test_omega_table_properties():
    t = rsvd.omega_table()
    assert t.shape == (65536,)
    assert np.array_equal(t[::-1], -t)                 # antisymmetric
    assert np.all(np.diff(t) >= 0)                     # monotone
    assert abs(t.mean()) < 1e-12
    assert abs(t.var() - 1.0) < 2e-3
    # bf16 values
    assert np.array_equal(torch.from_numpy(t).to(torch.bfloat16).double().numpy(), t)


def test_omega_table_is_the_normal_quantile():
    # independent check with the CDF from math.erfc: the exact quantile of
    # (t + 0.5) / 65536 lies within half a bf16 ulp of T[t]
    t = rsvd.omega_table()
    for i in list(range(0, 65536, 97)) + [0, 1, 32767, 32768, 65535]:
        v = t[i]
        ulp = 2.0 ** (math.frexp(v)[1] - 8)
        cdf = lambda z: 0.5 * math.erfc(-z / math.sqrt(2.0))
        p = (i + 0.5) / 65536.0
        assert cdf(v - ulp / 2) <= p * (1 + 1e-12) and p <= cdf(v + ulp / 2) * (1 + 1e-12)


def test_omega_matrix_shape_and_stream():
    om = rsvd.omega(64, 16, seed=0, tag=philox.make_tag(0, 1, 0), step=0)
    assert om.shape == (64, 16)
    om2 = rsvd.omega(64, 16, seed=0, tag=philox.make_tag(0, 1, 0), step=8)
    assert not np.array_equal(om, om2)
    # columns nearly orthogonal with norm ~ sqrt(64)
    g = om.T @ om / 64
    assert np.all(np.abs(np.diag(g) - 1) < 0.6)


# ----------------------------------------------------------------- sampler --

def test_sample_indices_basic():
    idx = rsvd.sample_indices(1000, 37, 0, philox.make_tag(0, 2, 0), 0)
    assert len(idx) == 37 and len(set(idx.tolist())) == 37
    assert np.all(np.diff(idx) > 0) and idx.min() >= 0 and idx.max() < 1000
    assert np.array_equal(rsvd.sample_indices(50, 50, 0, 0, 0), np.arange(50))


def test_sample_indices_uniform_inclusion():
    r, l_k, trials = 200, 20, 600
    counts = np.zeros(r)
    for step in range(trials):
        counts[rsvd.sample_indices(r, l_k, 1, philox.make_tag(0, 2, 0), step)] += 1
    p = l_k / r
    exp = trials * p
    chi2 = float(np.sum((counts - exp) ** 2 / (exp * (1 - p))))
    assert chi2 < (r - 1) + 6 * math.sqrt(2 * (r - 1))


def test_sample_is_the_smallest_keys():
    # brute force: the chosen rows are exactly those with the l_k smallest
    # (key, index) pairs
    r, l_k = 300, 31
    tag = philox.make_tag(2, 3, 0)
    idx = rsvd.sample_indices(r, l_k, 5, tag, 4)
    keys = [(philox.word_scalar(i, 5, philox.with_role(tag, philox.ROLE_SAMPLE), 4), i) for i in range(r)]
    want = sorted(i for _, i in sorted(keys)[:l_k])
    assert idx.tolist() == want
