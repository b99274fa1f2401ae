"""Pins of the MXFP4 oracle (oracle/mxfp4.py) to the format's definition: hand
cases worked from the OCP MX rules (shared scale 2**(floor(log2 amax) - 2),
E2M1 elements, nearest with ties to even, saturating at 6), a brute-force
nearest-value search, the round trip, the nibble layout and a loop-level
product."""

import itertools

import numpy as np
import pytest

from oracle import mxfp4

GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _block(vals):
    x = np.zeros((1, 32))
    x[0, :len(vals)] = vals
    return x


def _codes(q):
    c, _ = q
    out = np.empty(c.shape[1] * 2, np.uint8)
    out[0::2] = c[0] & 15
    out[1::2] = c[0] >> 4
    return out


def test_block_with_amax_six_is_exact():
    vals = [6, -4, 3, 0.5, -1.5, 2, 1, 0]
    q = mxfp4.quantize(_block(vals))
    assert q[1][0, 0] == 127  # 2**0
    want = [7, 8 | 6, 5, 1, 8 | 3, 4, 2, 0]
    assert list(_codes(q)[:8]) == want
    assert np.array_equal(mxfp4.dequantize(*q)[0, :8], vals)


def test_saturation_and_ties():
    # amax 7: floor(log2 7) = 2, scale 2**0; 7 saturates to 6; 5 is the 4/6
    # midpoint and goes to 4 (even mantissa); 2.5 ties to 2, 3.5 to 4, 0.25 to 0
    q = mxfp4.quantize(_block([7, 5, 2.5, 3.5, 0.25, 0.75, -7]))
    assert q[1][0, 0] == 127
    assert list(_codes(q)[:7]) == [7, 6, 4, 6, 0, 2, 8 | 7]


def test_small_block_scale():
    # amax 0.3: floor(log2 0.3) = -2, scale 2**-4, 0.3 * 16 = 4.8 -> 4 (code 6)
    q = mxfp4.quantize(_block([0.3, -0.1]))
    assert q[1][0, 0] == 127 - 4
    # -0.1 * 16 = -1.6 -> -1.5 (code 8 | 3)
    assert list(_codes(q)[:2]) == [6, 8 | 3]
    assert np.allclose(mxfp4.dequantize(*q)[0, :2], [0.25, -1.5 / 16])


def test_zero_block_and_scale_clamps():
    q = mxfp4.quantize(np.zeros((2, 64)))
    assert np.all(q[0] == 0) and np.all(q[1] == 0)
    # amax 2**-140 -> exponent clamped to -127; 2**-140 * 2**127 rounds to 0
    q = mxfp4.quantize(_block([2.0 ** -140]))
    assert q[1][0, 0] == 0 and _codes(q)[0] == 0
    # amax 2**127: floor(log2) = 127, exponent 125
    q = mxfp4.quantize(_block([2.0 ** 127]))
    assert q[1][0, 0] == 127 + 125 and _codes(q)[0] == 6


def test_matches_brute_force_nearest():
    """Each element against an exhaustive search over the 15 signed grid
    values times the block scale (ties to the even-mantissa value)."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((16, 64)) * np.exp(rng.uniform(-6, 6, (16, 1)))
    x[0, :32] *= 0  # one zero block
    codes, scales = mxfp4.quantize(x)
    got = mxfp4.dequantize(codes, scales)
    for r, b in itertools.product(range(16), range(2)):
        blk = x[r, 32 * b:32 * b + 32]
        amax = np.abs(blk).max()
        e = -127 if amax == 0 else max(-127, int(np.floor(np.log2(amax))) - 2)
        assert scales[r, b] == e + 127
        s = 2.0 ** e
        for j, v in enumerate(blk):
            cands = sorted(set(g * sg for g in GRID for sg in (1, -1)))
            best = min(cands, key=lambda c: (abs(v / s - c), GRID.index(abs(c)) % 2 if abs(c) in GRID else 0))
            assert got[r, 32 * b + j] == best * s


def test_round_trip_and_nibble_order():
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 256, (8, 32), dtype=np.uint8)
    scales = rng.integers(100, 150, (8, 2), dtype=np.uint8)
    v = mxfp4.dequantize(codes, scales)
    assert np.array_equal(mxfp4.dequantize(*mxfp4.quantize(v)), v)
    # element 2i is the low nibble of byte i
    c1 = np.zeros((1, 16), np.uint8)
    c1[0, 0] = 0x52  # element 0: code 2 (1.0), element 1: code 5 (3.0)
    d = mxfp4.dequantize(c1, np.array([[127]], np.uint8))
    assert d[0, 0] == 1.0 and d[0, 1] == 3.0 and not d[0, 2:].any()


def test_axis0_is_the_transpose():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((64, 48))
    a = mxfp4.quantize(x, axis=0)
    b = mxfp4.quantize(x.T.copy(), axis=1)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    with pytest.raises(ValueError):
        mxfp4.quantize(np.zeros((4, 48)), axis=1)


def test_gemm_against_loops():
    rng = np.random.default_rng(9)
    a = mxfp4.quantize(rng.standard_normal((3, 64)))
    b = mxfp4.quantize(rng.standard_normal((2, 64)))
    da, db = mxfp4.dequantize(*a), mxfp4.dequantize(*b)
    want = [[sum(da[i, t] * db[j, t] for t in range(64)) for j in range(2)] for i in range(3)]
    assert np.allclose(mxfp4.gemm(a, b), want, rtol=1e-15, atol=0)


def test_stochastic_rounding_picks_a_neighbour_and_is_unbiased():
    """SR codes are the two E2M1 neighbours of x / X (6 when saturated), the
    draws are deterministic in (seed, tag, step), and the mean over many tags
    approaches x within the binomial bound."""
    rng = np.random.default_rng(13)
    x = rng.standard_normal((4, 64)) * 3.0
    a = mxfp4.quantize(x, rounding="sr", seed=1, tag=5, step=2)
    b = mxfp4.quantize(x, rounding="sr", seed=1, tag=5, step=2)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert not np.array_equal(a[0], mxfp4.quantize(x, rounding="sr", seed=1, tag=6, step=2)[0])
    scale = np.repeat(np.ldexp(1.0, a[1].astype(np.int64) - 127), 32, axis=1)
    y = np.abs(x) / scale
    got = np.abs(mxfp4.dequantize(*a)) / scale
    grid = np.array(GRID)
    lo = grid[np.searchsorted(grid, np.minimum(y, 6.0), side="right") - 1]
    hi = grid[np.minimum(np.searchsorted(grid, np.minimum(y, 6.0), side="right"), 7)]
    assert np.all((got == lo) | (got == hi) | ((y >= 6) & (got == 6)))
    # unbiasedness on one row over 400 tags
    v = np.array([[0.3, -1.1, 2.6, 4.9, 0.0, 5.5] + [1.0] * 26])
    acc = np.zeros(32)
    n = 400
    for t in range(n):
        acc += mxfp4.dequantize(*mxfp4.quantize(v, rounding="sr", seed=3, tag=t))[0]
    mean = acc / n
    s = 2.0 ** (mxfp4.block_exponent(np.abs(v).max())) * 1.0
    # per element: |mean - v| <= 4 sigma of a Bernoulli mixture with gap <= 2 s
    assert np.all(np.abs(mean - v[0]) <= 4 * (2 * s) * 0.5 / np.sqrt(n) + 1e-12)
    with pytest.raises(ValueError):
        mxfp4.quantize(v, rounding="up")
