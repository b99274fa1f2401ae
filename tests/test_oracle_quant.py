"""Pins of the oracle's NVFP4 quantiser (module oracle.nvfp4)."""

import numpy as np
import pytest

from oracle import formats, nvfp4, philox


def _grid_tensor(rng, rows, cols, axis, pow2_scales, exp=-3):
    """A tensor every element of which is +-grid * s_b * s_g exactly, with
    A_T = 2688 * 2**exp (so s_g = 2**exp) and each block's max = 6 s_b s_g.

    Blocks run along ``axis``.  Quantising it must reproduce it exactly."""
    s_g = 2.0 ** exp
    n_outer, K = (rows, cols) if axis == 1 else (cols, rows)
    nb = K // 16
    if pow2_scales:
        sb = 2.0 ** rng.integers(-9, 7, size=(n_outer, nb)).astype(np.float64)
    else:
        # any E4M3 value from the normal range below 448
        sb = formats.e4m3_decode(rng.integers(0x08, 0x7E, size=(n_outer, nb)))
    sb[0, 0] = 448.0                                   # the tensor max block
    m = rng.integers(0, 8, size=(n_outer, nb, 16))
    m[:, :, 0] = 7                                     # each block reaches 6 s_b
    sign = np.where(rng.random((n_outer, nb, 16)) < 0.5, -1.0, 1.0)
    x = sign * formats.E2M1_GRID[m] * sb[:, :, None] * s_g
    x = x.reshape(n_outer, K)
    x = x if axis == 1 else x.T
    assert np.array_equal(x.astype(np.float32).astype(np.float64), x)
    return x.astype(np.float32)


@pytest.mark.parametrize("axis", [0, 1])
def test_rne_idempotent_on_representable_tensor(axis):
    rng = np.random.default_rng(7 + axis)
    x = _grid_tensor(rng, 64, 96, axis, pow2_scales=False)
    q = nvfp4.quantize(x, axis, "rne")
    assert q.s_g == np.float32(2.0 ** -3)
    assert np.array_equal(nvfp4.dequantize(q), x.astype(np.float64))


@pytest.mark.parametrize("axis", [0, 1])
def test_sr_idempotent_on_representable_tensor(axis):
    rng = np.random.default_rng(11 + axis)
    x = _grid_tensor(rng, 48, 64, axis, pow2_scales=True)
    q = nvfp4.quantize(x, axis, "sr", seed=5, tag=0x123, step=3)
    assert np.array_equal(nvfp4.dequantize(q), x.astype(np.float64))


@pytest.mark.parametrize("rounding", ["rne", "sr"])
def test_axis0_is_axis1_of_transpose(rounding):
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((64, 48)) * np.exp(rng.standard_normal((64, 48)))).astype(np.float32)
    q0 = nvfp4.quantize(x, 0, rounding, seed=4, tag=9, step=1)
    q1t = nvfp4.quantize(np.ascontiguousarray(x.T), 1, rounding, seed=4, tag=9, step=1)
    assert np.array_equal(q0.codes, q1t.codes)
    assert np.array_equal(q0.scales, q1t.scales)
    assert q0.s_g == q1t.s_g
    assert q0.codes.shape == (48, 32) and q0.scales.shape == (48, 4)
    assert np.array_equal(nvfp4.dequantize(q0), nvfp4.dequantize(q1t).T)


def test_zero_tensor():
    x = np.zeros((16, 32), np.float32)
    x[3, 5] = -0.0
    q = nvfp4.quantize(x, 1, "rne")
    assert q.s_g == 1.0
    assert not q.scales.any()
    codes = nvfp4.unpack_codes(q)
    assert codes[3, 5] == 8 and np.count_nonzero(codes) == 1


def test_scale_rules_on_a_hand_block():
    # one block: A_T = 26.88 gives s_g = RN32(0.01), d = RN32(6 * s_g);
    # a_b = 26.88 -> t = a_b / d ~ 448 -> s_b = 448; element 13.44 = half the
    # max -> y ~ 3 -> magnitude 5 (value 3); -6.72 -> y ~ 1.5 -> 8 | 3
    x = np.zeros((1, 16), np.float32)
    x[0, :4] = [26.88, 13.44, -6.72, 0.001]
    q = nvfp4.quantize(x, 1, "rne")
    s_g = np.float32(np.float64(np.float32(26.88)) / 2688.0)
    assert q.s_g == s_g
    assert q.scales[0, 0] == 0x7E
    codes = nvfp4.unpack_codes(q)[0]
    assert list(codes[:4]) == [7, 5, 8 | 3, 0]


def test_rne_error_bound_random():
    # |x - x_hat| <= half the local grid step times s_eff, except for
    # saturation of the block max which the E4M3 rounding bounds by 2**-4
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((128, 256)) * np.exp(2 * rng.standard_normal((128, 1)))).astype(np.float32)
    q = nvfp4.quantize(x, 1, "rne")
    xh = nvfp4.dequantize(q)
    s_b = np.repeat(formats.e4m3_decode(q.scales), 16, axis=1)
    s_eff = s_b * np.float64(q.s_g)
    zero = s_b == 0
    # a block whose scale rounds to zero holds only values below d * 2**-10
    d = 6.0 * np.float64(q.s_g)
    assert np.all(np.abs(x[zero]) <= d * 2.0 ** -10 * (1 + 1e-6))
    assert np.all(xh[zero] == 0)
    nz = ~zero
    y = np.abs(x[nz]) / s_eff[nz]
    step = np.where(y < 2, 0.5, np.where(y < 4, 1.0, 2.0))
    bound = np.maximum(step / 2, y - 6.0) * s_eff[nz] * (1 + 1e-6)
    assert np.all(np.abs(xh[nz] - x[nz]) <= bound)
    # normal block scales keep the block max within the E4M3 rounding of 6
    normal = s_b[nz] >= 2.0 ** -6
    assert np.all(y[normal] <= 6.0 * (1 + 2.0 ** -4) + 1e-6)


def test_sr_unbiased():
    # E[x_hat] = x for values inside the range: 4096 seeds, 4 sigma bound
    rng = np.random.default_rng(9)
    x = rng.uniform(-1, 1, (1, 64)).astype(np.float32)
    x[0, 0] = 1.0
    n = 4096
    acc = np.zeros(x.shape)
    acc2 = np.zeros(x.shape)
    for seed in range(n):
        xh = nvfp4.dequantize(nvfp4.quantize(x, 1, "sr", seed=seed, tag=1, step=0))
        acc += xh
        acc2 += xh * xh
    mean = acc / n
    var = np.maximum(acc2 / n - mean ** 2, 1e-30)
    # scales do not depend on the seed: y < 6 are the in-range elements
    q = nvfp4.quantize(x, 1, "sr", seed=0, tag=1, step=0)
    s_eff = np.repeat(formats.e4m3_decode(q.scales), 16, axis=1) * np.float64(q.s_g)
    y = np.abs(x) / s_eff
    inr = y < 6
    assert inr.sum() >= 60
    # exact Bernoulli variance of the two-point rounding
    lo = formats.E2M1_GRID[formats.e2m1_floor(np.where(inr, y, 0))]
    hi = formats.E2M1_GRID[np.minimum(formats.e2m1_floor(np.where(inr, y, 0)) + 1, 7)]
    p = (np.where(inr, y, 0) - lo) / (hi - lo)
    sd = np.sqrt(p * (1 - p) / n) * (hi - lo) * s_eff
    assert np.all(np.abs(mean - x)[inr] <= 4 * sd[inr] + 1e-9 * s_eff[inr])
    assert np.all(var >= 0)
    # out of range: deterministic saturation to 6 s_eff
    assert np.all(np.abs(mean[~inr]) == 6 * s_eff[~inr])


def test_sr_uses_element_index_and_role():
    x = np.random.default_rng(2).standard_normal((32, 32)).astype(np.float32)
    a = nvfp4.quantize(x, 1, "sr", seed=1, tag=philox.make_tag(0, 2, 1), step=0)
    b = nvfp4.quantize(x, 1, "sr", seed=1, tag=philox.make_tag(0, 2, 1), step=0)
    c = nvfp4.quantize(x, 1, "sr", seed=1, tag=philox.make_tag(0, 2, 1), step=1)
    assert np.array_equal(a.codes, b.codes)
    assert not np.array_equal(a.codes, c.codes)


def test_k_not_multiple_of_16_rejected():
    with pytest.raises(ValueError):
        nvfp4.quantize(np.ones((4, 24), np.float32), 1)


@pytest.mark.parametrize("rounding", ["rne", "sr"])
def test_part_quantisation_matches_whole(rounding):
    # a panel quantised with the whole tensor's amax and its origin equals the
    # corresponding rows (axis 1) / outer rows (axis 0) of the whole result
    x = (np.random.default_rng(21).standard_normal((96, 80)) * 3).astype(np.float32)
    amax = np.float32(np.max(np.abs(x)))
    full1 = nvfp4.quantize(x, 1, rounding, seed=3, tag=77, step=2)
    part1 = nvfp4.quantize(x[32:64], 1, rounding, seed=3, tag=77, step=2, amax=amax, origin=(32, 0, 80))
    assert np.array_equal(part1.codes, full1.codes[32:64])
    assert np.array_equal(part1.scales, full1.scales[32:64])
    assert part1.s_g == full1.s_g
    full0 = nvfp4.quantize(x, 0, rounding, seed=3, tag=77, step=2)
    # columns 16..31, rows 48..95 (whole 16-row blocks along K = rows)
    part0 = nvfp4.quantize(x[48:96, 16:32], 0, rounding, seed=3, tag=77, step=2, amax=amax,
                           origin=(16, 48, 96))
    assert np.array_equal(part0.codes, full0.codes[16:32, 24:48])
    assert np.array_equal(part0.scales, full0.scales[16:32, 3:6])


@pytest.mark.parametrize("rounding", ["rne", "sr"])
def test_part_quantisation_matches_whole_matrix_draws(rounding):
    # the same with draws laid out by the tensor's own row-major positions:
    # a panel's origin is its (row, column) in the whole tensor
    x = (np.random.default_rng(22).standard_normal((96, 80)) * 3).astype(np.float32)
    amax = np.float32(np.max(np.abs(x)))
    kw = dict(seed=3, tag=77, step=2, draws="matrix")
    full1 = nvfp4.quantize(x, 1, rounding, **kw)
    part1 = nvfp4.quantize(x[32:64, 16:48], 1, rounding, amax=amax, origin=(32, 16, 80), **kw)
    assert np.array_equal(part1.codes, full1.codes[32:64, 8:24])
    assert np.array_equal(part1.scales, full1.scales[32:64, 1:3])
    full0 = nvfp4.quantize(x, 0, rounding, **kw)
    part0 = nvfp4.quantize(x[48:96, 16:32], 0, rounding, amax=amax, origin=(48, 16, 80), **kw)
    assert np.array_equal(part0.codes, full0.codes[16:32, 24:48])
    assert np.array_equal(part0.scales, full0.scales[16:32, 3:6])


def test_matrix_draws_shared_between_orientations():
    # Every 16-block of x, along rows and along columns, holds one entry 6 and
    # smaller magnitudes elsewhere (6 at (i, i % 16) and (i, 16 + i % 16)), so
    # all block scales are equal in both orientations and each element gets
    # the same y in both.  With one draw per element (draws="matrix") the two
    # orientations then round every element alike; with a draw per position
    # in each orientation's own layout they disagree on many elements.
    rng = np.random.default_rng(23)
    x = rng.uniform(-5.0, 5.0, (32, 32)).astype(np.float32)
    i = np.arange(32)
    x[i, i % 16] = 6.0
    x[i, 16 + i % 16] = 6.0
    kw = dict(seed=8, tag=5, step=1)
    q1 = nvfp4.quantize(x, 1, "sr", draws="matrix", **kw)
    q0 = nvfp4.quantize(x, 0, "sr", draws="matrix", **kw)
    assert np.all(q1.scales == q1.scales[0, 0]) and np.all(q0.scales == q1.scales[0, 0])
    assert np.array_equal(nvfp4.unpack_codes(q1), nvfp4.unpack_codes(q0).T)
    o1 = nvfp4.quantize(x, 1, "sr", draws="own", **kw)
    o0 = nvfp4.quantize(x, 0, "sr", draws="own", **kw)
    assert np.array_equal(nvfp4.unpack_codes(o1), nvfp4.unpack_codes(q1))  # same index along axis 1
    assert (nvfp4.unpack_codes(o1) != nvfp4.unpack_codes(o0).T).mean() > 0.1
