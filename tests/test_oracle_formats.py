"""Pins of the oracle's number formats against hand-fixed cases.

The golden files under tests/golden/ carry their own citations."""

import os

import numpy as np
import pytest
import torch

from oracle import formats, nvfp4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                a, b = line.split()
                rows.append((a, b))
    return rows


def test_e2m1_golden_rne():
    rows = _read("e2m1_rne.txt")
    y = np.array([np.float32(float(a)) for a, _ in rows], dtype=np.float64)
    want = np.array([int(b) for _, b in rows])
    got = formats.e2m1_rne(y)
    assert list(got) == list(want)


def test_e4m3_golden_rne():
    rows = _read("e4m3_rne.txt")
    t = np.array([np.float32(float(a)) for a, _ in rows], dtype=np.float64)
    want = np.array([int(b, 16) for _, b in rows])
    got = formats.e4m3_encode(t)
    assert [hex(v) for v in got] == [hex(v) for v in want]


def test_e4m3_roundtrip_all_bytes():
    # every finite non-negative E4M3 value encodes back to its own byte
    b = np.arange(0x7F, dtype=np.uint8)           # 0x7F is NaN
    v = formats.e4m3_decode(b)
    assert np.all(np.diff(v) > 0)                 # strictly increasing
    assert v[0x38] == 1.0 and v[0x7E] == 448.0 and v[0x08] == 2.0 ** -6 and v[1] == 2.0 ** -9
    assert np.array_equal(formats.e4m3_encode(v), b)


def test_e4m3_matches_torch_float8_e4m3fn():
    # independent library routine: torch's float8_e4m3fn cast rounds to
    # nearest even; below 448 the two definitions coincide
    rng = np.random.default_rng(1)
    t = np.concatenate([rng.uniform(0, 448, 20000), 2.0 ** rng.uniform(-12, 8.8, 20000)])
    t = t[t < 448].astype(np.float32)
    ours = formats.e4m3_encode(t.astype(np.float64))
    ref = torch.from_numpy(t).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e2m1_sr_never_moves_grid_values_and_saturates():
    g = formats.E2M1_GRID
    u = np.linspace(0, 1 - 2 ** -24, g.size)
    assert np.array_equal(formats.e2m1_sr(g, u), np.arange(8))
    assert np.all(formats.e2m1_sr(np.array([6.0, 7.5, 1e30]), np.zeros(3)) == 7)


def test_e2m1_sr_probability_is_linear_interpolation():
    # y = 2.25 lies a quarter of the way from 2 to 3; with a uniform grid of
    # u values exactly a quarter must round up
    u = (np.arange(4096) >> 0) / 4096.0
    m = formats.e2m1_sr(np.full(4096, 2.25), u)
    assert np.sum(m == 5) == 1024 and np.sum(m == 4) == 3072


def test_grid_is_the_e2m1_bit_layout():
    # decode every 3-bit magnitude from its bit fields (bias 1, one mantissa bit)
    vals = []
    for m in range(8):
        e, f = m >> 1, m & 1
        vals.append(f * 0.5 if e == 0 else (1 + f / 2) * 2.0 ** (e - 1))
    assert np.array_equal(np.array(vals), formats.E2M1_GRID)


def test_signed_zero_codes():
    x = np.zeros((1, 16), np.float32)
    x[0, 0] = 1.0
    x[0, 1] = -1e-6          # far below the block's quantisation step
    x[0, 2] = -0.0
    q = nvfp4.quantize(x, 1, "rne")
    codes = nvfp4.unpack_codes(q)[0]
    assert codes[1] == 0x8 and codes[2] == 0x8 and codes[3] == 0x0


def test_e2m1_sr_golden():
    rows = []
    with open(os.path.join(GOLDEN, "e2m1_sr.txt")) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                a, h, c = line.split()
                rows.append((np.float32(float(a)), int(h), int(c)))
    y = np.array([r[0] for r in rows], dtype=np.float64)
    u = np.array([r[1] for r in rows], dtype=np.float64) * 2.0 ** -16
    want = [r[2] for r in rows]
    assert list(formats.e2m1_sr(y, u)) == want


def test_e2m1_sr_truncation_only_below_one():
    # a binary32 y in [1, 6) has exactly 22 bits below its E2M1 spacing, so
    # there the rule is the plain "hi iff u < p"; below 1 it differs only
    # where p has bits past the 22nd and u sits within 2**-22 under p
    rng = np.random.default_rng(7)
    y = rng.uniform(1.0, 6.0, 200000).astype(np.float32).astype(np.float64)
    h = rng.integers(0, 65536, y.size)
    lo = formats.e2m1_floor(y)
    glo, ghi = formats.E2M1_GRID[lo], formats.E2M1_GRID[np.minimum(lo + 1, 7)]
    p = (y - glo) / (ghi - glo)
    plain = np.where(h * 2.0 ** -16 < p, lo + 1, lo)
    assert np.array_equal(formats.e2m1_sr(y, h * 2.0 ** -16), plain)
    ys = rng.uniform(0.0, 1.0, 200000).astype(np.float32).astype(np.float64)
    lo = formats.e2m1_floor(ys)
    p = (ys - formats.E2M1_GRID[lo]) / 0.5
    u = np.floor(p * 2 ** 16) * 2.0 ** -16          # the largest draw below p
    m = formats.e2m1_sr(ys, u)
    p22 = np.floor(p * 2 ** 22) / 2 ** 22
    assert np.array_equal(m == lo + 1, u < p22)
    assert np.any(u < p) and np.all((u < p22) <= (u < p))
