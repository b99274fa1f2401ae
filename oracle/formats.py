"""Bit-level definitions of the two number formats NVFP4 uses.

The Metis notes page (section 研究背景与动机) names FP4 as E2M1 and the NVFP4
block format as blocks of 16 values sharing one FP8 scale.  The pages do not
fix the FP8 flavour; E4M3 ("FN": bias 7, no infinities, largest finite 448,
smallest normal 2**-6, subnormal step 2**-9) is taken, as in the OCP 8-bit
floating point specification.

E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit.  Magnitude index m = 0..7
maps to {0, 0.5, 1, 1.5, 2, 3, 4, 6}; a code is sign << 3 | m.

All functions are vectorised over numpy arrays and work in float64, in which
every binary32 value and every product of two binary32 values is exact.
"""

import numpy as np

E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E4M3_MAX = 448.0


def e2m1_rne(y):
    """Magnitude index of the nearest E2M1 value to y >= 0, ties to the value
    whose mantissa bit is 0, saturating at 6.

    Midpoints between neighbours and their winners:
      0.25 -> 0, 0.75 -> 1, 1.25 -> 1, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4.
    """
    y = np.asarray(y, np.float64)
    m = np.full(y.shape, 7, dtype=np.uint8)
    m[y <= 5.0] = 6
    m[y < 3.5] = 5
    m[y <= 2.5] = 4
    m[y < 1.75] = 3
    m[y <= 1.25] = 2
    m[y < 0.75] = 1
    m[y <= 0.25] = 0
    return m


def e2m1_floor(y):
    """Index of the largest grid value <= y (y >= 0, y < 6)."""
    y = np.asarray(y, np.float64)
    return (np.searchsorted(E2M1_GRID, y, side="right") - 1).astype(np.uint8)


SR_FRACTION_BITS = 22


def e2m1_sr(y, u):
    """Stochastic rounding of y >= 0 onto the E2M1 grid with uniforms u.

    y >= 6 saturates to 6.  Otherwise lo = floor-grid(y), hi = the next grid
    value, p = (y - lo) / (hi - lo) (exact: hi - lo is a power of two and
    y - lo is exact by Sterbenz), and the result is hi iff u < p22, where p22
    is p truncated to SR_FRACTION_BITS = 22 binary fraction digits,
    floor(p * 2**22) / 2**22.

    The truncation is a reading (the pages give stochastic rounding without
    a precision): a binary32 value in [1, 6) carries exactly 22 bits below
    the E2M1 spacing, so p22 = p there; only values below 1 (E2M1's
    subnormal range), whose binary32 form has further bits, lose
    probability mass below 2**-22.  With 16-bit uniforms the decision
    u < p22 is that of adding a random integer to those 22 bits and
    truncating, the classic way stochastic rounding is built.
    """
    y = np.asarray(y, np.float64)
    u = np.asarray(u, np.float64)
    sat = y >= 6.0
    ys = np.where(sat, 0.0, y)
    lo = e2m1_floor(ys)
    hi = np.minimum(lo + 1, 7)
    glo = E2M1_GRID[lo]
    ghi = E2M1_GRID[hi]
    p = (ys - glo) / (ghi - glo)
    p22 = np.floor(p * 2.0 ** SR_FRACTION_BITS) / 2.0 ** SR_FRACTION_BITS
    m = np.where(u < p22, hi, lo).astype(np.uint8)
    return np.where(sat, np.uint8(7), m)


def e4m3_encode(t):
    """E4M3 byte of the round-to-nearest-even value of t >= 0, saturating.

    t >= 448 (including +inf) gives 448 (0x7E).  Below 2**-6 the subnormal
    grid has step 2**-9; 2**-10 rounds to 0 (tie to even)."""
    t = np.asarray(t, np.float64)
    out = np.zeros(t.shape, dtype=np.uint8)
    sat = t >= E4M3_MAX
    sub = t < 2.0 ** -6
    # subnormals: integer multiple of 2**-9, ties to even (np.rint is RNE)
    q = np.rint(np.where(sub, t, 0.0) * 512.0).astype(np.int64)  # 0..8
    out = np.where(sub, q.astype(np.uint8), out)  # q == 8 encodes 2**-6 = 0x08
    # normals: exponent from frexp (t = f * 2**e, 0.5 <= f < 1)
    tn = np.where(sub | sat, 1.0, t)
    f, e = np.frexp(tn)
    ex = e - 1                                # t = (2f) * 2**ex, 1 <= 2f < 2
    mq = np.rint((2.0 * f - 1.0) * 8.0).astype(np.int64)  # 0..8, RNE
    carry = mq == 8
    ex = np.where(carry, ex + 1, ex)
    mq = np.where(carry, 0, mq)
    over = (ex > 8) | ((ex == 8) & (mq == 7))  # 480 and above saturate
    code = ((ex + 7) << 3) | mq
    code = np.where(over, 0x7E, code)
    out = np.where(~sub & ~sat, code.astype(np.uint8), out)
    out = np.where(sat, np.uint8(0x7E), out)
    return out.astype(np.uint8)


def e4m3_decode(b):
    """Value (float64) of non-negative E4M3 bytes (sign bit must be 0)."""
    b = np.asarray(b, np.int64)
    if np.any(b & 0x80):
        raise ValueError("negative E4M3 scales are not produced by the quantiser")
    if np.any(b == 0x7F):
        raise ValueError("E4M3 NaN encoding")
    e = (b >> 3) & 0xF
    m = b & 0x7
    sub = e == 0
    val = np.where(sub, m * 2.0 ** -9,
                   (1.0 + m / 8.0) * np.exp2(np.where(sub, 1, e) - 7.0))
    return val.astype(np.float64)


def f32(x):
    """Round float64 values to binary32 (one IEEE RNE rounding)."""
    return np.asarray(x, np.float64).astype(np.float32)
