"""NVFP4 fake quantiser Q_b and its dequantiser, bit-exact definition.

Source: Metis notes page, 研究背景与动机 (E2M1 values, block size 16, one FP8
scale per block) and 损失函数/训练策略 (stochastic rounding on by default).
The pages leave the scale rules open; the readings taken are:

  Q1  A_T = max |x| over the tensor.  A_T = 0: s_g = 1, every block scale 0.
  Q2  s_g = RN32(A_T / 2688)   (2688 = 6 * 448: largest E2M1 x largest E4M3)
  Q3  d   = RN32(6 * s_g)
  Q4  per block of 16 along K: a_b = max |x|; t_b = RN32(a_b / d);
      s_b = E4M3 round-to-nearest-even, saturating at 448
  Q5  s_b = 0: every code in the block is a (signed) zero
  Q6  s_eff = RN32(s_b * s_g); inv = RN32(1 / s_eff)
  Q7  y = RN32(|x| * inv); an input of +-0 always gives magnitude 0
  Q8  RNE: nearest grid value, ties to even mantissa, saturate at 6.
      SR: y >= 6 -> 6; otherwise hi iff u < p22, p22 = (y - lo) / (hi - lo)
      truncated to 22 binary fraction digits (formats.e2m1_sr), with u the
      element's 16-bit Philox uniform (oracle.philox, 16-bit draws)
  Q9  code = sign(x) << 3 | m  (the sign bit of x is kept, also for zeros)

RN32 is one binary32 round-to-nearest-even operation.  Every binary32 operand
is exact in float64, a product of two binary32 values is exact in float64, and
rounding a float64 quotient of binary32 values to binary32 gives the correctly
rounded binary32 quotient (53 >= 2*24 + 2), so each RN32 step below is
``f32(float64 op float64)`` and matches a binary32 machine bit for bit.

Layout of one quantised orientation (the "K axis" is the axis the blocks run
along, i.e. the GEMM's reduction axis):
  codes  uint8 [n_outer, K/2]  two codes per byte, even K index in the low nibble
  scales uint8 [n_outer, K/16] E4M3 bytes
  s_g    float32 scalar
For axis 1 (K = columns) n_outer is the row count; for axis 0 (K = rows) the
tensor is taken transposed, so n_outer is the column count.

Stochastic rounding draws (readings; the pages name no random stream):
  draws="own"     an element's draw is indexed by its position in the
                  quantised orientation's own row-major layout (n_outer x K):
                  e = i * cols + j along axis 1, e = j * rows + i along axis 0
                  (the factors U and V, quantised along one axis only);
  draws="matrix"  by its position in the tensor's row-major layout,
                  e = i * cols + j along either axis, so an operand's two
                  orientations round each element with the same uniform.
                  Each orientation's rounding stays unbiased on its own; the
                  Philox work per element of an operand halves.
"""

import numpy as np

from . import formats, philox

TENSOR_DIVISOR = 2688.0
BLOCK = 16


class QTensor:
    """One quantised orientation of a tensor (see module docstring)."""

    def __init__(self, codes, scales, s_g, rows, cols, axis):
        self.codes = codes
        self.scales = scales
        self.s_g = np.float32(s_g)
        self.rows = rows
        self.cols = cols
        self.axis = axis

    @property
    def k_len(self):
        return self.rows if self.axis == 0 else self.cols


def tensor_scale(amax):
    """(s_g, d) from the tensor amax (Q1-Q3), both binary32."""
    amax = np.float32(amax)
    if amax == 0:
        return np.float32(1.0), formats.f32(6.0)
    s_g = formats.f32(np.float64(amax) / TENSOR_DIVISOR)
    d = formats.f32(6.0 * np.float64(s_g))
    return s_g, d


def quantize(x, axis, rounding="rne", seed=0, tag=0, step=0, amax=None, origin=None, draws="own"):
    """Quantise a 2-D binary32 tensor along ``axis``; returns a QTensor.

    ``rounding`` is "rne" or "sr" (Philox uniforms with seed/tag/step, laid
    out as ``draws`` says: "own" or "matrix", see the module docstring).

    To quantise part of a larger tensor, pass the larger tensor's ``amax``
    (its exact max |x|, Q1) and ``origin``, which fixes the Philox index of
    every element.  With draws="own", origin = (outer0, k0, K_full): the
    part's first element sits at row outer0, column k0 of the larger tensor's
    quantised orientation (n_outer x K_full).  With draws="matrix", origin =
    (row0, col0, cols_full): it sits at row row0, column col0 of the larger
    tensor itself.  K blocks of the part must be whole blocks of the larger
    tensor."""
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2:
        raise ValueError("2-D input expected")
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input")
    rows, cols = x.shape
    xt = x if axis == 1 else x.T
    n_outer, K = xt.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 16")
    if amax is None:
        amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    amax = np.float32(amax)
    if draws not in ("own", "matrix"):
        raise ValueError("draws must be 'own' or 'matrix'")
    if draws == "own":
        outer0, k0, k_full = (0, 0, K) if origin is None else (int(origin[0]), int(origin[1]), int(origin[2]))
        if k0 % BLOCK or k0 + K > k_full:
            raise ValueError("origin must place whole blocks inside the larger tensor")
    else:
        row0, col0, cols_full = (0, 0, cols) if origin is None else (int(origin[0]), int(origin[1]), int(origin[2]))
        if (row0 if axis == 0 else col0) % BLOCK or col0 + cols > cols_full:
            raise ValueError("origin must place whole blocks inside the larger tensor")
    s_g, d = tensor_scale(amax)
    ax = np.abs(xt).astype(np.float64).reshape(n_outer, K // BLOCK, BLOCK)
    a_b = ax.max(axis=2)
    if amax == 0:
        sb_code = np.zeros(a_b.shape, np.uint8)
    else:
        t_b = formats.f32(a_b / np.float64(d)).astype(np.float64)
        sb_code = formats.e4m3_encode(t_b)
    s_b = formats.e4m3_decode(sb_code)
    s_eff = formats.f32(s_b * np.float64(s_g)).astype(np.float64)
    with np.errstate(divide="ignore"):
        inv = formats.f32(1.0 / s_eff).astype(np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        y = formats.f32(ax * inv[:, :, None]).astype(np.float64)
    y = np.where(ax == 0.0, 0.0, y)
    if rounding == "rne":
        m = formats.e2m1_rne(y)
    elif rounding == "sr":
        if draws == "own":
            # index in the (n_outer x K_full) layout of the whole tensor
            et = ((np.arange(n_outer, dtype=np.uint64) + np.uint64(outer0))[:, None] * np.uint64(k_full)
                  + (np.arange(K, dtype=np.uint64) + np.uint64(k0))[None, :])
        else:
            # index in the tensor's own row-major layout, in xt's order
            e = ((np.arange(rows, dtype=np.uint64) + np.uint64(row0))[:, None] * np.uint64(cols_full)
                 + (np.arange(cols, dtype=np.uint64) + np.uint64(col0))[None, :])
            et = e if axis == 1 else e.T
        et = np.ascontiguousarray(et).ravel()
        u = philox.uniform_from_halves(philox.halves(et, seed, tag, step))
        m = formats.e2m1_sr(y, u.reshape(n_outer, K // BLOCK, BLOCK))
    else:
        raise ValueError("rounding must be 'rne' or 'sr'")
    m = np.where((s_b == 0.0)[:, :, None], np.uint8(0), m).astype(np.uint8)
    sign = np.signbit(xt).reshape(n_outer, K // BLOCK, BLOCK).astype(np.uint8)
    code = ((sign << 3) | m).reshape(n_outer, K)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return QTensor(packed, sb_code.astype(np.uint8), s_g, rows, cols, axis)


def unpack_codes(q):
    """[n_outer, K] uint8 codes (0..15) of a QTensor."""
    lo = q.codes & 0xF
    hi = q.codes >> 4
    out = np.empty((q.codes.shape[0], q.codes.shape[1] * 2), np.uint8)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


def dequantize(q):
    """float64 dequantised tensor in the ORIGINAL orientation (rows x cols):
    x-hat = +-grid[m] * s_b * s_g."""
    code = unpack_codes(q)
    n_outer, K = code.shape
    mag = formats.E2M1_GRID[code & 7]
    sgn = np.where(code & 8, -1.0, 1.0)
    s_b = formats.e4m3_decode(q.scales)
    val = sgn * mag * np.repeat(s_b, BLOCK, axis=1) * np.float64(q.s_g)
    return val if q.axis == 1 else val.T
