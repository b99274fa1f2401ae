"""MXFP4 reference: quantiser, dequantiser and the product of two quantised
operands.  Test infrastructure: only the tests, the smoke check and the
bench's CPU-baseline leg use the oracle.

The pages do not define MXFP4.  "Full-Stack FP4: Stable LLM Pretraining with
Quantized Projections, Optimizers, and Attention" (局限性) names it only as the
other FP4 format, to which its NVFP4 recipes are not claimed to carry over.
The format is taken from the OCP Microscaling (MX) v1.0 specification, the
plainest reading:
  * 32 consecutive elements along the reduction (K) axis share one scale;
  * the scale is a power of two stored as E8M0 (byte b <-> 2**(b - 127));
  * it is X = 2**(floor(log2 amax) - 2), 2 being the exponent of the largest
    E2M1 value (6 = 1.5 * 2**2), clamped to the E8M0 range;
  * each element is x / X rounded to the nearest E2M1 value (ties to even
    mantissa), saturating at +-6: a block's amax maps into [4, 8), so values
    of 7 and above land on 6;
  * an all-zero block takes the smallest scale (byte 0).
Rounding is to nearest, or stochastic with the generator of the NVFP4 path
(Philox4x32-10, 16-bit draws; oracle/philox.py): an element's draw is indexed
by its position in the quantised output's own row-major layout (outer x K),
and it rounds up to the next E2M1 value iff draw * 2**-16 is below the
element's fractional position between its two neighbours, truncated to 22
binary digits (formats.e2m1_sr; values from 6 up saturate to 6).

Every step is exact in float64 (and in binary32): the exponent is read off
amax, X is a power of two and x / X only shifts exponents, so the codes are
the same whichever of the two precisions takes the decision.

Layout (the GEMM's operand layout): codes uint8 [outer, K/2], element 2i in
the low nibble of byte i; scales uint8 [outer, K/32].  axis names the K axis
of the input matrix (1: along a row, 0: down a column, so that the output is
the quantised transpose).
"""

import numpy as np

from . import philox
from .formats import E2M1_GRID, e2m1_rne, e2m1_sr

BLOCK = 32
EMAX_ELEM = 2


def block_exponent(amax):
    """Shared-scale exponent of blocks with largest magnitude amax (array):
    floor(log2 amax) - 2, clamped to [-127, 127]; -127 for an all-zero block."""
    amax = np.asarray(amax, np.float64)
    e = np.full(amax.shape, -127, dtype=np.int64)
    nz = amax > 0
    # frexp: amax = f * 2**ex with f in [0.5, 1), so floor(log2 amax) = ex - 1
    _, ex = np.frexp(amax[nz])
    e[nz] = np.clip(ex.astype(np.int64) - 1 - EMAX_ELEM, -127, 127)
    return e


def quantize(x, axis=1, rounding="rne", seed=0, tag=0, step=0):
    """MXFP4 codes and E8M0 scales of matrix x along K axis ``axis``, rounded
    to nearest ("rne") or stochastically ("sr", draws from seed, tag, step).
    Returns (codes [outer, K/2] uint8, scales [outer, K/32] uint8)."""
    x = np.asarray(x, np.float64)
    if axis == 0:
        x = x.T
    outer, k = x.shape
    if k % BLOCK:
        raise ValueError("K must be a multiple of 32")
    blocks = x.reshape(outer, k // BLOCK, BLOCK)
    e = block_exponent(np.abs(blocks).max(axis=2))
    y = blocks * np.ldexp(1.0, -e)[:, :, None]
    if rounding == "rne":
        mag = e2m1_rne(np.abs(y))
    elif rounding == "sr":
        idx = (np.arange(outer, dtype=np.uint64)[:, None] * np.uint64(k) + np.arange(k, dtype=np.uint64)[None, :])
        u = philox.uniform_from_halves(philox.halves(idx.ravel(), seed, tag, step))
        mag = e2m1_sr(np.abs(y), u.reshape(outer, k // BLOCK, BLOCK))
    else:
        raise ValueError("rounding must be 'rne' or 'sr'")
    code = (mag | np.where(y < 0, 8, 0)).astype(np.uint8).reshape(outer, k)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, (e + 127).astype(np.uint8)


def dequantize(codes, scales):
    """float64 matrix [outer, K] of the quantised values."""
    codes = np.asarray(codes, np.uint8)
    outer = codes.shape[0]
    c = np.empty((outer, codes.shape[1] * 2), np.uint8)
    c[:, 0::2] = codes & 15
    c[:, 1::2] = codes >> 4
    v = E2M1_GRID[c & 7] * np.where(c & 8, -1.0, 1.0)
    x = np.ldexp(1.0, np.asarray(scales, np.int64) - 127)
    return v * np.repeat(x, BLOCK, axis=1)


def gemm(a, b):
    """C = A-hat B-hat^T of two quantised operands (A: [M, K], B: [N, K], each
    as (codes, scales)), in float64 -- the value a scaled-FP4 matrix
    instruction with exact products and wide accumulation computes."""
    return dequantize(*a) @ dequantize(*b).T
