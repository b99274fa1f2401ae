"""Philox4x32-10 (Salmon, Moraes, Dror & Shaw, "Parallel Random Numbers: As
Easy as 1, 2, 3", SC'11), written from the paper's description.

The Metis notes page (section 损失函数/训练策略) says stochastic rounding is on
by default but names no generator; the randomized sketch (关键设计 2) needs a
Gaussian test matrix and a random row sample.  Reading taken here: every random
draw of the path comes from one counter-based Philox4x32-10 stream so that the
GPU and this oracle consume identical randomness.

Layout (a reading; the pages fix none):
  key     = (seed & 0xffffffff, seed >> 32)
  counter = (q & 0xffffffff, q >> 32, tag, step)
  32-bit draws (row sampling): q = e >> 2, element e takes word (e & 3)
  16-bit draws (stochastic rounding, Omega): q = e >> 3, element e takes
      16-bit half (e & 1) (low half first) of word ((e >> 1) & 3); the
      rounding uniform is u = h * 2**-16, exact in binary32.  Sixteen random
      bits per element keep the probability error of the rounding below
      2**-16 of a grid step while one block serves eight elements.

Round function (paper, section 3 "Philox"): with multipliers M0, M1 the block
(c0, c1, c2, c3) becomes (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1,
lo(M0*c0)); the key is bumped by the Weyl constants between rounds.

Parity unpinned for the exact output stream: no known-answer vectors are
available in this environment.  The constants below are the published ones;
the tests check statistics and that the scalar and vectorised forms agree.
"""

import numpy as np

MASK32 = 0xFFFFFFFF
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
ROUNDS = 10

# tag roles (bits 8..11 of the 32-bit tag word); both quantised orientations
# of an operand (its residual, or the operand itself) draw from ROLE_RESID,
# role 1 is unused
ROLE_RESID = 0
ROLE_U = 2
ROLE_V = 3
ROLE_OMEGA = 4
ROLE_SAMPLE = 5


def make_tag(layer, operand, role):
    """tag = layer << 16 | operand << 12 | role << 8 (operand: W=1, X=2, D=3)."""
    return ((layer & 0xFFFF) << 16) | ((operand & 0xF) << 12) | ((role & 0xF) << 8)


def with_role(tag, role):
    """Replace the role field of a tag."""
    return (tag & ~0xF00) | ((role & 0xF) << 8)


def block(ctr, key):
    """One Philox4x32-10 block on Python ints: ctr 4-tuple, key 2-tuple."""
    c0, c1, c2, c3 = (int(v) & MASK32 for v in ctr)
    k0, k1 = (int(v) & MASK32 for v in key)
    for _ in range(ROUNDS):
        p0 = PHILOX_M0 * c0
        p1 = PHILOX_M1 * c2
        hi0, lo0 = p0 >> 32, p0 & MASK32
        hi1, lo1 = p1 >> 32, p1 & MASK32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
        k0 = (k0 + PHILOX_W0) & MASK32
        k1 = (k1 + PHILOX_W1) & MASK32
    return c0, c1, c2, c3


def block_vec(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox4x32-10 over numpy arrays (any broadcastable shapes).

    Every value is held in uint64 so the 32x32 products are exact."""
    m = np.uint64(MASK32)
    c0 = np.asarray(c0, np.uint64) & m
    c1 = np.asarray(c1, np.uint64) & m
    c2 = np.asarray(c2, np.uint64) & m
    c3 = np.asarray(c3, np.uint64) & m
    k0 = np.uint64(int(k0) & MASK32)
    k1 = np.uint64(int(k1) & MASK32)
    s32 = np.uint64(32)
    for _ in range(ROUNDS):
        p0 = np.uint64(PHILOX_M0) * c0
        p1 = np.uint64(PHILOX_M1) * c2
        n0 = (p1 >> s32) ^ c1 ^ k0
        n1 = p1 & m
        n2 = (p0 >> s32) ^ c3 ^ k1
        n3 = p0 & m
        c0, c1, c2, c3 = n0, n1, n2, n3
        k0 = np.uint64((int(k0) + PHILOX_W0) & MASK32)
        k1 = np.uint64((int(k1) + PHILOX_W1) & MASK32)
    return c0, c1, c2, c3


def words(elem, seed, tag, step):
    """Philox word of each logical element index in ``elem`` (uint64 array)."""
    e = np.asarray(elem, np.uint64)
    q = e >> np.uint64(2)
    lane = (e & np.uint64(3)).astype(np.int64)
    m = np.uint64(MASK32)
    out = block_vec(q & m, q >> np.uint64(32), np.uint64(tag & MASK32),
                    np.uint64(step & MASK32), seed & MASK32, (seed >> 32) & MASK32)
    stacked = np.stack(out, axis=0)
    return np.take_along_axis(stacked, lane[None, ...], axis=0)[0]


def word_scalar(e, seed, tag, step):
    """Scalar form of :func:`words` on Python ints (slow; for cross-checks)."""
    q = e >> 2
    out = block((q & MASK32, q >> 32, tag, step), (seed & MASK32, seed >> 32))
    return out[e & 3]


def halves(elem, seed, tag, step):
    """16-bit draw of each logical element index (uint64 array -> int64)."""
    e = np.asarray(elem, np.uint64)
    q = e >> np.uint64(3)
    word = ((e >> np.uint64(1)) & np.uint64(3)).astype(np.int64)
    half = (e & np.uint64(1)).astype(np.uint64)
    m = np.uint64(MASK32)
    out = block_vec(q & m, q >> np.uint64(32), np.uint64(tag & MASK32),
                    np.uint64(step & MASK32), seed & MASK32, (seed >> 32) & MASK32)
    w = np.take_along_axis(np.stack(out, axis=0), word[None, ...], axis=0)[0]
    return ((w >> (half * np.uint64(16))) & np.uint64(0xFFFF)).astype(np.int64)


def half_scalar(e, seed, tag, step):
    """Scalar form of :func:`halves` on Python ints."""
    q = e >> 3
    out = block((q & MASK32, q >> 32, tag, step), (seed & MASK32, seed >> 32))
    return (out[(e >> 1) & 3] >> (16 * (e & 1))) & 0xFFFF


def uniform_from_halves(h):
    """u = h * 2**-16 in [0, 1), exact in binary32 (returned as float64)."""
    return np.asarray(h, np.float64) * 2.0 ** -16
