"""Helpers shared by the GPU parity tests: run the HIP path on one layer and
convert its outputs into the oracle's types."""

import math
import sys

import numpy as np
import torch

from oracle import nvfp4, philox, rsvd, split_gemm
from spectral_split_quantized_amd import metis, synth


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_np(t):
    return t.detach().float().cpu().numpy() if t.dtype == torch.bfloat16 else t.detach().cpu().numpy()


def qt_from_gpu(q4, rows, cols, axis):
    """oracle QTensor holding the GPU's codes, scales and tensor scale."""
    return nvfp4.QTensor(q4.codes.cpu().numpy(), q4.scales.cpu().numpy(),
                         np.float32(q4.tensor_scale.cpu().item()), rows, cols, axis)


def qop_from_gpu(q):
    op = split_gemm.QOperand(q.rows, q.cols)
    if q.k:
        op.s = q.S.cpu().numpy().astype(np.float32)
        op.u_q = qt_from_gpu(q.U, q.rows, q.k, 0)
        op.v_q = qt_from_gpu(q.V, q.cols, q.k, 0)
    if q.R_ax0 is not None:
        op.r_ax0 = qt_from_gpu(q.R_ax0, q.rows, q.cols, 0)
    if q.R_ax1 is not None:
        op.r_ax1 = qt_from_gpu(q.R_ax1, q.rows, q.cols, 1)
    return op


def assert_qtensor_equal(gpu_q4, oracle_q, what):
    codes = gpu_q4.codes.cpu().numpy()
    scales = gpu_q4.scales.cpu().numpy()
    sg = np.float32(gpu_q4.tensor_scale.cpu().item())
    assert sg == oracle_q.s_g, "%s: tensor scale %r vs oracle %r" % (what, sg, oracle_q.s_g)
    bad_s = np.argwhere(scales != oracle_q.scales)
    assert bad_s.size == 0, "%s: %d block scales differ, first at %s" % (what, len(bad_s), bad_s[:3])
    bad_c = np.argwhere(codes != oracle_q.codes)
    assert bad_c.size == 0, "%s: %d code bytes differ, first at %s" % (what, len(bad_c), bad_c[:3])


def sin_max(a, b):
    """sine of the largest principal angle between span(a) and span(b)."""
    qa = np.linalg.qr(np.asarray(a, np.float64))[0]
    qb = np.linalg.qr(np.asarray(b, np.float64))[0]
    return float(np.linalg.norm(qb - qa @ (qa.T @ qb), 2))


def rel_fro(a, b):
    return split_gemm.rel_fro(a, b)


class Layer:
    """One linear layer (X: l x m, W: m x n, D: l x n) through the HIP path."""

    def __init__(self, X, W, D, k, s, l_k, rounding, seed=0, layer=0, refresh=8):
        self.X, self.W, self.D = X, W, D
        self.cfg = metis.make_config(k=k, s=s, l_k=l_k, refresh=refresh,
                                     rounding=metis.SR if rounding == "sr" else metis.RNE, seed=seed)
        self.ocfg = rsvd.Config(k=k, s=s, l_k=l_k, refresh=refresh, rounding=rounding, seed=seed)
        self.rounding = rounding
        self.seed = seed
        self.tags = {"X": metis.make_tag(layer, metis.OPERAND_X),
                     "W": metis.make_tag(layer, metis.OPERAND_W),
                     "D": metis.make_tag(layer, metis.OPERAND_D)}
        self.sample = {"X": True, "W": False, "D": True}
        self.factors = {}
        self.q = {}
        self.resid = {}

    def mats(self):
        return {"X": self.X, "W": self.W, "D": self.D}

    def decompose(self, names=("X", "W", "D"), step=0):
        for n in names:
            M = self.mats()[n]
            if M is None:
                continue
            if n not in self.factors:
                self.factors[n] = metis.Factors(M.shape[0], M.shape[1], self.cfg.k, M.device)
            metis.decompose(M, self.cfg, self.sample[n], self.tags[n], step, self.factors[n])

    def quantize(self, names=("X", "W", "D"), step=0, export=True, direct=False):
        for n in names:
            M = self.mats()[n]
            if M is None:
                continue
            res = torch.empty(M.shape, dtype=torch.float32, device=M.device) if export else None
            f = None if direct else self.factors[n]
            self.q[n] = metis.quantize(M, self.cfg, self.tags[n], step, metis.AXIS0 | metis.AXIS1,
                                       factors=f, residual_out=res)
            self.resid[n] = res
