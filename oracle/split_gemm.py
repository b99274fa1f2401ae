"""Quantised operands and the split GEMMs, by dense dequantisation.

Source: Metis notes page, 关键设计 1: the forward GEMM is
    Y-hat = (Q(A_k) Lambda_k Q(B_k^T) + Q(X_R)) (Q(U_k) S_k Q(V_k^T) + Q(W_R))
with Q applied to every matrix except the singular values; 整体框架 and
损失函数/训练策略 say the split is embedded in all forward and backward GEMMs
(W4A4G4).  For Y = X W with X (l x m), W (m x n) and output gradient D (l x n):
    Y  = X-hat W-hat        (both quantised along m)
    dX = D-hat W-hat^T      (both quantised along n)
    dW = X-hat^T D-hat      (both quantised along l)
Readings: U_k is blocked along its rows and V_k along its rows (16 consecutive
entries of each singular vector share a scale), so each factor is quantised
once for all three GEMMs; the residual is quantised once per K axis it is
consumed along; outputs are float64 here (binary32 on the GPU).

The oracle forms each dequantised operand densely and multiplies with numpy's
float64 matmul, so no algebraic re-association is involved.
"""

import numpy as np

from . import nvfp4, philox


class QOperand:
    """Quantised operand: factors U (rows x k), V (cols x k) as QTensors along
    axis 0, S (binary32, length k), and the residual in up to two K axes."""

    def __init__(self, rows, cols, u_q=None, v_q=None, s=None, r_ax0=None, r_ax1=None):
        self.rows = rows
        self.cols = cols
        self.u_q = u_q
        self.v_q = v_q
        self.s = None if s is None else np.asarray(s, np.float32)
        self.r_ax0 = r_ax0
        self.r_ax1 = r_ax1

    @property
    def k(self):
        return 0 if self.s is None else len(self.s)


def quantize_operand(m, u, s, v, rounding, seed, tag, step, axes=(0, 1), m_r=None):
    """Quantise one operand: factors (if any) and the residual.

    m        the operand (rows x cols); its residual M - U diag(S) V^T is
             formed in float64 and rounded once to binary32 unless ``m_r`` (a
             binary32 residual, e.g. one exported by another implementation)
             is given.
    u, s, v  factors (binary32 values) or None for direct NVFP4.
    tag      base Philox tag (layer/operand); roles are filled in here.
    """
    m = np.asarray(m, np.float64)
    rows, cols = m.shape
    if m_r is None:
        if u is None:
            m_r = m.astype(np.float32)
        else:
            m_r = (m - (np.asarray(u, np.float64) * np.asarray(s, np.float64))
                   @ np.asarray(v, np.float64).T).astype(np.float32)
    op = QOperand(rows, cols)
    if u is not None:
        op.s = np.asarray(s, np.float32)
        op.u_q = nvfp4.quantize(np.asarray(u, np.float32), 0, rounding, seed,
                                philox.with_role(tag, philox.ROLE_U), step)
        op.v_q = nvfp4.quantize(np.asarray(v, np.float32), 0, rounding, seed,
                                philox.with_role(tag, philox.ROLE_V), step)
    # both orientations of the residual round each element with one draw
    resid_tag = philox.with_role(tag, philox.ROLE_RESID)
    if 0 in axes:
        op.r_ax0 = nvfp4.quantize(m_r, 0, rounding, seed, resid_tag, step, draws="matrix")
    if 1 in axes:
        op.r_ax1 = nvfp4.quantize(m_r, 1, rounding, seed, resid_tag, step, draws="matrix")
    return op


def dense(op, axis):
    """float64 M-hat = Q(U) S Q(V)^T + Q(M_R) for the residual along ``axis``."""
    r = op.r_ax0 if axis == 0 else op.r_ax1
    if r is None:
        raise ValueError("operand not quantised along axis %d" % axis)
    out = nvfp4.dequantize(r)
    if op.k:
        uh = nvfp4.dequantize(op.u_q)
        vh = nvfp4.dequantize(op.v_q)
        out = out + (uh * op.s.astype(np.float64)) @ vh.T
    return out


def gemm_fwd(xq, wq):
    """Y = X-hat W-hat, X quantised along its columns (m), W along its rows (m)."""
    return dense(xq, 1) @ dense(wq, 0)


def gemm_bwd(dq, wq, xq):
    """(dX, dW) = (D-hat W-hat^T along n, X-hat^T D-hat along l)."""
    dx = dense(dq, 1) @ dense(wq, 1).T
    dw = dense(xq, 0).T @ dense(dq, 0)
    return dx, dw


def rel_fro(a, b):
    """||a - b||_F / ||b||_F."""
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(np.asarray(a, np.float64) - b) / max(np.linalg.norm(b), 1e-300))
