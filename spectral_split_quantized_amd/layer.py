"""A PyTorch linear layer whose three GEMMs run through the Metis path.

"Metis: Training LLMs with FP4 Quantization" (整体框架): the weight W, the
activation X and the output gradient D of a linear layer are each split into
a low-rank part and a residual (关键设计 1), quantised to NVFP4 (W4A4G4), and
every GEMM of the forward and backward pass -- Y = X W, dX = D W^T,
dW = X^T D -- is evaluated through the split.  The right factor of each
operand is cached and re-sketched every ``refresh`` steps (关键设计 3).

This module is marshalling only: ``metis.prepare_operand`` and
``metis.gemm_fwd`` / ``metis.gemm_bwd`` run every step in the HIP library.
The weight is stored as in the pages' notation, ``in_features x
out_features`` (Y = X W), as an fp32 master.
"""

import torch

from . import metis

__all__ = ["MetisLinear", "set_step"]


class _MetisLinearFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, w, mod):
        lead = x.shape[:-1]
        x2 = x.reshape(-1, x.shape[-1]).contiguous()
        # X is the K-along-columns operand of Y = X W and the K-along-rows
        # operand of dW = X^T D; W the reverse (Y = X W, then dX = D W^T)
        both = metis.AXIS0 | metis.AXIS1
        qx = metis.prepare_operand(x2, mod.cfg, True, mod.tags["X"], mod.step, mod._factors("X", x2), both)
        qw = metis.prepare_operand(w.detach(), mod.cfg, False, mod.tags["W"], mod.step, mod._factors("W", w), both)
        y = metis.gemm_fwd(qx, qw)
        ctx.mod, ctx.qx, ctx.qw, ctx.lead = mod, qx, qw, lead
        ctx.x_dtype = x.dtype
        mod.last = {"X": qx, "W": qw}
        return y.reshape(*lead, w.shape[1])

    @staticmethod
    def backward(ctx, dy):
        mod = ctx.mod
        d2 = dy.reshape(-1, dy.shape[-1]).contiguous().float()
        both = metis.AXIS0 | metis.AXIS1
        qd = metis.prepare_operand(d2, mod.cfg, True, mod.tags["D"], mod.step, mod._factors("D", d2), both)
        want_dx, want_dw = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        dx, dw = metis.gemm_bwd(qd, ctx.qw, ctx.qx, want_dx=want_dx, want_dw=want_dw)
        mod.last["D"] = qd
        gx = dx.reshape(*ctx.lead, dx.shape[1]).to(ctx.x_dtype) if want_dx else None
        return gx, dw if want_dw else None, None


class MetisLinear(torch.nn.Module):
    """y = x W (no bias) with W, X and the output gradient quantised through
    the spectral split.

    ``k``: rank of the split; ``s``: oversampling of the sketch; ``l_k``:
    rows sampled from X and D for the sketch (W is not sampled); ``refresh``:
    steps between re-sketches; ``rounding``: "sr" (the pages' default) or
    "rne"; ``seed`` and ``layer`` select the Philox streams.  The caller sets
    the training step with :func:`set_step` (a factor sketched at step t is
    reused while step - t < refresh).  Dimensions must be multiples of 16."""

    def __init__(self, in_features, out_features, k, s=8, l_k=0, refresh=8, rounding="sr", seed=0, layer=0,
                 device="cuda", weight=None):
        super().__init__()
        if weight is None:
            weight = torch.empty(in_features, out_features, dtype=torch.float32, device=device)
            torch.nn.init.normal_(weight, std=in_features ** -0.5)
        if tuple(weight.shape) != (in_features, out_features):
            raise ValueError("weight must be in_features x out_features")
        self.weight = torch.nn.Parameter(weight.to(device=device, dtype=torch.float32).contiguous())
        self.k = k
        self.cfg = metis.make_config(k=k, s=s, l_k=l_k, refresh=refresh,
                                     rounding=metis.SR if rounding == "sr" else metis.RNE, seed=seed)
        self.tags = {"X": metis.make_tag(layer, metis.OPERAND_X),
                     "W": metis.make_tag(layer, metis.OPERAND_W),
                     "D": metis.make_tag(layer, metis.OPERAND_D)}
        self.step = 0
        self.factors = {}
        self.last = {}

    def _factors(self, name, m):
        f = self.factors.get(name)
        if f is None or (f.rows, f.cols) != tuple(m.shape):
            f = metis.Factors(m.shape[0], m.shape[1], self.k, m.device)
            self.factors[name] = f
        return f

    def forward(self, x):
        return _MetisLinearFn.apply(x, self.weight, self)


def set_step(model, step):
    """Set the training step of every MetisLinear in ``model``."""
    for m in model.modules():
        if isinstance(m, MetisLinear):
            m.step = step
