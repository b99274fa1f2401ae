"""Host-side checks of the autograd layer's wiring (no GPU work)."""

import pytest
import torch

from spectral_split_quantized_amd import metis
from spectral_split_quantized_amd.layer import MetisLinear, set_step


def test_layer_config_and_tags():
    lin = MetisLinear(32, 48, 4, s=8, l_k=16, refresh=5, rounding="rne", seed=3, layer=7, device="cpu")
    assert tuple(lin.weight.shape) == (32, 48) and lin.weight.dtype == torch.float32
    assert (lin.cfg.k, lin.cfg.s, lin.cfg.l_k, lin.cfg.refresh) == (4, 8, 16, 5)
    assert lin.cfg.rounding == metis.RNE and lin.cfg.seed == 3
    assert lin.tags == {"X": metis.make_tag(7, metis.OPERAND_X), "W": metis.make_tag(7, metis.OPERAND_W),
                        "D": metis.make_tag(7, metis.OPERAND_D)}
    assert len(set(lin.tags.values())) == 3


def test_layer_rejects_mis_shaped_weight():
    with pytest.raises(ValueError):
        MetisLinear(32, 48, 4, weight=torch.zeros(48, 32), device="cpu")


def test_set_step_reaches_every_layer():
    model = torch.nn.Sequential(MetisLinear(16, 32, 2, device="cpu"), torch.nn.GELU(),
                                MetisLinear(32, 16, 2, layer=1, device="cpu"))
    set_step(model, 9)
    assert [m.step for m in model if isinstance(m, MetisLinear)] == [9, 9]


def test_mxfp4_binding_rejects_mismatched_operands():
    a = metis.MX4(32, 1024, device="cpu")
    b = metis.MX4(32, 2048, device="cpu")
    with pytest.raises(ValueError):
        metis.mxfp4_gemm(a, b)
    with pytest.raises(ValueError):
        metis.mxfp4_quantize(torch.zeros(64, 64)[:, ::2], 1)
    with pytest.raises(ValueError):
        metis.mxfp4_quantize(torch.zeros(64, 64), 1, out=metis.MX4(32, 64, device="cpu"))


def test_gemm_bindings_reject_mis_shaped_outputs():
    x = metis.QOperand(64, 32, 0, metis.AXIS1, device="cpu")
    w = metis.QOperand(32, 48, 0, metis.AXIS0, device="cpu")
    with pytest.raises(ValueError):
        metis.gemm_fwd(x, w, Y=torch.empty(64, 40))
    with pytest.raises(ValueError):
        metis.gemm_fwd(x, w, Y=torch.empty(64, 48, dtype=torch.float64))
