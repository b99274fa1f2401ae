"""GPU tests of the autograd layer (spectral_split_quantized_amd.layer).

The layer is wiring only, so its forward output and both gradients must equal,
bit for bit, the library calls it stands for on the same operands, tags and
step; and the whole pipeline behind it must match the float64 oracle with the
flip-rate and output bounds of the end-to-end comparison (gpu_helpers)."""

import numpy as np
import pytest
import torch

from oracle import rsvd, split_gemm
from spectral_split_quantized_amd import metis, synth
from spectral_split_quantized_amd.layer import MetisLinear, set_step

from gpu_helpers import E2E_TOL, assert_e2e_codes, rel_fro, say, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X; none is visible")
    metis.load()
    torch.cuda.set_device(0)


def _layer(config, refresh=8):
    c = synth.CONFIGS[config]
    X, W, D = synth.layer_operands(config, device="cuda")
    lin = MetisLinear(W.shape[0], W.shape[1], c["k"], s=c["s"], l_k=c["l_k"], refresh=refresh,
                      rounding=c["rounding"], weight=W.float())
    return c, X, W, D, lin


@pytest.mark.parametrize("config", [0, 1])
def test_layer_equals_library_calls(config):
    c, X, W, D, lin = _layer(config)
    if D is None:
        g = torch.Generator(device="cuda").manual_seed(7)
        D = torch.randn(X.shape[0], W.shape[1], device="cuda", generator=g) * 1e-2
    say("layer vs library calls, config %d, X %s W %s" % (config, tuple(X.shape), tuple(W.shape)))
    for step in (0, 1):  # a refresh step, then a cached one
        set_step(lin, step)
        x = X.clone().requires_grad_(True)
        lin.weight.grad = None
        y = lin(x)
        y.backward(D.float())
        # the same calls by hand, with their own factor caches replayed to this step
        both = metis.AXIS0 | metis.AXIS1
        f = {n: metis.Factors(m.shape[0], m.shape[1], c["k"]) for n, m in (("X", X), ("W", W), ("D", D))}
        for t in range(step + 1):
            q = {n: metis.prepare_operand(m, lin.cfg, n != "W", lin.tags[n], t, f[n], both)
                 for n, m in (("X", X), ("W", W.float()), ("D", D.float()))}
        y_ref = metis.gemm_fwd(q["X"], q["W"])
        dx_ref, dw_ref = metis.gemm_bwd(q["D"], q["W"], q["X"])
        metis.status_sync()
        assert torch.equal(y, y_ref), "forward differs at step %d" % step
        assert torch.equal(x.grad.float(), dx_ref.to(x.dtype).float()), "dX differs at step %d" % step
        assert torch.equal(lin.weight.grad, dw_ref), "dW differs at step %d" % step
        assert lin.factors["W"].refreshed_at == 0


def test_layer_end_to_end_matches_oracle():
    """Seeded X, W, D of the GPT-2 MLP-up shape through the layer's forward
    and backward, against the whole float64 oracle pipeline."""
    config = 1
    c, X, W, D, lin = _layer(config)
    say("layer end to end vs oracle, config %d" % config)
    x = X.clone().float().requires_grad_(True)
    y = lin(x)
    y.backward(D.float())
    metis.status_sync()
    ocfg = rsvd.Config(k=c["k"], s=c["s"], l_k=c["l_k"], refresh=8, rounding=c["rounding"], seed=0)
    oq = {}
    for n, M, sample in (("X", X, True), ("W", W, False), ("D", D, True)):
        m = to_np(M).astype(np.float64)
        v0 = rsvd.rsvd_sketch(m, ocfg, sample, lin.tags[n], 0)
        u, s, v, _ = rsvd.project_rediag(m, v0)
        oq[n] = split_gemm.quantize_operand(m, u, s, v, c["rounding"], 0, lin.tags[n], 0)
        assert_e2e_codes(lin.last[n], oq[n], n)
    wy = split_gemm.gemm_fwd(oq["X"], oq["W"])
    wdx, wdw = split_gemm.gemm_bwd(oq["D"], oq["W"], oq["X"])
    errs = [rel_fro(to_np(y).astype(np.float64), wy), rel_fro(to_np(x.grad).astype(np.float64), wdx),
            rel_fro(to_np(lin.weight.grad).astype(np.float64), wdw)]
    say("layer end-to-end rel Frobenius errors: %s" % ", ".join("%.2e" % e for e in errs))
    assert max(errs) <= E2E_TOL


def test_layer_refresh_period():
    """The weight's factor is re-sketched exactly at steps 0, refresh, 2 refresh."""
    c, X, W, D, lin = _layer(0, refresh=3)
    g = torch.Generator(device="cuda").manual_seed(11)
    dy = torch.randn(X.shape[0], W.shape[1], device="cuda", generator=g)
    seen = []
    for step in range(7):
        set_step(lin, step)
        lin(X.float()).backward(dy)
        seen.append(lin.factors["W"].refreshed_at)
    metis.status_sync()
    assert seen == [0, 0, 0, 3, 3, 3, 6]


def test_layer_batched_input_shape():
    """A (batch, sequence, features) input: the layer flattens the leading
    dimensions for the library and restores them on the output and gradient."""
    c, X, W, D, lin = _layer(1)
    x = X.float().reshape(4, X.shape[0] // 4, X.shape[1]).clone().requires_grad_(True)
    y = lin(x)
    assert tuple(y.shape) == (4, X.shape[0] // 4, W.shape[1])
    y.backward(D.float().reshape(4, -1, W.shape[1]))
    metis.status_sync()
    assert tuple(x.grad.shape) == tuple(x.shape) and tuple(lin.weight.grad.shape) == tuple(W.shape)
    # the same numbers as the flat call on the same step
    lin2 = MetisLinear(W.shape[0], W.shape[1], c["k"], s=c["s"], l_k=c["l_k"], rounding=c["rounding"],
                       weight=W.float())
    x2 = X.float().clone().requires_grad_(True)
    y2 = lin2(x2)
    y2.backward(D.float())
    metis.status_sync()
    assert torch.equal(y.reshape(y2.shape), y2)
    assert torch.equal(x.grad.reshape(x2.grad.shape), x2.grad)
    assert torch.equal(lin.weight.grad, lin2.weight.grad)


def test_layer_two_forwards_before_backward():
    """Two forwards of one module on different inputs, then both backwards (a
    weight-shared layer, micro-batches in flight): each backward uses the
    quantised operands and singular values of its own forward, so its
    gradients equal those of a lone forward + backward at the same step.  The
    module refreshes every step and the second forward runs at step 1, so its
    factors overwrite those the first forward quantised with."""
    c, X, W, D, lin = _layer(0, refresh=1)
    g = torch.Generator(device="cuda").manual_seed(5)
    X2 = X.float() + 0.5 * torch.randn(X.shape, device="cuda", generator=g)
    D1 = torch.randn(X.shape[0], W.shape[1], device="cuda", generator=g)
    D2 = torch.randn(X.shape[0], W.shape[1], device="cuda", generator=g)
    say("layer: two forwards, then both backwards")

    def lone(xin, dout, step):
        ref = MetisLinear(W.shape[0], W.shape[1], c["k"], s=c["s"], l_k=c["l_k"], refresh=1,
                          rounding=c["rounding"], weight=W.float())
        set_step(ref, step)
        xr = xin.clone().requires_grad_(True)
        ref(xr).backward(dout)
        metis.status_sync()
        return xr.grad, ref.weight.grad

    dx1, dw1 = lone(X.float(), D1, 0)
    dx2, dw2 = lone(X2, D2, 1)
    x1 = X.float().clone().requires_grad_(True)
    x2 = X2.clone().requires_grad_(True)
    set_step(lin, 0)
    y1 = lin(x1)
    set_step(lin, 1)
    y2 = lin(x2)          # re-sketches X and W: the first forward's factors are overwritten
    set_step(lin, 0)
    y1.backward(D1)       # D sketched at step 0, as in the lone run
    metis.status_sync()
    assert torch.equal(x1.grad, dx1)
    assert torch.equal(lin.weight.grad, dw1)
    set_step(lin, 1)
    y2.backward(D2)
    metis.status_sync()
    assert torch.equal(x2.grad, dx2)
    assert torch.equal(lin.weight.grad, dw1 + dw2)
