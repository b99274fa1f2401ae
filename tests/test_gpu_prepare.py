"""GPU tests of metis_prepare_operand (decompose + quantise in one call, the
residual quantised from the projection while the rediagonalisation runs on a
second stream).

Against the two-call path on the same seeded inputs: the factors U, S, V and
their codes are the same computation and must match bit for bit; the
residual is formed as M - P V_old^T instead of M - U diag(S) V^T (equal in
exact arithmetic, the rotation being orthogonal), so the two binary32
residuals agree to rounding and only codes at a rounding boundary may
differ.  Against the float64 oracle: the whole pipeline, with the flip-rate
and output bounds of the end-to-end comparison (gpu_helpers.E2E_TOL)."""

import numpy as np
import pytest
import torch

from oracle import rsvd, split_gemm
from spectral_split_quantized_amd import metis, synth

from gpu_helpers import E2E_TOL, Layer, assert_e2e_codes, rel_fro, say, to_np

pytestmark = pytest.mark.gpu

RESID_TOL = 1e-5       # |residual difference| / max |M|
CODE_DIFF_FRAC = 1e-3  # residual codes allowed to differ (rounding boundaries)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X; none is visible")
    metis.load()
    torch.cuda.set_device(0)


def _layer(config):
    c = synth.CONFIGS[config]
    X, W, D = synth.layer_operands(config, device="cuda")
    return Layer(X, W, D, c["k"], c["s"], c["l_k"], c["rounding"], seed=0)


def _codes_differ(a, b):
    return float((a.codes != b.codes).float().mean().item())


@pytest.mark.parametrize("config", [0, 1])
@pytest.mark.parametrize("side", [True, False])
def test_prepare_matches_two_calls(config, side):
    L = _layer(config)
    say("prepare vs decompose + quantize, config %d, side stream %s" % (config, side))
    stream2 = torch.cuda.Stream() if side else None
    for n, M in L.mats().items():
        if M is None:
            continue
        rows, cols = M.shape
        fa = metis.Factors(rows, cols, L.cfg.k, M.device)
        fb = metis.Factors(rows, cols, L.cfg.k, M.device)
        for step in (0, 1, 2):  # a refresh step, then cached steps
            ra = torch.empty(rows, cols, dtype=torch.float32, device=M.device)
            rb = torch.empty_like(ra)
            metis.decompose(M, L.cfg, L.sample[n], L.tags[n], step, fa)
            qa = metis.quantize(M, L.cfg, L.tags[n], step, metis.AXIS0 | metis.AXIS1, factors=fa,
                                residual_out=ra)
            qb = metis.prepare_operand(M, L.cfg, L.sample[n], L.tags[n], step, fb,
                                       metis.AXIS0 | metis.AXIS1, residual_out=rb, side_stream=stream2)
            metis.status_sync()
            assert fa.refreshed_at == fb.refreshed_at
            for name in ("U", "S", "V"):
                ta, tb = getattr(fa, name), getattr(fb, name)
                assert torch.equal(ta, tb), "%s %s step %d differs" % (n, name, step)
            for name in ("U", "V"):
                a, b = getattr(qa, name), getattr(qb, name)
                assert torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales)
                assert torch.equal(a.tensor_scale, b.tensor_scale)
            mmax = M.abs().max().float().item()
            dr = (ra - rb).abs().max().item() / mmax
            fr0 = _codes_differ(qa.R_ax0, qb.R_ax0)
            fr1 = _codes_differ(qa.R_ax1, qb.R_ax1)
            say("  %s step %d: residual diff %.2e of max|M|, codes differing %.2e / %.2e" % (n, step, dr, fr0, fr1))
            assert dr <= RESID_TOL
            assert fr0 <= CODE_DIFF_FRAC and fr1 <= CODE_DIFF_FRAC


@pytest.mark.parametrize("config", [0, 1])
def test_prepare_end_to_end_matches_oracle(config):
    """Seeded X, W, D through prepare_operand (with a side stream) and the
    split GEMMs, against the whole oracle pipeline."""
    L = _layer(config)
    say("prepare end to end, config %d" % config)
    side = torch.cuda.Stream()
    q, oq = {}, {}
    for n, M in L.mats().items():
        if M is None:
            continue
        f = metis.Factors(M.shape[0], M.shape[1], L.cfg.k, M.device)
        q[n] = metis.prepare_operand(M, L.cfg, L.sample[n], L.tags[n], 0, f, metis.AXIS0 | metis.AXIS1,
                                     side_stream=side)
        m = to_np(M).astype(np.float64)
        v0 = rsvd.rsvd_sketch(m, L.ocfg, L.sample[n], L.tags[n], 0)
        u, s, v, _ = rsvd.project_rediag(m, v0)
        oq[n] = split_gemm.quantize_operand(m, u, s, v, L.rounding, L.seed, L.tags[n], 0)
        assert_e2e_codes(q[n], oq[n], n)
    Y = metis.gemm_fwd(q["X"], q["W"])
    metis.status_sync()
    errs = [rel_fro(Y.cpu().double().numpy(), split_gemm.gemm_fwd(oq["X"], oq["W"]))]
    if L.D is not None:
        dX, dW = metis.gemm_bwd(q["D"], q["W"], q["X"])
        metis.status_sync()
        wdx, wdw = split_gemm.gemm_bwd(oq["D"], oq["W"], oq["X"])
        errs += [rel_fro(dX.cpu().double().numpy(), wdx), rel_fro(dW.cpu().double().numpy(), wdw)]
    say("prepare end-to-end rel Frobenius errors: %s" % ", ".join("%.2e" % e for e in errs))
    assert max(errs) <= E2E_TOL
