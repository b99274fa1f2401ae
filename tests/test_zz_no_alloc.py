"""GPU test of metis_quantize_static, the quantiser entry point that
allocates nothing (its scratch is the library's static per-GPU array).

Through the C ABI it must give the same codes, scales, tensor scales and
singular values as metis_quantize with a caller workspace, bit for bit, on two
calls in a row, the second with a smaller operand (the array keeps the first
call's contents, which must not leak into the second), for direct NVFP4 and
for the residual with factors; and an operand whose scratch exceeds the array
is refused before anything is enqueued."""

import numpy as np
import pytest
import torch

from spectral_split_quantized_amd import metis, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X; none is visible")
    metis.load()
    torch.cuda.set_device(0)
    # the set-up a graph-capturing caller does before capture; idempotent
    metis.init_device()
    metis.init_device()


def _factors(rows, cols, k, seed):
    u, s, v = synth.exact_factors(rows, cols, k, seed)
    f = metis.Factors(rows, cols, k)
    f.U.copy_(torch.from_numpy(u))
    f.S.copy_(torch.from_numpy(s))
    f.V.copy_(torch.from_numpy(v))
    return f


def _same(a, b):
    for name in ("R_ax0", "R_ax1", "U", "V"):
        qa, qb = getattr(a, name), getattr(b, name)
        if qa is None:
            assert qb is None
            continue
        assert torch.equal(qa.codes, qb.codes), name + " codes"
        assert torch.equal(qa.scales, qb.scales), name + " scales"
        assert torch.equal(qa.tensor_scale, qb.tensor_scale), name + " tensor scale"
    if a.S is not None:
        assert torch.equal(a.S, b.S)


@pytest.mark.parametrize("with_factors", [False, True])
def test_static_quantize_equals_workspace_quantize(with_factors):
    both = metis.AXIS0 | metis.AXIS1
    cfg = metis.make_config(k=12, rounding=metis.SR, seed=0)
    tag = metis.make_tag(2, metis.OPERAND_X)
    print("quantize_static vs quantize, factors %s" % with_factors, flush=True)
    for i, (rows, cols) in enumerate(((1024, 768), (256, 512))):  # the second call is smaller
        M, _ = synth.anisotropic_fast(rows, cols, synth.FRAC_X, 600 + i, device="cuda")
        f = _factors(rows, cols, 12, 40 + i) if with_factors else None
        ra = torch.empty(rows, cols, dtype=torch.float32, device="cuda") if with_factors else None
        rb = torch.empty_like(ra) if with_factors else None
        a = metis.quantize(M, cfg, tag, 3, both, factors=f, residual_out=ra)
        b = metis.quantize_static(M, cfg, tag, 3, both, factors=f, residual_out=rb)
        metis.status_sync()
        _same(a, b)
        if with_factors:
            assert torch.equal(ra, rb)


def test_static_quantize_refuses_operands_beyond_its_scratch():
    cap = metis.quantize_static_capacity()
    assert cap == 16 << 20
    rows, cols, k = 1 << 16, 4096, 61  # (rows + cols) * 6 * 64 bytes > 16 MiB
    M = torch.zeros(rows, cols, dtype=torch.bfloat16, device="cuda")
    f = metis.Factors(rows, cols, k)
    cfg = metis.make_config(k=k, rounding=metis.RNE)
    with pytest.raises(metis.MetisError) as ei:
        metis.quantize_static(M, cfg, 0, 0, metis.AXIS1, factors=f)
    assert ei.value.status == metis.E_UNSUPPORTED
    assert b"static" in metis.load().metis_last_error()
    metis.status_sync()
