"""The quantiser's two schedules give the same codes.

Whole-tile bf16 operands (rows % 128 == 0, cols % 64 == 0) take the streaming
sweeps of quant_fast.hpp; everything else, and every call that exports the
residual, takes the general sweeps of quant.hpp, which the oracle parity
tests pin (and the streaming sweeps are pinned there too at full size).  Both
form the residual with the same MFMA chain and the same fused subtraction,
so on one input they must agree bit for bit: codes, scales and tensor scales
of both orientations and of the factors.  The shapes make the streaming
schedule walk one tile and four tiles per workgroup, with last chunks cut to
one and to three tiles by the operand's edge and work-item counts that are
not multiples of the eight XCDs, for every supported rank width."""

import numpy as np
import pytest
import torch

from spectral_split_quantized_amd import metis, synth

from gpu_helpers import gpu_factors, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X; none is visible")
    metis.load()
    torch.cuda.set_device(0)


def _equal(a, b, what):
    for name in ("R_ax0", "R_ax1", "U", "V"):
        qa, qb = getattr(a, name), getattr(b, name)
        if qa is None:
            continue
        for part in ("codes", "scales", "tensor_scale"):
            ta, tb = getattr(qa, part), getattr(qb, part)
            bad = int((ta != tb).sum().item())
            assert bad == 0, "%s %s %s: %d entries differ" % (what, name, part, bad)


@pytest.mark.parametrize("shape", [(1024, 16384), (1024, 28672), (2048, 16320), (1152, 16448), (16384, 4096), (384, 768)])
@pytest.mark.parametrize("k", [0, 12, 20, 40, 61])
@pytest.mark.parametrize("rounding", ["sr", "rne"])
def test_streaming_sweeps_equal_general_sweeps(shape, k, rounding):
    rows, cols = shape
    say("quantiser schedules %s k=%d %s" % (shape, k, rounding))
    M, _ = synth.anisotropic_fast(rows, cols, synth.FRAC_X, rows + cols + k, device="cuda")
    cfg = metis.make_config(k=max(k, 1), rounding=metis.SR if rounding == "sr" else metis.RNE, seed=5)
    tag = metis.make_tag(4, metis.OPERAND_D)
    f = None
    if k:
        u, s, v = synth.exact_factors(rows, cols, k, seed=k + rows)
        f = gpu_factors(u, s, v)
    both = metis.AXIS0 | metis.AXIS1
    fast = metis.quantize(M, cfg, tag, 6, both, factors=f)
    export = torch.empty(rows, cols, dtype=torch.float32, device="cuda")
    general = metis.quantize(M, cfg, tag, 6, both, factors=f, residual_out=export)
    metis.status_sync()
    _equal(fast, general, "%s k=%d" % (shape, k))


@pytest.mark.parametrize("axes", [1, 2])
def test_streaming_sweeps_single_axis(axes):
    rows, cols, k = 1024, 28672, 61
    M, _ = synth.anisotropic_fast(rows, cols, synth.FRAC_X, 17, device="cuda")
    u, s, v = synth.exact_factors(rows, cols, k, seed=3)
    f = gpu_factors(u, s, v)
    cfg = metis.make_config(k=k, rounding=metis.SR, seed=1)
    fast = metis.quantize(M, cfg, 0, 0, axes, factors=f)
    export = torch.empty(rows, cols, dtype=torch.float32, device="cuda")
    general = metis.quantize(M, cfg, 0, 0, axes, factors=f, residual_out=export)
    metis.status_sync()
    _equal(fast, general, "axes %d" % axes)


@pytest.mark.parametrize("k", [0, 61])
def test_streaming_sweeps_strided_rows(k):
    """M as a column slice of a wider matrix (leading dimension cols + 64):
    the streaming sweeps read rows at the leading dimension."""
    rows, cols = 1024, 16384
    wide, _ = synth.anisotropic_fast(rows, cols + 64, synth.FRAC_X, 23, device="cuda")
    M = wide[:, :cols]
    assert M.stride(0) == cols + 64
    cfg = metis.make_config(k=max(k, 1), rounding=metis.SR, seed=2)
    f = None
    if k:
        u, s, v = synth.exact_factors(rows, cols, k, seed=9)
        f = gpu_factors(u, s, v)
    both = metis.AXIS0 | metis.AXIS1
    fast = metis.quantize(M, cfg, 0, 3, both, factors=f)
    dense = metis.quantize(M.contiguous(), cfg, 0, 3, both, factors=f)
    export = torch.empty(rows, cols, dtype=torch.float32, device="cuda")
    general = metis.quantize(M, cfg, 0, 3, both, factors=f, residual_out=export)
    metis.status_sync()
    _equal(fast, dense, "strided vs contiguous")
    _equal(fast, general, "strided streaming vs general")


@pytest.mark.parametrize("k", [0, 61])
@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
def test_streaming_sweeps_non_finite_status(k, bad):
    """The streaming sweeps (whole-tile bf16 operand) report a NaN or an
    infinity in M through the status word, with and without factors, and
    the flag clears afterwards."""
    rows, cols = 1024, 16384
    say("streaming sweeps non-finite input k=%d %s" % (k, bad))
    M, _ = synth.anisotropic_fast(rows, cols, synth.FRAC_X, 31, device="cuda")
    M[300, 9001] = bad
    cfg = metis.make_config(k=max(k, 1), rounding=metis.SR, seed=4)
    f = None
    if k:
        u, s, v = synth.exact_factors(rows, cols, k, seed=6)
        f = gpu_factors(u, s, v)
    metis.quantize(M, cfg, 0, 2, metis.AXIS0 | metis.AXIS1, factors=f)
    with pytest.raises(metis.MetisError) as ei:
        metis.status_sync()
    assert ei.value.status == metis.E_NUMERIC
    M[300, 9001] = 0.0
    metis.quantize(M, cfg, 0, 2, metis.AXIS0 | metis.AXIS1, factors=f)
    metis.status_sync()
