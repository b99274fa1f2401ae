"""GPU parity of the MXFP4 path (metis_mxfp4_quantize, metis_mxfp4_gemm)
against oracle/mxfp4.py.

The quantiser's codes and E8M0 scales are exact in binary32 and must match
the oracle bit for bit, on both K axes and both input dtypes, including an
all-zero block, negative zeros, saturating blocks and tiny magnitudes, with
nearest and stochastic rounding.  The
GEMM's products are exact and only the fp32 accumulation rounds: every output
is held to the recursive-summation bound K * 2**-24 * (|A| |B|^T), on ragged
multi-tile shapes from oracle-made codes, end to end, and at the gate
projection's full size on sampled outputs."""

import numpy as np
import pytest
import torch

from oracle import mxfp4
from spectral_split_quantized_amd import metis, synth

from gpu_helpers import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X; none is visible")
    metis.load()
    torch.cuda.set_device(0)


def _inputs(rows, cols, seed, dtype, axis=1):
    """Gaussian values with a wide per-row (axis 1) or per-column (axis 0)
    magnitude spread, plus special blocks along K."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(rows, cols, generator=g, dtype=torch.float64)
    spread = torch.exp(torch.empty(rows if axis == 1 else cols).uniform_(-12, 12, generator=g))
    x = x * (spread[:, None] if axis == 1 else spread[None, :])
    xt = x if axis == 1 else x.T          # view with K along the last dimension
    xt[0, :32] = 0.0                      # all-zero block
    xt[1, :32] = -0.0                     # negative zeros
    xt[2, :32] = torch.linspace(-7.5, 7.5, 32, dtype=torch.float64)  # saturating block (amax 7.5)
    xt[3, 32:64] *= 1e-35                 # tiny magnitudes (bf16/fp32 subnormal range for some)
    return x.to(dtype).contiguous()


def _upload(q):
    codes, scales = q
    mx = metis.MX4(codes.shape[0], codes.shape[1] * 2)
    mx.codes.copy_(torch.from_numpy(codes))
    mx.scales.copy_(torch.from_numpy(scales))
    return mx


def _bound(a, b, k):
    """Elementwise bound of fp32 accumulation of k exact products."""
    return k * 2.0 ** -24 * (np.abs(mxfp4.dequantize(*a)) @ np.abs(mxfp4.dequantize(*b)).T) + 1e-300


@pytest.mark.parametrize("rounding", ["rne", "sr"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("axis,shape", [(1, (96, 160)), (0, (160, 96)), (1, (40, 1024)), (0, (1024, 72))])
def test_quantize_bit_exact(dtype, axis, shape, rounding):
    x = _inputs(*shape, 11 + shape[0], dtype, axis)
    say("mxfp4 quantize %s axis %d %s %s" % (tuple(shape), axis, dtype, rounding))
    r = metis.SR if rounding == "sr" else metis.RNE
    q = metis.mxfp4_quantize(x.cuda(), axis, rounding=r, seed=0x1234567890AB, tag=0x5A3C, step=7)
    metis.status_sync()
    oc, osc = mxfp4.quantize(x.double().numpy(), axis, rounding, seed=0x1234567890AB, tag=0x5A3C, step=7)
    assert np.array_equal(q.scales.cpu().numpy(), osc)
    assert np.array_equal(q.codes.cpu().numpy(), oc)


@pytest.mark.parametrize("M,N,K", [(264, 520, 1024), (256, 256, 2048), (8, 264, 3072)])
def test_gemm_matches_oracle(M, N, K):
    rng = np.random.default_rng(M + N + K)
    a = mxfp4.quantize(rng.standard_normal((M, K)) * np.exp(rng.uniform(-4, 4, (M, 1))))
    b = mxfp4.quantize(rng.standard_normal((N, K)) * np.exp(rng.uniform(-4, 4, (N, 1))))
    say("mxfp4 gemm %d x %d x %d" % (M, N, K))
    C = metis.mxfp4_gemm(_upload(a), _upload(b))
    metis.status_sync()
    want = mxfp4.gemm(a, b)
    err = np.abs(C.cpu().double().numpy() - want)
    assert np.all(err <= _bound(a, b, K))
    # and the rounding is that of fp32 accumulation, not of a lower precision
    assert err.max() <= 1e-5 * np.abs(want).max()


def test_gemm_leading_dimension_and_end_to_end():
    """GPU quantiser feeding the GPU GEMM (bf16 inputs, the weight quantised
    down its columns) against the oracle pipeline, output written into a wider
    row-major buffer."""
    M, N, K = 264, 520, 2048
    x = _inputs(M, K, 3, torch.bfloat16, 1)
    w = _inputs(K, N, 4, torch.bfloat16, 0)
    say("mxfp4 end to end %d x %d x %d" % (M, N, K))
    qx = metis.mxfp4_quantize(x.cuda(), 1)
    qw = metis.mxfp4_quantize(w.cuda(), 0)
    Cbuf = torch.full((M, N + 24), 7.0, dtype=torch.float32, device="cuda")
    metis.mxfp4_gemm(qx, qw, Cbuf[:, :N])
    metis.status_sync()
    a = mxfp4.quantize(x.double().numpy(), 1)
    b = mxfp4.quantize(w.double().numpy(), 0)
    assert np.array_equal(qx.codes.cpu().numpy(), a[0]) and np.array_equal(qw.codes.cpu().numpy(), b[0])
    got = Cbuf.cpu().double().numpy()
    assert np.all(got[:, N:] == 7.0)
    assert np.all(np.abs(got[:, :N] - mxfp4.gemm(a, b)) <= _bound(a, b, K))


def test_full_size_gate_projection_sampled():
    """The gate projection's shape (16384 x 4096 activations, 4096 x 14336
    weight; the bench's MXFP4 workload): codes of sampled rows and columns
    bit-exact, sampled outputs within the accumulation bound."""
    T, H, F = 16384, 4096, 14336
    X, _ = synth.anisotropic_fast(T, H, synth.FRAC_X, 21, device="cuda")
    W, _ = synth.anisotropic_fast(H, F, synth.FRAC_W, 22, device="cuda")
    say("mxfp4 full size %d x %d x %d" % (T, F, H))
    qx = metis.mxfp4_quantize(X, 1)
    qw = metis.mxfp4_quantize(W, 0)
    C = metis.mxfp4_gemm(qx, qw)
    metis.status_sync()
    rng = np.random.default_rng(5)
    rows = np.concatenate([rng.choice(T, 24, replace=False), [0, T - 1]])
    cols = np.concatenate([rng.choice(F, 24, replace=False), [0, F - 1]])
    a = mxfp4.quantize(X[rows].double().cpu().numpy(), 1)
    b = mxfp4.quantize(W[:, cols].double().cpu().numpy(), 0)
    assert np.array_equal(qx.codes[rows].cpu().numpy(), a[0]) and np.array_equal(qx.scales[rows].cpu().numpy(), a[1])
    assert np.array_equal(qw.codes[cols].cpu().numpy(), b[0]) and np.array_equal(qw.scales[cols].cpu().numpy(), b[1])
    got = C[rows][:, cols].cpu().double().numpy()
    assert np.all(np.abs(got - mxfp4.gemm(a, b)) <= _bound(a, b, H))


@pytest.mark.parametrize("axis", [1, 0])
def test_quantize_strided_input(axis):
    """A view into a wider row-major buffer (leading dimension > columns)."""
    wide = _inputs(96, 224, 17, torch.float32, axis)
    x = wide[:, :160] if axis == 1 else wide[:64, :200]
    say("mxfp4 quantize strided view %s (ld %d) axis %d" % (tuple(x.shape), x.stride(0), axis))
    q = metis.mxfp4_quantize(wide.cuda()[:x.shape[0], :x.shape[1]], axis)
    metis.status_sync()
    oc, osc = mxfp4.quantize(x.double().numpy(), axis)
    assert np.array_equal(q.scales.cpu().numpy(), osc) and np.array_equal(q.codes.cpu().numpy(), oc)


@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
@pytest.mark.parametrize("axis", [0, 1])
def test_quantize_non_finite_sets_numeric_status(axis, bad):
    """A NaN or an infinity anywhere in the operand is reported through the
    status word (E_NUMERIC at the next status_sync), and the flag clears."""
    say("MXFP4 non-finite input axis %d %s" % (axis, bad))
    M = torch.randn(64, 128, dtype=torch.float32, device="cuda")
    M[17, 45] = bad
    metis.mxfp4_quantize(M, axis)
    with pytest.raises(metis.MetisError) as ei:
        metis.status_sync()
    assert ei.value.status == metis.E_NUMERIC
    metis.mxfp4_quantize(torch.randn(64, 128, dtype=torch.float32, device="cuda"), axis)
    metis.status_sync()
