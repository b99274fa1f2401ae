"""Seeded synthetic anisotropic operands (inputs only; none of the method's
arithmetic lives here, so both the HIP path and the CPU oracle may use it).

The Metis notes page (研究背景与动机) reports that under 3% of the singular
values dominate the spectrum: 0.63% for weights, 3.15% for activations and
2.91% for gradients.  An r x c operand is built as

    M = U diag(sigma) V^T + 0.01 N(0, 1)

with rho = min(r, c), n_dom = ceil(frac * rho) dominant values
sigma_i = 10**(1 + u_i), u_i ~ U[0, 1) sorted descending, a tail
sigma_i = i**-0.5 (global 1-based index i > n_dom), and U (r x rho), V (c x rho)
Haar-distributed (Q of the QR of a Gaussian, columns signed so diag(R) > 0).
The sum is formed in float32 or wider and rounded once to the target dtype.

Generator seeds: 1000 * config + 10 * operand + step (operand W=1, X=2, D=3).
"""

import math

import torch

FRAC_W = 0.0063
FRAC_X = 0.0315
FRAC_D = 0.0291
OPERAND_ID = {"W": 1, "X": 2, "D": 3}


def gen_seed(config, operand, step=0):
    return 1000 * config + 10 * OPERAND_ID[operand] + step


def n_dominant(rows, cols, frac):
    # small epsilon guards against binary rounding of frac * rho
    return int(math.ceil(frac * min(rows, cols) - 1e-9))


def spectrum(rho, n_dom, gen, dtype=torch.float64):
    """Dominant log-uniform values in [10, 100) then the i**-0.5 tail."""
    u = torch.rand(n_dom, generator=gen, dtype=torch.float64, device=gen.device)
    dom = torch.sort(10.0 ** (1.0 + u), descending=True).values
    i = torch.arange(n_dom + 1, rho + 1, dtype=torch.float64, device=gen.device)
    return torch.cat([dom, i ** -0.5]).to(dtype)


def haar(rows, cols, gen, dtype=torch.float32):
    """rows x cols matrix with Haar-distributed orthonormal columns.  The
    Gaussian draw stays on the generator's device; the QR runs on the host in
    float64 (no device solver library is involved)."""
    g = torch.randn(rows, cols, generator=gen, dtype=dtype, device=gen.device)
    q, r = torch.linalg.qr(g.to(dtype=torch.float64, device="cpu"), mode="reduced")
    d = torch.sign(torch.diagonal(r))
    d[d == 0] = 1
    return (q * d).to(dtype=dtype, device=gen.device)


def _generator(seed, device):
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return gen


def anisotropic(rows, cols, frac, seed, out_dtype=torch.bfloat16, device="cpu",
                work_dtype=None, noise=0.01, return_parts=False, v=None):
    """One operand as described in the module docstring.

    ``v`` may supply the right singular basis (cols x rho) to reuse a subspace
    across steps.  With ``return_parts`` the float work-precision (U, sigma,
    V) are returned too."""
    if work_dtype is None:
        work_dtype = torch.float64 if str(device) == "cpu" else torch.float32
    gen = _generator(seed, device)
    rho = min(rows, cols)
    n_dom = n_dominant(rows, cols, frac)
    sigma = spectrum(rho, n_dom, gen, work_dtype)
    u = haar(rows, rho, gen, work_dtype)
    if v is None:
        v = haar(cols, rho, gen, work_dtype)
    m = (u * sigma) @ v.T.to(work_dtype)
    m += noise * torch.randn(rows, cols, generator=gen, dtype=work_dtype, device=device)
    out = m.to(out_dtype)
    if return_parts:
        return out, (u, sigma, v, n_dom)
    return out


def anisotropic_fast(rows, cols, frac, seed, out_dtype=torch.bfloat16, device="cuda",
                     basis=None, theta=0.0, noise=0.01, work_dtype=torch.float32):
    """Large-shape variant of :func:`anisotropic` (LLaMA-3-8B-sized operands).

    The dominant part is exact: U_dom (rows x n_dom) is Haar and the right
    basis comes from ``basis`` (cols x 2 n_dom, Haar; drawn when None), whose
    first n_dom columns are turned towards the next n_dom by ``theta``
    (the dominant subspace rotated by theta).  The tail sigma_i = i**-0.5 uses
    Gaussian bases with unit expected column norm instead of exactly
    orthonormal ones, which avoids full-width QRs; at these shapes the tail
    lies below the 0.01 N(0,1) noise floor.  Returns (M, basis)."""
    gen = _generator(seed, device)
    rho = min(rows, cols)
    n_dom = n_dominant(rows, cols, frac)
    sigma = spectrum(rho, n_dom, gen, work_dtype)
    u_dom = haar(rows, n_dom, gen, work_dtype)
    if basis is None:
        basis = haar(cols, 2 * n_dom, gen, work_dtype)
    c, s = math.cos(theta), math.sin(theta)
    v_dom = c * basis[:, :n_dom] + s * basis[:, n_dom:2 * n_dom]
    m = (u_dom * sigma[:n_dom]) @ v_dom.T
    nt = rho - n_dom
    if nt > 0:
        gu = torch.randn(rows, nt, generator=gen, dtype=work_dtype, device=device) / math.sqrt(rows)
        gv = torch.randn(cols, nt, generator=gen, dtype=work_dtype, device=device) / math.sqrt(cols)
        m.addmm_(gu * sigma[n_dom:], gv.T)
        del gu, gv
    m.add_(torch.randn(rows, cols, generator=gen, dtype=work_dtype, device=device), alpha=noise)
    return m.to(out_dtype), basis


def rotate_dominant(v, n_dom, theta):
    """Rotate each dominant right vector v_i in the plane (v_i, v_{n_dom+i})
    by angle theta; the partner turns the other way so V stays orthonormal."""
    v = v.clone()
    a = v[:, :n_dom].clone()
    b = v[:, n_dom:2 * n_dom].clone()
    c, s = math.cos(theta), math.sin(theta)
    v[:, :n_dom] = c * a + s * b
    v[:, n_dom:2 * n_dom] = -s * a + c * b
    return v


def drift_weight(w_master, seed, scale=1e-3):
    """W_{t+1} = W_t + scale * ||W_t||_F / sqrt(numel) * N(0, 1) (float master)."""
    gen = _generator(seed, w_master.device)
    step = scale * torch.linalg.norm(w_master) / math.sqrt(w_master.numel())
    return w_master + step * torch.randn(w_master.shape, generator=gen,
                                         dtype=w_master.dtype, device=w_master.device)


# ------------------------------------------------- seeded quantised operands --
# Random but valid NVFP4 operands (codes, E4M3 block scales, tensor scales,
# singular values) used as GEMM inputs by both the HIP path and the oracle.

def q4_arrays(n_outer, k_len, seed, zero_block_frac=0.02):
    """One quantised orientation as numpy arrays: codes uint8 [n_outer,
    k_len/2] (uniform random bytes), E4M3 scale bytes uint8 [n_outer,
    k_len/16] and a binary32 tensor scale.  The scale bytes cover every
    finite non-negative E4M3 value, 0x00 .. 0x7E (zero, the subnormals
    2^-9 .. 7 2^-9, normals up to 448), and each row holds at least one 448
    block, as a real tensor's rows do (its largest block maps to 448)."""
    import numpy as np
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(n_outer, k_len // 2), dtype=np.uint8)
    nb = k_len // 16
    scales = rng.integers(0x00, 0x7F, size=(n_outer, nb), dtype=np.uint8)
    scales[rng.random(scales.shape) < zero_block_frac] = 0
    scales[np.arange(n_outer), rng.integers(0, nb, size=n_outer)] = 0x7E
    ts = np.float32(2.0 ** rng.uniform(-6, -2))
    return codes, scales, ts


def qoperand_arrays(rows, cols, k, seed):
    """A quantised operand (rows x cols, rank k) as numpy arrays: residual
    orientations 'R0' (K = rows) and 'R1' (K = cols); for k > 0 factors 'U'
    (k x rows, blocked along rows), 'V' (k x cols) and descending binary32 'S'."""
    import numpy as np
    out = {"R0": q4_arrays(cols, rows, seed + 1), "R1": q4_arrays(rows, cols, seed + 2)}
    if k > 0:
        out["U"] = q4_arrays(k, rows, seed + 3)
        out["V"] = q4_arrays(k, cols, seed + 4)
        rng = np.random.default_rng(seed + 5)
        out["S"] = np.sort(rng.uniform(0.5, 40.0, size=k)).astype(np.float32)[::-1].copy()
    return out


def exact_factors(rows, cols, k, seed):
    """Factors whose product U diag(S) V^T is exact in binary32 (and in any
    wider format): U = a/16, V = b/16 with integers |a|, |b| <= 8, and S
    powers of two 2^3 .. 2^-2 (descending); every partial sum is a multiple
    of 2^-10 below 2^8.  Returns float32 numpy arrays U (rows x k), S (k),
    V (cols x k)."""
    import numpy as np
    rng = np.random.default_rng(seed)
    u = (rng.integers(-8, 9, size=(rows, k)) / 16.0).astype(np.float32)
    v = (rng.integers(-8, 9, size=(cols, k)) / 16.0).astype(np.float32)
    e = np.sort(rng.integers(-2, 4, size=k))[::-1]
    s = (2.0 ** e).astype(np.float32)
    return u, s, v


# ---------------------------------------------------------------- configs ---

C0 = dict(name="c0_fwd_256x512", X=(256, 512), W=(512, 512), k=8, s=8, l_k=64,
          rounding="rne", dtype=torch.float32)
C1 = dict(name="c1_gpt2_130m_mlp_up", X=(8192, 768), W=(768, 3072), D=(8192, 3072),
          k=12, s=8, l_k=82, rounding="sr", dtype=torch.bfloat16)
C2 = dict(name="c2_llama3_8b_q_proj", X=(16384, 4096), W=(4096, 4096), D=(16384, 4096),
          k=61, s=8, l_k=164, rounding="sr", dtype=torch.bfloat16)
C3 = dict(name="c3_llama3_8b_mlp_8step", tokens=16384, hidden=4096, ffn=14336,
          k=61, s=8, l_k=164, refresh=8, rounding="sr", dtype=torch.bfloat16)
C4 = dict(name="c4_activation_1m_x_4096", X=(1048576, 4096), k=61, s=8, l_k=10486,
          rounding="sr", dtype=torch.bfloat16)
CONFIGS = {0: C0, 1: C1, 2: C2, 3: C3, 4: C4}
FRACS = {"W": FRAC_W, "X": FRAC_X, "D": FRAC_D}


def layer_operands(config, device="cpu", step=0):
    """(X, W, D) of config 0/1/2 (D is None for config 0)."""
    cfg = CONFIGS[config]
    out = {}
    for op in ("X", "W", "D"):
        if op not in cfg:
            out[op] = None
            continue
        r, c = cfg[op]
        out[op] = anisotropic(r, c, FRACS[op], gen_seed(config, op, step),
                              out_dtype=cfg["dtype"], device=device)
    return out["X"], out["W"], out["D"]
