"""CPU-side checks of the C-ABI library (no GPU calls): it loads, exports every
symbol include/metis.h declares, its host-side definitions of the random draws
agree with the oracle's independent ones, and argument errors are reported
synchronously."""

import ctypes
import os
import re

import numpy as np
import pytest

from oracle import philox, rsvd
from spectral_split_quantized_amd import metis

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "metis.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(metis_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = metis.load()
    names = _declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert lib.metis_abi_version() == 1


def test_init_device_reports_a_missing_gpu():
    """metis_init_device is the one call that sets up a device ahead of a
    graph capture: with no GPU it returns METIS_E_HIP with a message, it does
    not crash; with one it succeeds, and again at once."""
    lib = metis.load()
    from conftest import gpu_available
    if gpu_available():
        assert lib.metis_init_device() == metis.OK
        assert lib.metis_init_device() == metis.OK
    else:
        assert lib.metis_init_device() == metis.E_HIP
        assert lib.metis_last_error()


def test_omega_table_matches_oracle():
    ours = metis.omega_table_bits().astype(np.uint32)
    lib_vals = (ours << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(lib_vals, rsvd.omega_table())


def test_philox_matches_oracle():
    rng = np.random.default_rng(0)
    for _ in range(200):
        ctr = [int(v) for v in rng.integers(0, 2 ** 32, 4, dtype=np.uint64)]
        key = [int(v) for v in rng.integers(0, 2 ** 32, 2, dtype=np.uint64)]
        assert metis.philox_block(ctr, key) == philox.block(ctr, key)


def _expect(status, code):
    assert status == code, metis.load().metis_last_error()


def test_argument_errors_are_synchronous():
    lib = metis.load()
    cfg = metis.make_config(k=8, s=8, l_k=64)
    f = metis._Factors(None, None, None, 256, 512, 8, -1)
    # NULL operand
    _expect(lib.metis_decompose(None, 0, 256, 512, 512, ctypes.byref(cfg), 1, 0, 0, ctypes.byref(f),
                                None, 0, None), metis.E_INVALID)
    # k + s too large for the sample
    bad = metis.make_config(k=60, s=8, l_k=64)
    dummy = ctypes.c_void_p(16)
    f2 = metis._Factors(dummy, dummy, dummy, 256, 512, 60, -1)
    _expect(lib.metis_decompose(dummy, 0, 256, 512, 512, ctypes.byref(bad), 1, 0, 0, ctypes.byref(f2),
                                dummy, 1 << 30, None), metis.E_INVALID)
    # rank beyond the supported width
    huge = metis.make_config(k=120, s=8, l_k=4096)
    _expect(lib.metis_decompose(dummy, 0, 8192, 512, 512, ctypes.byref(huge), 1, 0, 0,
                                ctypes.byref(f2), dummy, 1 << 30, None), metis.E_INVALID)
    # ld < cols
    _expect(lib.metis_decompose(dummy, 0, 256, 512, 100, ctypes.byref(cfg), 1, 0, 0, ctypes.byref(f),
                                dummy, 1 << 30, None), metis.E_INVALID)
    # a row sample beyond the sampler's candidate capacity (2^27 rows)
    big_rows = (1 << 27) + 16
    fb = metis._Factors(dummy, dummy, dummy, big_rows, 512, 8, -1)
    _expect(lib.metis_decompose(dummy, 0, big_rows, 512, 512, ctypes.byref(cfg), 1, 0, 0, ctypes.byref(fb),
                                dummy, 1 << 40, None), metis.E_UNSUPPORTED)
    # the same operand as an unsampled weight is not limited by the sampler
    wide = metis.make_config(k=8, s=8, l_k=0)
    assert lib.metis_decompose(dummy, 0, big_rows, 512, 512, ctypes.byref(wide), 0, 0, 0, ctypes.byref(fb),
                               dummy, 16, None) == metis.E_WORKSPACE
    # quantise along an axis whose length is not a multiple of 16
    q = metis._QOperand(256, 24, 0, None)
    _expect(lib.metis_quantize(dummy, 0, 256, 24, 24, None, ctypes.byref(cfg), 0, 0, metis.AXIS1,
                               ctypes.byref(q), None, dummy, 1 << 30, None), metis.E_INVALID)
    # undersized workspace
    q4 = metis._Q4(dummy, dummy, dummy, 256, 512)
    q = metis._QOperand(256, 512, 0, None, metis._Q4(), metis._Q4(), metis._Q4(), q4)
    _expect(lib.metis_quantize(dummy, 0, 256, 512, 512, None, ctypes.byref(cfg), 0, 0, metis.AXIS1,
                               ctypes.byref(q), None, dummy, 16, None), metis.E_WORKSPACE)
    # GEMM with mismatched inner dimensions
    x = metis._QOperand(64, 32, 0, None)
    w = metis._QOperand(48, 16, 0, None)
    _expect(lib.metis_gemm_fwd(ctypes.byref(x), ctypes.byref(w), dummy, 16, dummy, 1 << 20, None),
            metis.E_INVALID)
    assert b"inner" in lib.metis_last_error()
    # the two-phase GEMM: same checks, plus the product selector
    _expect(lib.metis_gemm_fwd_prepare(ctypes.byref(x), ctypes.byref(w), dummy, 1 << 20, None), metis.E_INVALID)
    _expect(lib.metis_gemm_fwd_prepared(ctypes.byref(x), ctypes.byref(w), dummy, 16, dummy, 1 << 20, None),
            metis.E_INVALID)
    d = metis._QOperand(64, 16, 0, None)
    w2 = metis._QOperand(32, 16, 0, None)
    for which in (0, 4, -1):
        _expect(lib.metis_gemm_bwd_prepare(ctypes.byref(d), ctypes.byref(w2), ctypes.byref(x), which, dummy,
                                           1 << 20, None), metis.E_INVALID)
    _expect(lib.metis_gemm_bwd_prepare(None, ctypes.byref(w2), ctypes.byref(x), metis.GRAD_DX, dummy, 1 << 20,
                                       None), metis.E_INVALID)


def test_workspace_sizes_are_positive_and_monotone():
    lib = metis.load()
    cfg = metis.make_config(k=61, s=8, l_k=164)
    a = lib.metis_decompose_workspace(16384, 4096, ctypes.byref(cfg), 1)
    b = lib.metis_decompose_workspace(16384, 14336, ctypes.byref(cfg), 1)
    assert 0 < a < b
    assert lib.metis_quantize_workspace(4096, 4096, 61) > lib.metis_quantize_workspace(4096, 4096, 0) > 0


def test_mxfp4_argument_errors_are_synchronous():
    lib = metis.load()
    d = ctypes.c_void_p(4096)  # 16-byte aligned stand-in, never dereferenced
    # quantiser: null input, K not a multiple of 32, bad axis, misaligned codes
    _expect(lib.metis_mxfp4_quantize(None, 0, 64, 64, 64, 1, 0, 0, 0, 0, d, d, None), metis.E_INVALID)
    _expect(lib.metis_mxfp4_quantize(d, 0, 64, 48, 48, 1, 0, 0, 0, 0, d, d, None), metis.E_INVALID)
    _expect(lib.metis_mxfp4_quantize(d, 0, 48, 64, 64, 0, 0, 0, 0, 0, d, d, None), metis.E_INVALID)
    _expect(lib.metis_mxfp4_quantize(d, 0, 64, 64, 64, 2, 0, 0, 0, 0, d, d, None), metis.E_INVALID)
    _expect(lib.metis_mxfp4_quantize(d, 0, 64, 64, 64, 1, 0, 0, 0, 0, ctypes.c_void_p(4100), d, None), metis.E_INVALID)
    _expect(lib.metis_mxfp4_quantize(d, 0, 64, 64, 32, 1, 0, 0, 0, 0, d, d, None), metis.E_INVALID)
    _expect(lib.metis_mxfp4_quantize(d, 0, 64, 64, 64, 1, 7, 0, 0, 0, d, d, None), metis.E_INVALID)
    # GEMM: K not a multiple of 1024, M or N not a multiple of 8, ldc < N, misaligned scales, null C
    _expect(lib.metis_mxfp4_gemm(d, d, d, d, 64, 64, 512, d, 64, None), metis.E_UNSUPPORTED)
    _expect(lib.metis_mxfp4_gemm(d, d, d, d, 60, 64, 1024, d, 64, None), metis.E_UNSUPPORTED)
    _expect(lib.metis_mxfp4_gemm(d, d, d, d, 64, 64, 1024, d, 32, None), metis.E_INVALID)
    _expect(lib.metis_mxfp4_gemm(d, ctypes.c_void_p(4104), d, d, 64, 64, 1024, d, 64, None), metis.E_INVALID)
    _expect(lib.metis_mxfp4_gemm(d, d, d, d, 64, 64, 1024, None, 64, None), metis.E_INVALID)
    # an empty product is a no-op
    assert lib.metis_mxfp4_gemm(d, d, d, d, 0, 64, 1024, d, 64, None) == metis.OK


def test_header_is_plain_c99(tmp_path):
    """include/metis.h compiles as strict C99 with no warnings (no C++ or
    torch types in the boundary)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "h.c"
    src.write_text('#include "metis.h"\nint main(void) { return metis_abi_version() == 1 ? 0 : 1; }\n')
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I",
                        os.path.join(ROOT, "include"), "-c", str(src), "-o", str(tmp_path / "h.o")],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
