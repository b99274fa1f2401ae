"""Run by test_abi_sanitized.py inside a process that preloads the ASan
runtime: confirms that the process loaded the sanitized library and drives
the host-side size and argument paths of every entry point."""

import ctypes
import os

import pytest

from spectral_split_quantized_amd import metis


@pytest.fixture(scope="module")
def lib():
    if not os.environ.get("METIS_LIBRARY"):
        pytest.skip("run by test_abi_sanitized.py only")
    return metis.load()


def test_sanitized_library_is_the_one_loaded(lib):
    maps = open("/proc/self/maps").read()
    assert os.environ["METIS_LIBRARY"] in maps
    assert "asan" in maps


def test_workspace_queries_over_shapes(lib):
    for rows, cols in ((1, 1), (16, 16), (256, 512), (16384, 14336), (1 << 20, 4096), (3, 100000)):
        for k in (0, 1, 12, 61, 64):
            assert lib.metis_quantize_workspace(rows, cols, k) > 0
            cfg = metis.make_config(k=max(k, 1), s=8, l_k=min(rows, 164))
            for sample in (0, 1):
                lib.metis_decompose_workspace(rows, cols, ctypes.byref(cfg), sample)
                lib.metis_prepare_operand_workspace(rows, cols, ctypes.byref(cfg), sample)


def test_static_capacity_and_errors(lib):
    assert metis.quantize_static_capacity() > 0
    assert lib.metis_last_error() is not None
