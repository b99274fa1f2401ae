"""The CPU ABI tests again, against the library's host code built with
AddressSanitizer and UndefinedBehaviorSanitizer (build.build_host_sanitized):
argument checking, error reporting, workspace-size arithmetic and the
host-side random tables run without an out-of-bounds access, a
use-after-free or undefined behaviour.  The sanitized build takes about a
minute; it is reused while the sources are older than it."""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/lib/llvm/bin/clang"


def _asan_runtime():
    try:
        out = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                             text=True, check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return out if os.path.isabs(out) and os.path.exists(out) else None


def test_abi_checks_under_host_sanitizers():
    from spectral_split_quantized_amd import build
    rt = _asan_runtime()
    if rt is None or not os.path.exists(os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")):
        pytest.skip("no hipcc / ASan runtime here")
    srcs = glob.glob(os.path.join(build.CSRC, "*"))
    if not os.path.exists(build.SAN_OUT) or os.path.getmtime(build.SAN_OUT) < max(os.path.getmtime(f) for f in srcs):
        build.build_host_sanitized()
    env = dict(os.environ, METIS_LIBRARY=build.SAN_OUT, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py"),
                        os.path.join(ROOT, "tests", "test_abi_sanitized_probe.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out and "skipped" not in out, out[-2000:]
