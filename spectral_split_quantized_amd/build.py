"""Build libmetis.so in-tree with hipcc for gfx950.

Usage: python -m spectral_split_quantized_amd.build
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
OUT = os.path.join(HERE, "libmetis.so")

# translation units and their extra flags: the register-dequant GEMM is
# scheduled for instruction-level parallelism (its expansion instructions
# must interleave with the matrix instructions of the same wave); the rest
# keeps the default strategy
UNITS = [
    ("metis.hip", []),
    ("gemm_big.hip", ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]),
]

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # keep every binary32 rounding of the quantiser explicit
    "-ffp-contract=off",
    # packed FP32 instructions are avoided on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose=False):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(OBJ, exist_ok=True)
    objs = []
    for src, extra in UNITS:
        obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
        _run([hipcc] + FLAGS + extra + ["-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    tmp = OUT + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp], verbose)
    os.replace(tmp, OUT)
    return OUT


# Host code under AddressSanitizer and UndefinedBehaviorSanitizer (the device
# code is built as usual): each sanitizer option applies to the host pass only.
HOST_SANITIZE = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=all",
    "-Xarch_host", "-fno-omit-frame-pointer",
]
SAN_OUT = os.path.join(OBJ, "libmetis_san.so")


def build_host_sanitized(verbose=False):
    """_build/libmetis_san.so: the C-ABI translation unit (metis.hip, all of
    the host-side argument checking, workspace carving and scheduling) with
    host ASan + UBSan, linked with the regular GEMM unit.  Load it with
    METIS_LIBRARY set to its path and the ASan runtime preloaded; only calls
    that need no GPU can run where there is none."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(OBJ, exist_ok=True)
    gemm_obj = os.path.join(OBJ, "gemm_big.o")
    if not os.path.exists(gemm_obj):
        build(verbose)
    obj = os.path.join(OBJ, "metis_san.o")
    flags = [f for f in FLAGS if f != "-O3"] + ["-O1", "-g"] + HOST_SANITIZE
    _run([hipcc] + flags + ["-c", os.path.join(CSRC, "metis.hip"), "-o", obj], verbose)
    tmp = SAN_OUT + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC"] + HOST_SANITIZE[:4] + [obj, gemm_obj, "-o", tmp],
         verbose)
    os.replace(tmp, SAN_OUT)
    return SAN_OUT


if __name__ == "__main__":
    build(verbose=True)
    print("built", OUT)
    sys.exit(0)
