"""ctypes binding of libmetis (include/metis.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  torch supplies device memory and the current HIP stream.  If the
library is missing the first call raises; there is no fallback.
"""

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# METIS_LIBRARY names another build of the same library (the CPU tests use it
# for a host-sanitized build); by default the in-tree libmetis.so
LIB_PATH = os.environ.get("METIS_LIBRARY") or os.path.join(HERE, "libmetis.so")

OK, E_INVALID, E_UNSUPPORTED, E_HIP, E_NUMERIC, E_WORKSPACE = 0, -1, -2, -3, -4, -5
BF16, F32 = 0, 1
RNE, SR = 0, 1
OPERAND_W, OPERAND_X, OPERAND_D = 1, 2, 3
AXIS0, AXIS1 = 1, 2


class MetisError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("metis status %d: %s" % (status, msg))
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [("k", ctypes.c_int32), ("s", ctypes.c_int32), ("l_k", ctypes.c_int64),
                ("refresh", ctypes.c_int32), ("rounding", ctypes.c_int32),
                ("seed", ctypes.c_uint64)]


class _Factors(ctypes.Structure):
    _fields_ = [("U", ctypes.c_void_p), ("S", ctypes.c_void_p), ("V", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("k", ctypes.c_int32),
                ("refreshed_at", ctypes.c_int64)]


class _Q4(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("tensor_scale", ctypes.c_void_p), ("n_outer", ctypes.c_int64),
                ("k_len", ctypes.c_int64)]


class _QOperand(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("k", ctypes.c_int32),
                ("S", ctypes.c_void_p), ("U", _Q4), ("V", _Q4), ("R_ax0", _Q4), ("R_ax1", _Q4)]


_lib = None


def load():
    """Load libmetis.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libmetis.so not found at %s; run python -m "
                          "spectral_split_quantized_amd.build" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    i32, i64, u32, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_size_t
    lib.metis_abi_version.restype = i32
    lib.metis_last_error.restype = ctypes.c_char_p
    lib.metis_decompose_workspace.argtypes = [i64, i64, ctypes.POINTER(Config), i32]
    lib.metis_decompose_workspace.restype = sz
    lib.metis_quantize_workspace.argtypes = [i64, i64, i32]
    lib.metis_quantize_workspace.restype = sz
    lib.metis_gemm_fwd_workspace.argtypes = [ctypes.POINTER(_QOperand)] * 2
    lib.metis_gemm_fwd_workspace.restype = sz
    lib.metis_gemm_bwd_workspace.argtypes = [ctypes.POINTER(_QOperand)] * 3
    lib.metis_gemm_bwd_workspace.restype = sz
    lib.metis_mxfp4_quantize.argtypes = [P, i32, i64, i64, i64, i32, i32, ctypes.c_uint64, u32, i64, P, P, P]
    lib.metis_mxfp4_quantize.restype = i32
    lib.metis_mxfp4_gemm.argtypes = [P, P, P, P, i64, i64, i64, P, i64, P]
    lib.metis_mxfp4_gemm.restype = i32
    lib.metis_decompose.argtypes = [P, i32, i64, i64, i64, ctypes.POINTER(Config), i32, u32, i64,
                                    ctypes.POINTER(_Factors), P, sz, P]
    lib.metis_decompose.restype = i32
    lib.metis_quantize.argtypes = [P, i32, i64, i64, i64, ctypes.POINTER(_Factors),
                                   ctypes.POINTER(Config), u32, i64, i32,
                                   ctypes.POINTER(_QOperand), P, P, sz, P]
    lib.metis_quantize.restype = i32
    lib.metis_quantize_static.argtypes = [P, i32, i64, i64, i64, ctypes.POINTER(_Factors),
                                          ctypes.POINTER(Config), u32, i64, i32,
                                          ctypes.POINTER(_QOperand), P, P]
    lib.metis_quantize_static.restype = i32
    lib.metis_quantize_static_capacity.restype = sz
    lib.metis_prepare_operand_workspace.argtypes = [i64, i64, ctypes.POINTER(Config), i32]
    lib.metis_prepare_operand_workspace.restype = sz
    lib.metis_prepare_operand.argtypes = [P, i32, i64, i64, i64, ctypes.POINTER(Config), i32, u32, i64,
                                          ctypes.POINTER(_Factors), i32, ctypes.POINTER(_QOperand), P, P,
                                          sz, P, P]
    lib.metis_prepare_operand.restype = i32
    lib.metis_gemm_fwd.argtypes = [ctypes.POINTER(_QOperand), ctypes.POINTER(_QOperand), P, i64, P,
                                   sz, P]
    lib.metis_gemm_fwd.restype = i32
    lib.metis_gemm_bwd.argtypes = [ctypes.POINTER(_QOperand)] * 3 + [P, i64, P, i64, P, sz, P]
    lib.metis_gemm_bwd.restype = i32
    lib.metis_gemm_fwd_prepare.argtypes = [ctypes.POINTER(_QOperand)] * 2 + [P, sz, P]
    lib.metis_gemm_fwd_prepare.restype = i32
    lib.metis_gemm_fwd_prepared.argtypes = [ctypes.POINTER(_QOperand)] * 2 + [P, i64, P, sz, P]
    lib.metis_gemm_fwd_prepared.restype = i32
    lib.metis_gemm_bwd_prepare.argtypes = [ctypes.POINTER(_QOperand)] * 3 + [i32, P, sz, P]
    lib.metis_gemm_bwd_prepare.restype = i32
    lib.metis_gemm_bwd_prepared.argtypes = [ctypes.POINTER(_QOperand)] * 3 + [P, i64, P, i64, P, sz, P]
    lib.metis_gemm_bwd_prepared.restype = i32
    lib.metis_status_sync.argtypes = [P]
    lib.metis_status_sync.restype = i32
    lib.metis_init_device.argtypes = []
    lib.metis_init_device.restype = i32
    lib.metis_omega_table.argtypes = [P]
    lib.metis_omega_table.restype = None
    lib.metis_timing_enable.argtypes = [i32]
    lib.metis_timing_kinds.argtypes = [i32]
    lib.metis_timing_kinds.restype = i32
    lib.metis_timing_enable.restype = i32
    lib.metis_timing_read.argtypes = [P, P, i32]
    lib.metis_timing_read.restype = i32
    lib.metis_philox4x32_10.argtypes = [ctypes.POINTER(ctypes.c_uint32)] * 3
    lib.metis_philox4x32_10.restype = None
    _lib = lib
    return lib


def _check(status):
    if status != OK:
        raise MetisError(status, load().metis_last_error().decode(errors="replace"))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _rows_check(M):
    """The boundary takes row-major matrices with a leading dimension: the
    elements of a row must be contiguous."""
    if M.dim() != 2 or (M.shape[1] > 1 and M.stride(1) != 1):
        raise ValueError("M must be a 2-D row-major view (stride(1) == 1), got strides %s" % (M.stride(),))


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError("operands must be bfloat16 or float32, got %s" % t.dtype)


def make_config(k, s=8, l_k=0, refresh=8, rounding=RNE, seed=0):
    return Config(k, s, l_k, refresh, rounding, seed)


def make_tag(layer, operand):
    return ((layer & 0xFFFF) << 16) | ((operand & 0xF) << 12)


class Factors:
    """Device factors U (rows x k), S (k), V (cols x k) and the cache state."""

    def __init__(self, rows, cols, k, device="cuda"):
        self.U = torch.empty(rows, k, dtype=torch.float32, device=device)
        self.S = torch.empty(k, dtype=torch.float32, device=device)
        self.V = torch.zeros(cols, k, dtype=torch.float32, device=device)
        self.rows, self.cols, self.k = rows, cols, k
        self.refreshed_at = -1

    def _c(self):
        return _Factors(self.U.data_ptr(), self.S.data_ptr(), self.V.data_ptr(), self.rows,
                        self.cols, self.k, self.refreshed_at)


class Q4:
    """One quantised orientation: codes [n_outer, k_len/2], scales
    [n_outer, k_len/16] (E4M3 bytes), tensor scale (1 float)."""

    def __init__(self, n_outer, k_len, device="cuda"):
        self.codes = torch.empty(n_outer, k_len // 2, dtype=torch.uint8, device=device)
        self.scales = torch.empty(n_outer, k_len // 16, dtype=torch.uint8, device=device)
        self.tensor_scale = torch.empty(1, dtype=torch.float32, device=device)
        self.n_outer, self.k_len = n_outer, k_len

    def _c(self):
        return _Q4(self.codes.data_ptr(), self.scales.data_ptr(), self.tensor_scale.data_ptr(),
                   self.n_outer, self.k_len)


class QOperand:
    """Quantised operand (rows x cols): Q(U), S, Q(V) and the residual in the
    requested K orientations."""

    def __init__(self, rows, cols, k, axes, device="cuda"):
        self.rows, self.cols, self.k = rows, cols, k
        self.U = Q4(k, rows, device) if k else None
        self.V = Q4(k, cols, device) if k else None
        self.R_ax0 = Q4(cols, rows, device) if axes & AXIS0 else None
        self.R_ax1 = Q4(rows, cols, device) if axes & AXIS1 else None
        # the library copies the factors' S here, so the operand keeps the
        # singular values its codes were made with
        self.S = torch.empty(k, dtype=torch.float32, device=device) if k else None

    def _c(self):
        z = _Q4(None, None, None, 0, 0)
        return _QOperand(self.rows, self.cols, self.k,
                         self.S.data_ptr() if self.S is not None else None,
                         self.U._c() if self.U else z, self.V._c() if self.V else z,
                         self.R_ax0._c() if self.R_ax0 else z,
                         self.R_ax1._c() if self.R_ax1 else z)



def _out_check(T, rows, cols, name):
    """A caller-provided output must be a float32 rows x cols row-major view:
    the library writes rows x cols values at its leading dimension."""
    if T.dtype != torch.float32 or tuple(T.shape) != (rows, cols) or T.stride(1) != 1:
        raise ValueError("%s must be a float32 %d x %d row-major matrix" % (name, rows, cols))
    return T

def _workspace(nbytes, device):
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def decompose(M, cfg, sample_rows, tag, step, factors, workspace=None):
    """Spectral split of M (metis_decompose); updates ``factors`` in place."""
    _rows_check(M)
    lib = load()
    rows, cols = M.shape
    need = lib.metis_decompose_workspace(rows, cols, ctypes.byref(cfg), int(sample_rows))
    ws = workspace if workspace is not None and workspace.numel() >= need else _workspace(need, M.device)
    fc = factors._c()
    _check(lib.metis_decompose(_ptr(M), _dtype_code(M), rows, cols, M.stride(0), ctypes.byref(cfg),
                               int(sample_rows), tag, step, ctypes.byref(fc), _ptr(ws), ws.numel(),
                               _stream()))
    factors.refreshed_at = fc.refreshed_at
    return factors


def quantize(M, cfg, tag, step, axes, factors=None, out=None, residual_out=None, workspace=None):
    """NVFP4 quantisation of M or of its residual (metis_quantize)."""
    _rows_check(M)
    lib = load()
    rows, cols = M.shape
    k = factors.k if factors is not None else 0
    if out is None:
        out = QOperand(rows, cols, k, axes, M.device)
    need = lib.metis_quantize_workspace(rows, cols, k)
    ws = workspace if workspace is not None and workspace.numel() >= need else _workspace(need, M.device)
    oc = out._c()
    fcp = ctypes.byref(factors._c()) if factors is not None else None
    _check(lib.metis_quantize(_ptr(M), _dtype_code(M), rows, cols, M.stride(0), fcp, ctypes.byref(cfg),
                              tag, step, axes, ctypes.byref(oc), _ptr(residual_out), _ptr(ws),
                              ws.numel(), _stream()))
    return out


def quantize_static(M, cfg, tag, step, axes, factors=None, out=None, residual_out=None):
    """metis_quantize without a workspace: the library's static per-GPU scratch
    (metis_quantize_static) serves as workspace, so the call allocates no
    device memory (``out`` given: none at all)."""
    _rows_check(M)
    lib = load()
    rows, cols = M.shape
    k = factors.k if factors is not None else 0
    if out is None:
        out = QOperand(rows, cols, k, axes, M.device)
    oc = out._c()
    fcp = ctypes.byref(factors._c()) if factors is not None else None
    _check(lib.metis_quantize_static(_ptr(M), _dtype_code(M), rows, cols, M.stride(0), fcp, ctypes.byref(cfg),
                                     tag, step, axes, ctypes.byref(oc), _ptr(residual_out), _stream()))
    return out


def quantize_static_capacity():
    """Bytes of the static scratch behind quantize_static."""
    return int(load().metis_quantize_static_capacity())


def prepare_operand(M, cfg, sample_rows, tag, step, factors, axes, out=None, residual_out=None,
                    workspace=None, side_stream=None):
    """Decompose and quantise M in one call (metis_prepare_operand): the
    residual sweeps run on the current stream while the rediagonalisation runs
    on ``side_stream`` (a torch.cuda.Stream; None: the current stream)."""
    _rows_check(M)
    lib = load()
    rows, cols = M.shape
    if out is None:
        out = QOperand(rows, cols, factors.k, axes, M.device)
    need = lib.metis_prepare_operand_workspace(rows, cols, ctypes.byref(cfg), int(sample_rows))
    ws = workspace if workspace is not None and workspace.numel() >= need else _workspace(need, M.device)
    fc, oc = factors._c(), out._c()
    side = ctypes.c_void_p(side_stream.cuda_stream) if side_stream is not None else None
    _check(lib.metis_prepare_operand(_ptr(M), _dtype_code(M), rows, cols, M.stride(0), ctypes.byref(cfg),
                                     int(sample_rows), tag, step, ctypes.byref(fc), axes, ctypes.byref(oc),
                                     _ptr(residual_out), _ptr(ws), ws.numel(), _stream(), side))
    factors.refreshed_at = fc.refreshed_at
    return out


def gemm_fwd(xq, wq, Y=None, workspace=None):
    """Y = X-hat W-hat (metis_gemm_fwd), binary32."""
    lib = load()
    if Y is None:
        Y = torch.empty(xq.rows, wq.cols, dtype=torch.float32, device=xq.R_ax1.codes.device)
    _out_check(Y, xq.rows, wq.cols, "Y")
    xc, wc = xq._c(), wq._c()
    need = lib.metis_gemm_fwd_workspace(ctypes.byref(xc), ctypes.byref(wc))
    ws = workspace if workspace is not None and workspace.numel() >= need else _workspace(need, Y.device)
    _check(lib.metis_gemm_fwd(ctypes.byref(xc), ctypes.byref(wc), _ptr(Y), Y.stride(0), _ptr(ws),
                              ws.numel(), _stream()))
    return Y


def gemm_bwd(dq, wq, xq, dX=None, dW=None, want_dx=True, want_dw=True, workspace=None):
    """(dX, dW) = (D-hat W-hat^T, X-hat^T D-hat) (metis_gemm_bwd), binary32."""
    lib = load()
    dev = (dq.R_ax1 or dq.R_ax0).codes.device
    if want_dx and dX is None:
        dX = torch.empty(dq.rows, wq.rows, dtype=torch.float32, device=dev)
    if want_dw and dW is None:
        dW = torch.empty(xq.cols, dq.cols, dtype=torch.float32, device=dev)
    if want_dx:
        _out_check(dX, dq.rows, wq.rows, "dX")
    if want_dw:
        _out_check(dW, xq.cols, dq.cols, "dW")
    dc, wc, xc = dq._c(), wq._c(), xq._c()
    need = lib.metis_gemm_bwd_workspace(ctypes.byref(dc), ctypes.byref(wc), ctypes.byref(xc))
    ws = workspace if workspace is not None and workspace.numel() >= need else _workspace(need, dev)
    _check(lib.metis_gemm_bwd(ctypes.byref(dc), ctypes.byref(wc), ctypes.byref(xc),
                              _ptr(dX) if want_dx else None, dX.stride(0) if want_dx else 0,
                              _ptr(dW) if want_dw else None, dW.stride(0) if want_dw else 0,
                              _ptr(ws), ws.numel(), _stream()))
    return dX, dW


GRAD_DX, GRAD_DW = 1, 2


def _gemm_ws(need, workspace):
    if workspace is None or workspace.numel() < need:
        raise ValueError("the two-phase GEMM needs a workspace of at least %d bytes, shared by both calls" % need)
    return workspace


def gemm_fwd_prepare(xq, wq, workspace):
    """Build the low-rank K-extension of Y = X-hat W-hat into ``workspace``
    (metis_gemm_fwd_prepare) on the current stream."""
    lib = load()
    xc, wc = xq._c(), wq._c()
    ws = _gemm_ws(lib.metis_gemm_fwd_workspace(ctypes.byref(xc), ctypes.byref(wc)), workspace)
    _check(lib.metis_gemm_fwd_prepare(ctypes.byref(xc), ctypes.byref(wc), _ptr(ws), ws.numel(), _stream()))


def gemm_fwd_prepared(xq, wq, workspace, Y=None):
    """Y = X-hat W-hat from a K-extension built by gemm_fwd_prepare into the
    same workspace (metis_gemm_fwd_prepared)."""
    lib = load()
    if Y is None:
        Y = torch.empty(xq.rows, wq.cols, dtype=torch.float32, device=xq.R_ax1.codes.device)
    _out_check(Y, xq.rows, wq.cols, "Y")
    xc, wc = xq._c(), wq._c()
    ws = _gemm_ws(lib.metis_gemm_fwd_workspace(ctypes.byref(xc), ctypes.byref(wc)), workspace)
    _check(lib.metis_gemm_fwd_prepared(ctypes.byref(xc), ctypes.byref(wc), _ptr(Y), Y.stride(0), _ptr(ws),
                                       ws.numel(), _stream()))
    return Y


def gemm_bwd_prepare(dq, wq, xq, workspace, which=GRAD_DX | GRAD_DW):
    """Build the K-extensions of the backward products selected by ``which``
    into ``workspace`` (metis_gemm_bwd_prepare) on the current stream."""
    lib = load()
    dc, wc, xc = dq._c(), wq._c(), xq._c()
    ws = _gemm_ws(lib.metis_gemm_bwd_workspace(ctypes.byref(dc), ctypes.byref(wc), ctypes.byref(xc)), workspace)
    _check(lib.metis_gemm_bwd_prepare(ctypes.byref(dc), ctypes.byref(wc), ctypes.byref(xc), int(which), _ptr(ws),
                                      ws.numel(), _stream()))


def gemm_bwd_prepared(dq, wq, xq, workspace, dX=None, dW=None, want_dx=True, want_dw=True):
    """(dX, dW) from K-extensions built by gemm_bwd_prepare into the same
    workspace (metis_gemm_bwd_prepared)."""
    lib = load()
    dev = (dq.R_ax1 or dq.R_ax0).codes.device
    if want_dx and dX is None:
        dX = torch.empty(dq.rows, wq.rows, dtype=torch.float32, device=dev)
    if want_dw and dW is None:
        dW = torch.empty(xq.cols, dq.cols, dtype=torch.float32, device=dev)
    if want_dx:
        _out_check(dX, dq.rows, wq.rows, "dX")
    if want_dw:
        _out_check(dW, xq.cols, dq.cols, "dW")
    dc, wc, xc = dq._c(), wq._c(), xq._c()
    ws = _gemm_ws(lib.metis_gemm_bwd_workspace(ctypes.byref(dc), ctypes.byref(wc), ctypes.byref(xc)), workspace)
    _check(lib.metis_gemm_bwd_prepared(ctypes.byref(dc), ctypes.byref(wc), ctypes.byref(xc),
                                       _ptr(dX) if want_dx else None, dX.stride(0) if want_dx else 0,
                                       _ptr(dW) if want_dw else None, dW.stride(0) if want_dw else 0,
                                       _ptr(ws), ws.numel(), _stream()))
    return dX, dW


def init_device():
    """Set up the library on the current device (metis_init_device); needed
    only before capturing library calls into a graph."""
    _check(load().metis_init_device())


def status_sync():
    """Synchronise the current stream and raise on a device numeric failure."""
    _check(load().metis_status_sync(_stream()))


def omega_table_bits():
    """The library's 65536 bf16 bit patterns of the Gaussian quantile table (host only)."""
    import numpy as np
    out = np.zeros(65536, dtype=np.uint16)
    load().metis_omega_table(out.ctypes.data_as(ctypes.c_void_p))
    return out


def philox_block(ctr, key):
    """The library's Philox4x32-10 block function (host only)."""
    c = (ctypes.c_uint32 * 4)(*ctr)
    k = (ctypes.c_uint32 * 2)(*key)
    o = (ctypes.c_uint32 * 4)()
    load().metis_philox4x32_10(c, k, o)
    return tuple(o)


def timing_enable(capacity):
    """Start recording HIP events around the main GEMM and quantiser kernels."""
    _check(load().metis_timing_enable(int(capacity)))


def timing_kinds(mask):
    """Record only the kernel kinds whose bits are set (bit 0: main GEMM,
    1: amax sweep, 2: quantise sweep, 3: MXFP4 GEMM)."""
    _check(load().metis_timing_kinds(int(mask)))


def timing_read(max_records=1 << 16):
    """[(kind, ms, d0, d1, d2, d3), ...] for the recorded kernels (and reset)."""
    import numpy as np
    ms = np.zeros(max_records, dtype=np.float32)
    shape = np.zeros(5 * max_records, dtype=np.int64)
    n = load().metis_timing_read(ms.ctypes.data_as(ctypes.c_void_p),
                                 shape.ctypes.data_as(ctypes.c_void_p), max_records)
    out = []
    for i in range(n):
        k, d0, d1, d2, d3 = (int(v) for v in shape[5 * i:5 * i + 5])
        out.append((k, float(ms[i]), d0, d1, d2, d3))
    return out


# ----------------------------------------------------------------- MXFP4 --

class MX4:
    """One MXFP4 operand (metis_mxfp4_quantize): codes [outer, K/2], E8M0
    scales [outer, K/32]."""

    def __init__(self, outer, k_len, device="cuda"):
        self.codes = torch.empty(outer, k_len // 2, dtype=torch.uint8, device=device)
        self.scales = torch.empty(outer, k_len // 32, dtype=torch.uint8, device=device)
        self.outer, self.k_len = outer, k_len


def mxfp4_quantize(M, axis, out=None, rounding=RNE, seed=0, tag=0, step=0):
    """MXFP4 codes and scales of M along K axis ``axis`` (1: along rows, 0:
    down columns, giving the quantised transpose), rounded to nearest (RNE)
    or stochastically (SR, draws from seed, tag and step)."""
    lib = load()
    if M.dim() != 2 or M.stride(1) != 1:
        raise ValueError("M must be a row-major matrix (unit column stride)")
    rows, cols = M.shape
    outer, k_len = (rows, cols) if axis == 1 else (cols, rows)
    if out is None:
        out = MX4(outer, k_len, M.device)
    elif (out.outer, out.k_len) != (outer, k_len):
        raise ValueError("out holds a %d x %d operand, not %d x %d" % (out.outer, out.k_len, outer, k_len))
    _check(lib.metis_mxfp4_quantize(_ptr(M), _dtype_code(M), rows, cols, M.stride(0), axis, rounding, seed,
                                    tag, step, _ptr(out.codes), _ptr(out.scales), _stream()))
    return out


def mxfp4_gemm(a, b, C=None):
    """C = A-hat B-hat^T of two MXFP4 operands (metis_mxfp4_gemm), binary32."""
    lib = load()
    if a.k_len != b.k_len:
        raise ValueError("inner dimensions differ: %d and %d" % (a.k_len, b.k_len))
    if C is None:
        C = torch.empty(a.outer, b.outer, dtype=torch.float32, device=a.codes.device)
    _out_check(C, a.outer, b.outer, "C")
    _check(lib.metis_mxfp4_gemm(_ptr(a.codes), _ptr(a.scales), _ptr(b.codes), _ptr(b.scales), a.outer,
                                b.outer, a.k_len, _ptr(C), C.stride(0), _stream()))
    return C
