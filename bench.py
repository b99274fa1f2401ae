#!/usr/bin/env python
"""Benchmark: Metis spectral-split NVFP4 forward + backward on one MI355X.

Workload (the 8-step LLaMA-3-8B MLP case): 16384 tokens, hidden 4096, FFN
14336; projections gate and up (4096 -> 14336, sharing X) and down
(14336 -> 4096), bf16 inputs; rank k = 61, oversampling 8, 1% row sample
(164 rows), stochastic rounding, factors sketched every 8 steps and reused in
between.  Weights drift each step (W += 1e-3 ||W||_F / sqrt(numel) N(0,1));
activations and gradients are redrawn each step with their dominant right
subspace rotated by 0.01 rad per step; every step (warmup and timed) has
its own inputs, so both continue over the run.  A "step" is one pass of the whole
path over all three projections: decompose (sketch on refresh steps,
projection + rediag always), quantise (residual and factors, both K
orientations), split GEMM forward, split GEMM backward (dX and dW).

All inputs are synthetic and resident in HBM before the timed region starts.
The printed JSON line reports algorithmic TFLOP/s of the whole step, the
roofline of the dominant kernel (the main split-GEMM kernel, timed live with
HIP events on its stream) and the CPU oracle timed on a bounded sample.
Outside the timed region it also measures (unless --no-extras): the copy and
vendor bf16 GEMM ceilings of the GPU, plain NVFP4 (k = 0) through the same
kernels on the same workload (step time and quantisation error against
Metis), the GPT-2 130M MLP-up and LLaMA-3 8B q_proj projections on their
own (ms per step, TFLOP/s, rSVD ms of X, W and D), and the 1M x 4096
activation (decompose and quantise).
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Metis fwd+bwd layer TFLOP/s (8B MLP, 16K tok); rSVD ms; % of roofline"
PEAK_F16_TFLOPS = 2500.0      # MI355X dense fp16/bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E

TOKENS, HIDDEN, FFN = 16384, 4096, 14336
K_RANK, OVERSAMPLE, L_K, REFRESH = 61, 8, 164, 8
MAX_INPUT_STEPS = 64          # ~2 GB of bf16 inputs per step


# HBM traffic of the main split-GEMM kernel, bytes per launch averaged over
# the 18 launches of two steps (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE,
# on ``bench.py --steps 1 --warmup 1 --no-cpu-baseline --no-extras``; each counter scaled
# by what it reads for a plain 256 MiB copy, ``bench.py --copy-calibration``).
# The figure belongs to the kernel source it was taken on: if any file below
# changes, the stored figure no longer applies and ``traffic`` is reported null.
GEMM_TRAFFIC_BYTES = 1397967663
GEMM_TRAFFIC_SHA = "5ec41f2fe4a66bc1"
GEMM_SOURCES = ("common.hpp", "gemm_common.hpp", "gemm_reg.hpp", "gemm_launch.hpp", "gemm_big.hip")
# the same for both quantiser sweeps of one 16384 x 14336 residual (k = 61,
# SR, both orientations): FETCH_SIZE + WRITE_SIZE of the amax and quantise
# dispatches, scaled alike, per call
QUANT_TRAFFIC_BYTES = 1370589209
QUANT_TRAFFIC_SHA = "15dba22dd793e833"
QUANT_SOURCES = ("common.hpp", "quant.hpp", "quant_fast.hpp")


def source_sha(names):
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(os.path.dirname(os.path.abspath(__file__)), "spectral_split_quantized_amd", "csrc")
    for name in names:
        with open(os.path.join(d, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def gemm_source_sha():
    return source_sha(GEMM_SOURCES)


def mxfp4_only():
    """The MXFP4 variant alone on seeded gate-projection operands (16384 x
    4096 activations, 4096 x 14336 weight): one JSON line."""
    import torch
    from spectral_split_quantized_amd import metis, synth
    torch.cuda.set_device(0)
    metis.load()
    X, _ = synth.anisotropic_fast(TOKENS, HIDDEN, synth.FRAC_X, 1, device="cuda")
    W, _ = synth.anisotropic_fast(HIDDEN, FFN, synth.FRAC_W, 2, device="cuda")
    print(json.dumps(measure_mxfp4(metis, X, W, 0, None)), flush=True)
    return 0


def copy_calibration():
    """Three plain device-to-device copies of 256 MiB: the reference the PMC
    byte counters are scaled by."""
    import torch
    a = torch.empty(1 << 28, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": 1 << 28, "copy_bytes_written": 1 << 28, "launches": 3}))


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ------------------------------------------------------------- FLOP model --

def split_gemm_flops(M, N, K, kL, kR):
    """Algorithmic FLOP of one split product: the residual GEMM, the low-rank
    terms (P' J^T and H G) and the skinny products that build P' and G."""
    main = 2 * M * N * K
    lowrank = 2 * M * N * (kL + kR)
    skinny = 2 * M * K * kR + 2 * kL * K * N + 2 * kL * K * kR + 2 * kL * kR * N
    return main + lowrank + skinny


def decompose_flops(r, c, k, s, l_k, refresh):
    """Projection P = M V, Gram P^T P, U = P R; the sketch on refresh steps."""
    f = 2 * r * c * k + 2 * r * k * k + 2 * r * k * k
    if refresh:
        n = k + s
        f += 2 * l_k * c * n * 2 + 2 * l_k * n * n * 3
    return f


def residual_flops(r, c, k):
    return 2 * r * c * k


# ---------------------------------------------------------------- workload --

class Operand:
    def __init__(self, name, kind, layer, rows, cols):
        self.name, self.kind, self.layer = name, kind, layer
        self.rows, self.cols = rows, cols
        self.sample = kind != "W"


def operands():
    l, h, f = TOKENS, HIDDEN, FFN
    return [Operand("W_gate", "W", 0, h, f), Operand("W_up", "W", 1, h, f),
            Operand("W_down", "W", 2, f, h), Operand("X_gu", "X", 0, l, h),
            Operand("X_down", "X", 2, l, f), Operand("D_gate", "D", 0, l, f),
            Operand("D_up", "D", 1, l, f), Operand("D_down", "D", 2, l, h)]


PROJECTIONS = [("gate", "X_gu", "W_gate", "D_gate"), ("up", "X_gu", "W_up", "D_up"),
               ("down", "X_down", "W_down", "D_down")]


def build_inputs(n_steps, device):
    """Synthetic inputs for n_steps steps, all bf16 in HBM."""
    import torch
    from spectral_split_quantized_amd import synth
    seqs = {}
    for i, op in enumerate(operands()):
        frac = synth.FRACS[op.kind]
        base_seed = synth.gen_seed(3, op.kind) + 100 * op.layer
        if op.kind == "W":
            master, _ = synth.anisotropic_fast(op.rows, op.cols, frac, base_seed,
                                               out_dtype=torch.float32, device=device)
            seq = [master.to(torch.bfloat16)]
            for t in range(1, n_steps):
                master = synth.drift_weight(master, base_seed + 7919 * t)
                seq.append(master.to(torch.bfloat16))
            del master
        else:
            seq, basis = [], None
            for t in range(n_steps):
                m, basis = synth.anisotropic_fast(op.rows, op.cols, frac, base_seed + t,
                                                  device=device, basis=basis, theta=0.01 * t)
                seq.append(m)
        seqs[op.name] = seq
        torch.cuda.synchronize()
        log("  inputs %-7s %s x %d steps" % (op.name, tuple(seq[0].shape), n_steps))
    return seqs


class MetisMLP:
    """Persistent state of the path for the three projections: factor
    caches, quantised operands, outputs, one workspace per stream and one per
    split product.

    One step follows the layer's data dependencies on the main stream, two
    side streams and the main stream's companion: the weights (known when
    the step starts) are decomposed and quantised on the side streams while
    the main stream handles X_gu; the forward GEMMs wait for their weight;
    X_down follows the gate/up GEMMs and D_down the down GEMM (in a real
    layer they are computed from them); D_gate and D_up both come from the
    down projection's dX: D_gate is prepared on the main stream, D_up beside
    it on the side stream; the down projection's dW runs last.  Operands on
    the main stream rediagonalise on the companion while their residual is
    quantised, and the K-extension of every split product whose operands are
    ready early is built on the companion beside an earlier GEMM.  With
    streams=1 everything runs in that order on one stream."""

    def __init__(self, device, streams=3):
        import torch
        from spectral_split_quantized_amd import metis
        self.metis = metis
        self.torch = torch
        self.cfg = metis.make_config(k=K_RANK, s=OVERSAMPLE, l_k=L_K, refresh=REFRESH,
                                     rounding=metis.SR, seed=0)
        self.ops = {op.name: op for op in operands()}
        self.factors, self.q = {}, {}
        kind_id = {"W": metis.OPERAND_W, "X": metis.OPERAND_X, "D": metis.OPERAND_D}
        need = 0
        lib = metis.load()
        import ctypes
        for op in self.ops.values():
            op.tag = metis.make_tag(op.layer, kind_id[op.kind])
            self.factors[op.name] = metis.Factors(op.rows, op.cols, K_RANK, device)
            self.q[op.name] = metis.QOperand(op.rows, op.cols, K_RANK, metis.AXIS0 | metis.AXIS1, device)
            need = max(need, lib.metis_prepare_operand_workspace(op.rows, op.cols, ctypes.byref(self.cfg),
                                                                 int(op.sample)))
        self.out, self.gws = {}, {}
        for name, x, w, d in PROJECTIONS:
            X, W = self.ops[x], self.ops[w]
            self.out[name] = (torch.empty(X.rows, W.cols, dtype=torch.float32, device=device),
                              torch.empty(X.rows, W.rows, dtype=torch.float32, device=device),
                              torch.empty(W.rows, W.cols, dtype=torch.float32, device=device))
            xc, wc, dc = self.q[x]._c(), self.q[w]._c(), self.q[d]._c()
            # one workspace per split product: its K-extension stays there
            # from the prepare call to the GEMM
            self.gws[name] = (
                torch.empty(lib.metis_gemm_fwd_workspace(ctypes.byref(xc), ctypes.byref(wc)), dtype=torch.uint8,
                            device=device),
                torch.empty(lib.metis_gemm_bwd_workspace(ctypes.byref(dc), ctypes.byref(wc), ctypes.byref(xc)),
                            dtype=torch.uint8, device=device))
        self.nstreams = max(1, min(3, int(streams)))
        # default-priority streams only
        self.streams = [torch.cuda.current_stream(device)] + \
            [torch.cuda.Stream(device=device) for _ in range(self.nstreams - 1)]
        # companion of the main stream: the rediagonalisation of operands on
        # the critical path runs there while their residual is quantised
        self.side = torch.cuda.Stream(device=device) if self.nstreams > 1 else None
        self.ws = [torch.empty(need, dtype=torch.uint8, device=device) for _ in self.streams]
        self.free_gate = self.free_up = self.free_down = None
        log("  workspace %.1f MB x %d streams, %.1f MB for the split products"
            % (need / 1e6, self.nstreams, sum(a.numel() + b.numel() for a, b in self.gws.values()) / 1e6))

    def decompose(self, name, M, t):
        op = self.ops[name]
        self.metis.decompose(M, self.cfg, op.sample, op.tag, t, self.factors[name], workspace=self.ws[0])

    def _prep(self, name, t, inputs, si, companion=True):
        """Decompose and quantise one operand (both K orientations) on stream
        si; with ``companion`` the rediagonalisation runs on the main
        stream's companion (for operands on the critical path)."""
        m = self.metis
        op = self.ops[name]
        M = inputs[name][t % len(inputs[name])]
        side = self.side if companion else None
        with self.torch.cuda.stream(self.streams[si]):
            m.prepare_operand(M, self.cfg, op.sample, op.tag, t, self.factors[name], m.AXIS0 | m.AXIS1,
                              out=self.q[name], workspace=self.ws[si], side_stream=side)

    def _event(self, si):
        e = self.torch.cuda.Event()
        e.record(self.streams[si])
        return e

    def _names(self, name):
        _, x, w, d = next(p for p in PROJECTIONS if p[0] == name)
        return self.q[x], self.q[w], self.q[d]

    def _ext(self, name, kind, stream):
        """Build the K-extension of one split product ("fwd", "dx" or "dw")
        on ``stream``; returns an event that follows it."""
        m = self.metis
        X, W, D = self._names(name)
        wsf, wsb = self.gws[name]
        with self.torch.cuda.stream(stream):
            if kind == "fwd":
                m.gemm_fwd_prepare(X, W, wsf)
            else:
                m.gemm_bwd_prepare(D, W, X, wsb, which=m.GRAD_DX if kind == "dx" else m.GRAD_DW)
            e = self.torch.cuda.Event()
            e.record(stream)
        return e

    def _gemm(self, name, kind):
        """The main GEMM of one split product on the main stream, from the
        K-extension built by _ext."""
        m = self.metis
        X, W, D = self._names(name)
        Y, dX, dW = self.out[name]
        wsf, wsb = self.gws[name]
        if kind == "fwd":
            m.gemm_fwd_prepared(X, W, wsf, Y=Y)
        elif kind == "dx":
            m.gemm_bwd_prepared(D, W, X, wsb, dX=dX, want_dw=False)
        else:
            m.gemm_bwd_prepared(D, W, X, wsb, dW=dW, want_dx=False)

    def _ahead(self, name, kind, after):
        """The K-extension of a product whose GEMM comes later, built on the
        companion stream once the events ``after`` have fired (on the main
        stream when there is no companion)."""
        st = self.side if self.side is not None else self.streams[0]
        for e in after:
            st.wait_event(e)
        return self._ext(name, kind, st)

    def step(self, t, inputs):
        main = self.streams[0]
        sw = 1 if self.nstreams > 1 else 0
        sw2 = 2 if self.nstreams > 2 else sw
        # a side stream overwrites a weight's quantised operand once the
        # previous step's last GEMM reading it is done: the gate projection's
        # dW for W_gate (and the down projection's dX before it for W_down),
        # the up projection's dW for W_up.  A weight is also prepared only
        # after the previous step's gradient of that weight (W_down: the down
        # projection's dW, on the second side stream), as an optimizer
        # updates each weight as soon as its gradient is ready; the weights of
        # a step are thus prepared beside the previous step's last GEMMs.
        if self.free_gate is not None:
            self.streams[sw].wait_event(self.free_gate)
            self.streams[sw2].wait_event(self.free_up)

        ev = {}
        # the weights keep their rediagonalisation on their own stream (W_up
        # on the second side stream, so that at a refresh step its sketch
        # runs beside W_gate's instead of after it)
        for w, si in (("W_gate", sw), ("W_up", sw2), ("W_down", sw)):
            if w == "W_down" and self.free_down is not None:
                self.streams[si].wait_event(self.free_down)
            self._prep(w, t, inputs, si, companion=False)
            ev[w] = self._event(si)
        self._prep("X_gu", t, inputs, 0)
        x_ready = self._event(0)
        # forward: the up projection's K-extension is built beside the gate
        # projection's GEMM
        main.wait_event(ev["W_gate"])
        self._ext("gate", "fwd", main)
        self._gemm("gate", "fwd")
        e_up = self._ahead("up", "fwd", [x_ready, ev["W_up"]])
        main.wait_event(e_up)
        self._gemm("up", "fwd")
        # the previous step's down-projection dW (on a side stream) may still
        # read X_down, D_down and its K-extension, which are rewritten now
        if self.free_down is not None:
            main.wait_event(self.free_down)
        self._prep("X_down", t, inputs, 0)
        main.wait_event(ev["W_down"])
        self._ext("down", "fwd", main)
        self._gemm("down", "fwd")
        self._prep("D_down", t, inputs, 0)
        d_ready = self._event(0)
        # backward: dX of the down projection first (D_gate and D_up are
        # computed from it in a real layer); its dW, needed by nothing in the
        # step, then runs on the second side stream beside D_gate's
        # preparation on the main stream and D_up's on the first side stream
        # (with fewer streams it runs last on the main stream); every
        # K-extension that can be built ahead is built on the companion
        # stream beside an earlier GEMM
        self._ext("down", "dx", main)
        e_down_dw = self._ahead("down", "dw", [d_ready])
        self._gemm("down", "dx")
        dx_ready = self._event(0)
        if self.nstreams > 2:
            # the down projection's dW, needed by nothing in the step, runs on
            # the second side stream beside the D_gate and D_up preparations,
            # whose chains of small kernels leave most of the chip idle
            st2 = self.streams[sw2]
            st2.wait_event(dx_ready)
            st2.wait_event(e_down_dw)
            with self.torch.cuda.stream(st2):
                self._gemm("down", "dw")
            self.free_down = self._event(sw2)
        self.streams[sw].wait_event(dx_ready)
        self._prep("D_up", t, inputs, sw, companion=False)
        self._prep("D_gate", t, inputs, 0)
        g_ready = self._event(0)
        u_ready = self._event(sw)
        self._ext("gate", "dx", main)
        e_gate_dw = self._ahead("gate", "dw", [g_ready])
        self._gemm("gate", "dx")
        e_up_dx = self._ahead("up", "dx", [u_ready])
        e_up_dw = self._ahead("up", "dw", [])
        main.wait_event(e_gate_dw)
        self._gemm("gate", "dw")
        self.free_gate = self._event(0)
        main.wait_event(e_up_dx)
        self._gemm("up", "dx")
        main.wait_event(e_up_dw)
        self._gemm("up", "dw")
        self.free_up = self._event(0)
        if self.nstreams <= 2:
            main.wait_event(e_down_dw)
            self._gemm("down", "dw")

    def step_flops(self, t):
        refresh = (t % REFRESH) == 0
        f = 0
        for op in self.ops.values():
            lk = L_K if op.sample else op.rows
            f += decompose_flops(op.rows, op.cols, K_RANK, OVERSAMPLE, lk, refresh)
            f += residual_flops(op.rows, op.cols, K_RANK)
        for name, x, w, d in PROJECTIONS:
            X, W = self.ops[x], self.ops[w]
            l, mm, n = X.rows, X.cols, W.cols
            f += split_gemm_flops(l, n, mm, K_RANK, K_RANK)      # Y
            f += split_gemm_flops(l, mm, n, K_RANK, K_RANK)      # dX
            f += split_gemm_flops(mm, n, l, K_RANK, K_RANK)      # dW
        return f


def dense_equiv_flops():
    return 3 * 6 * TOKENS * HIDDEN * FFN


# ------------------------------------------------- measurements beside it --

def _median_ms(fn, reps):
    """Median wall time of fn() on the current stream (HIP events), after one
    untimed call."""
    import torch
    fn()
    torch.cuda.synchronize()
    evs = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in evs)
    return ts[len(ts) // 2]


def measure_ceilings(dev):
    """Practical ceilings on this GPU: a plain 1 GiB device copy (GB/s of
    bytes read + written) and the vendor library's dense bf16 GEMM at the
    gate projection's shape (torch.matmul -> hipBLASLt)."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    t_copy = _median_ms(lambda: dst.copy_(src), 10)
    del src, dst
    a = torch.randn(TOKENS, HIDDEN, device=dev).to(torch.bfloat16)
    b = torch.randn(HIDDEN, FFN, device=dev).to(torch.bfloat16)
    t_gemm = _median_ms(lambda: torch.matmul(a, b), 10)
    del a, b
    torch.cuda.empty_cache()
    return {"copy_GBps": round(2 * n / (t_copy * 1e-3) / 1e9, 1),
            "hipblaslt_bf16_TFLOPs": round(2 * TOKENS * HIDDEN * FFN / (t_gemm * 1e-3) / 1e12, 1),
            "hipblaslt_bf16_ms": round(t_gemm, 4), "gemm_shape_MNK": [TOKENS, FFN, HIDDEN]}


_E2M1 = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def dequant_q4(q4):
    """Dense binary32 values of one quantised orientation (n_outer x K): the
    E2M1 code (low nibble = even K index) times its E4M3 block scale times
    the tensor scale.  Measurement only."""
    import torch
    dev = q4.codes.device
    lut = torch.tensor(_E2M1 + tuple(-v for v in _E2M1), device=dev)
    c = q4.codes.to(torch.int64)
    vals = torch.stack((lut[c & 15], lut[c >> 4]), dim=-1).reshape(q4.codes.shape[0], -1)
    b = q4.scales.to(torch.int64)
    e, m = (b >> 3) & 15, (b & 7).to(torch.float32)
    sc = torch.where(e == 0, m * 2.0 ** -9, (8 + m) * torch.pow(2.0, (e - 10).to(torch.float32)))
    return vals * sc.repeat_interleave(16, dim=1) * q4.tensor_scale.float()


def tail_projector(M, r):
    """Projection onto the complements of M's top-r left and right singular
    subspaces, E -> (I - U U^T) E (I - V V^T).  U from the top-r eigenvectors
    of M M^T (M has no more rows than columns) by host LAPACK in float64,
    V = M^T U normalised.  Measurement only."""
    import scipy.linalg
    import torch
    Mf = M.float()
    G = (Mf @ Mf.T).double().cpu().numpy()
    n = G.shape[0]
    _, U = scipy.linalg.eigh(G, subset_by_index=[n - r, n - 1])
    U = torch.from_numpy(U).float().to(M.device)
    V = Mf.T @ U
    V = V / torch.linalg.norm(V, dim=0)

    def proj(E):
        E = E - U @ (U.T @ E)
        return E - (E @ V) @ V.T
    return proj


def operand_errors(M, qm, qd, V, tail_r=None):
    """Quantisation error of one operand for Metis (qm: factors + residual)
    and for plain NVFP4 (qd), in the K-along-columns orientation: over the
    whole matrix, and inside the residual subspace (the orthogonal
    complement of span(V), V = the cached right factor), where the pages
    place the small components that one block scale per 16 values flushes."""
    import torch
    Mf = M.float()
    U = dequant_q4(qm.U).T
    Vq = dequant_q4(qm.V).T
    metis_hat = (U * qm.S) @ Vq.T + dequant_q4(qm.R_ax1)
    plain_hat = dequant_q4(qd.R_ax1)

    def perp(A):
        return A - (A @ V) @ V.T
    ref_all, ref_perp = torch.linalg.norm(Mf), torch.linalg.norm(perp(Mf))
    # small values: below 1/8 of their 16-block's largest magnitude
    a = Mf.abs()
    small = a < a.reshape(a.shape[0], -1, 16).amax(dim=2).repeat_interleave(16, dim=1) / 8
    out = {}
    tail = tail_projector(M, tail_r) if tail_r else None
    for name, hat in (("metis", metis_hat), ("nvfp4", plain_hat)):
        E = hat - Mf
        out[name] = {"all": round(float(torch.linalg.norm(E) / ref_all), 6),
                     "residual_subspace": round(float(torch.linalg.norm(perp(E)) / ref_perp), 6),
                     "small_values_to_zero": round(float(((hat == 0) & small & (Mf != 0)).sum() / small.sum()), 6)}
        if tail is not None:
            out[name]["tail_two_sided"] = round(float(torch.linalg.norm(tail(E)) / torch.linalg.norm(tail(Mf))), 6)
    return out


def measure_direct(mlp, inputs, t_last, mlp_ms=None, steps=4, warmup=2, sample_rows=256):
    """The pages' comparison point: plain NVFP4 (k = 0) through the same
    quantiser and GEMM kernels.  Times whole steps (eight operands quantised
    in both orientations, the nine GEMMs) on one stream, and compares the
    forward outputs of both paths on the last timed step's inputs with the
    exact product X W on sampled rows."""
    import torch
    m = mlp.metis
    dev = mlp.streams[0].device
    q = {name: m.QOperand(op.rows, op.cols, 0, m.AXIS0 | m.AXIS1, dev) for name, op in mlp.ops.items()}
    out = {name: tuple(torch.empty_like(t) for t in mlp.out[name]) for name in mlp.out}
    ws = torch.empty(max(max(a.numel(), b.numel()) for a, b in mlp.gws.values()), dtype=torch.uint8, device=dev)

    def step(t):
        for name, op in mlp.ops.items():
            M = inputs[name][t % len(inputs[name])]
            m.quantize(M, mlp.cfg, op.tag, t, m.AXIS0 | m.AXIS1, out=q[name], workspace=mlp.ws[0])
        for name, x, w, d in PROJECTIONS:
            Y, dX, dW = out[name]
            m.gemm_fwd(q[x], q[w], Y=Y, workspace=ws)
            m.gemm_bwd(q[d], q[w], q[x], dX=dX, dW=dW, workspace=ws)

    for t in range(warmup):
        step(t)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for t in range(warmup, warmup + steps):
        step(t)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    step(t_last)
    m.status_sync()
    err = {}
    for name, x, w, d in PROJECTIONS:
        X = inputs[x][t_last % len(inputs[x])]
        W = inputs[w][t_last % len(inputs[w])]
        idx = torch.arange(0, X.shape[0], X.shape[0] // sample_rows, device=dev)
        exact = X[idx].float() @ W.float()

        def rel(Y):
            return float(torch.linalg.norm(Y[idx] - exact) / torch.linalg.norm(exact))
        err[name] = {"metis": round(rel(mlp.out[name][0]), 6), "nvfp4": round(rel(out[name][0]), 6)}
    ops = {}
    for name in ("X_gu", "W_gate", "D_gate"):
        M = inputs[name][t_last % len(inputs[name])]
        ops[name] = operand_errors(M, mlp.q[name], q[name], mlp.factors[name].V,
                                   tail_r=2 * K_RANK if name == "W_gate" else None)
    return {"ms_per_step": round(ms, 3), "streams": 1, "metis_over_nvfp4_time": round(mlp_ms / ms, 4) if mlp_ms else None,
            "y_rel_fro_err_vs_exact": err,
            "y_sample": "forward Y of each projection on %d evenly spaced token rows of the step-%d inputs"
                        % (sample_rows, t_last),
            "operand_rel_err": ops,
            "operand_note": "||M-hat - M|| / ||M|| over the matrix; the same ratio inside the orthogonal "
                            "complement of the cached right factor V (residual subspace); the fraction of values "
                            "below 1/8 of their 16-block's largest magnitude that dequantise to 0; for W_gate "
                            "also the two-sided tail metric ||P_u (M-hat - M) P_v|| / ||P_u M P_v|| with P_u, P_v "
                            "the projectors on the complements of W's top-2k singular subspaces"}


def measure_mxfp4(m, X, W, t_last, nvfp4_gemm_ms, reps=10, sample_rows=256):
    """The scaled-FP4 matrix-instruction variant: MXFP4 (block 32, E8M0
    power-of-two scales) operands of the gate projection, quantised by the
    library and multiplied on v_mfma_scale_f32_32x32x64_f8f6f4 with no
    expansion.  Times the GEMM at the gate shape (kind-3 HIP events on the
    launch stream, median of ``reps``) against the NVFP4 split GEMM's average
    from the timed steps, and reports the forward error against the exact
    product on the same sampled rows and inputs as ``direct_nvfp4``."""
    import torch
    T, H = X.shape
    F = W.shape[1]
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    qx = m.mxfp4_quantize(X, 1)
    qw = m.mxfp4_quantize(W, 0)
    b.record()
    C = m.mxfp4_gemm(qx, qw)
    m.status_sync()
    q_ms = a.elapsed_time(b)
    m.timing_kinds(1 << 3)
    m.timing_enable(reps)
    for _ in range(reps):
        m.mxfp4_gemm(qx, qw, C)
    recs = [r for r in m.timing_read() if r[0] == 3]
    m.timing_enable(0)
    m.timing_kinds(-1)
    ts = sorted(r[1] for r in recs)
    g_ms = ts[len(ts) // 2]
    flop = 2.0 * T * F * H
    tflops = flop / (g_ms * 1e-3) / 1e12
    idx = torch.arange(0, T, T // sample_rows, device=X.device)
    exact = X[idx].float() @ W.float()

    def rel(Y):
        return float(torch.linalg.norm(Y[idx] - exact) / torch.linalg.norm(exact))
    err = rel(C)
    # stochastic rounding, as the pages' default and the bench's NVFP4 path
    qxs = m.mxfp4_quantize(X, 1, rounding=m.SR, seed=0, tag=m.make_tag(0, m.OPERAND_X), step=t_last)
    qws = m.mxfp4_quantize(W, 0, rounding=m.SR, seed=0, tag=m.make_tag(0, m.OPERAND_W), step=t_last)
    err_sr = rel(m.mxfp4_gemm(qxs, qws))
    # plain NVFP4 with the same rounding (nearest), for a like-for-like error
    cfg = m.make_config(k=0, rounding=m.RNE)
    qxn = m.quantize(X, cfg, m.make_tag(0, m.OPERAND_X), 0, m.AXIS1)
    qwn = m.quantize(W, cfg, m.make_tag(0, m.OPERAND_W), 0, m.AXIS0)
    err_nv = rel(m.gemm_fwd(qxn, qwn))
    return {"shape_MNK": [T, F, H], "gemm_ms": round(g_ms, 4), "gemm_tflops": round(tflops, 1),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": 10100.0, "unit": "TFLOP/s",
                         "frac": round(tflops / 10100.0, 4), "dtype": "fp4 e2m1 x fp4 e2m1, e8m0 block scales"},
            "nvfp4_split_gemm_ms": round(nvfp4_gemm_ms, 4) if nvfp4_gemm_ms else None,
            "speedup_vs_nvfp4_split_gemm": round(nvfp4_gemm_ms / g_ms, 3) if nvfp4_gemm_ms else None,
            "quantize_both_operands_ms": round(q_ms, 3),
            "y_rel_fro_err_vs_exact": round(err, 6),
            "y_rel_fro_err_vs_exact_sr": round(err_sr, 6),
            "nvfp4_rne_y_rel_fro_err_vs_exact": round(err_nv, 6),
            "y_sample": "gate projection forward on %d evenly spaced token rows of the step-%d inputs (the rows "
                        "and inputs of direct_nvfp4)" % (sample_rows, t_last),
            "note": "a different format from the pages' NVFP4 (block 32 instead of 16, power-of-two scales, "
                    "no tensor scale, no spectral split; y_rel_fro_err_vs_exact rounds to nearest, _sr stochastically)"}


def decompose_timed(M, cfg, sample, tag, t, f, workspace=None):
    """metis_decompose on the current stream, timed with HIP events: (total
    ms, sketch ms, projection + rediagonalisation ms), the last two from the
    library's own event pairs (None where the call has no such part)."""
    import torch
    from spectral_split_quantized_amd import metis
    metis.timing_enable(8)
    metis.timing_kinds((1 << 4) | (1 << 5))
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    metis.decompose(M, cfg, sample, tag, t, f, workspace=workspace)
    b.record()
    torch.cuda.synchronize()
    parts = metis.timing_read(8)
    metis.timing_enable(0)
    metis.timing_kinds(-1)
    pick = [[r[1] for r in parts if r[0] == kind] for kind in (4, 5)]
    return (round(a.elapsed_time(b), 3),) + tuple(round(p[0], 3) if p else None for p in pick)


def measure_c4(dev, copy_gbps):
    """The 1M x 4096 activation (4.3e9 elements, l_k = 10486): decompose at a
    refresh and at a cached step, and the residual quantisation in both
    orientations, each timed alone."""
    import torch
    from spectral_split_quantized_amd import metis, synth
    c4 = synth.CONFIGS[4]
    rows, cols = c4["X"]
    k = c4["k"]
    M, _ = synth.anisotropic_fast(rows, cols, synth.FRAC_X, synth.gen_seed(4, "X"), device=dev)
    torch.cuda.synchronize()
    cfg = metis.make_config(k=k, s=c4["s"], l_k=c4["l_k"], refresh=REFRESH, rounding=metis.SR, seed=0)
    tag = metis.make_tag(0, metis.OPERAND_X)
    f = metis.Factors(rows, cols, k, dev)
    q = metis.QOperand(rows, cols, k, metis.AXIS0 | metis.AXIS1, dev)
    res = {}
    for label, t in (("decompose_refresh_ms", 0), ("decompose_cached_ms", 1)):
        res[label], sketch, proj = decompose_timed(M, cfg, True, tag, t, f)
        if t == 0:
            res["decompose_refresh_sketch_ms"], res["decompose_refresh_project_rediag_ms"] = sketch, proj
    t_q = _median_ms(lambda: metis.quantize(M, cfg, tag, 1, metis.AXIS0 | metis.AXIS1, factors=f, out=q), 5)
    metis.status_sync()
    # algorithmic bytes per element: M read twice (bf16), codes and scales of
    # two orientations, and the rank-k reconstruction operands
    per_elem = 2 * 2 + 2 * (0.5 + 1 / 16) + 2 * 4 * k / cols
    gbs = rows * cols * per_elem / (t_q * 1e-3) / 1e9
    res.update({"quantize_ms": round(t_q, 3), "quantize_GBps": round(gbs, 1),
                "quantize_frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
                "quantize_frac_copy": round(gbs / copy_gbps, 4) if copy_gbps else None,
                "bytes_per_elem": round(per_elem, 4), "shape": [rows, cols], "k": k, "l_k": c4["l_k"]})
    del M, f, q
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------ CPU baseline --

def host_cpu_model():
    """The host CPU's model name (Linux /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return None


def oracle_c0_single_thread():
    """The float64 oracle on the small single-layer workload (X 256 x 512, W
    512 x 512 fp32, k = 8, s = 8, l_k = 64, RNE; decompose and quantise X and
    W, forward GEMM) with its BLAS on one thread, in seconds (None if the
    thread count cannot be limited)."""
    import numpy as np
    from oracle import philox, rsvd, split_gemm
    from spectral_split_quantized_amd import synth
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        return None
    X, W, _ = synth.layer_operands(0)
    X = X.double().numpy()
    W = W.double().numpy()
    c = synth.CONFIGS[0]
    cfg = rsvd.Config(k=c["k"], s=c["s"], l_k=c["l_k"], refresh=REFRESH, rounding="rne", seed=0)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        q = {}
        for name, M, sample, oid in (("X", X, True, 2), ("W", W, False, 1)):
            tag = philox.make_tag(0, oid, 0)
            u, s, v, _ = rsvd.decompose(M, cfg, sample, tag, 0)
            q[name] = split_gemm.quantize_operand(M, u.astype(np.float32), s.astype(np.float32),
                                                  v.astype(np.float32), "rne", 0, tag, 0)
        split_gemm.gemm_fwd(q["X"], q["W"])
        return round(time.perf_counter() - t0, 3)


def cpu_baseline(inputs_cpu, tokens, ncols):
    """Time the float64 oracle on a bounded sample of the gate projection:
    `tokens` rows of X and D and the first `ncols` output columns of W."""
    import numpy as np
    from oracle import philox, rsvd, split_gemm
    X = inputs_cpu["X"][:tokens].astype(np.float64)
    W = inputs_cpu["W"][:, :ncols].astype(np.float64)
    D = inputs_cpu["D"][:tokens, :ncols].astype(np.float64)
    cfg = rsvd.Config(k=K_RANK, s=OVERSAMPLE, l_k=L_K, refresh=REFRESH, rounding="sr", seed=0)
    stages = {}

    def timed(key, fn):
        t = time.perf_counter()
        out = fn()
        stages[key] = round(time.perf_counter() - t, 3)
        return out

    t0 = time.perf_counter()
    q = {}
    for name, M, sample, oid in (("X", X, True, 2), ("W", W, False, 1), ("D", D, True, 3)):
        tag = philox.make_tag(0, oid, 0)
        u, s, v, _ = timed("decompose_" + name, lambda: rsvd.decompose(M, cfg, sample, tag, 0))
        q[name] = timed("quantize_" + name,
                        lambda: split_gemm.quantize_operand(M, u.astype(np.float32), s.astype(np.float32),
                                                            v.astype(np.float32), "sr", 0, tag, 0))
    timed("gemm_fwd", lambda: split_gemm.gemm_fwd(q["X"], q["W"]))
    timed("gemm_bwd", lambda: split_gemm.gemm_bwd(q["D"], q["W"], q["X"]))
    dt = time.perf_counter() - t0
    l, h, n = tokens, X.shape[1], ncols
    flops = 0
    for r, c, lk in ((l, h, L_K), (h, n, h), (l, n, L_K)):
        flops += decompose_flops(r, c, K_RANK, OVERSAMPLE, lk, True) + residual_flops(r, c, K_RANK)
    flops += split_gemm_flops(l, n, h, K_RANK, K_RANK) + split_gemm_flops(l, h, n, K_RANK, K_RANK)
    flops += split_gemm_flops(h, n, l, K_RANK, K_RANK)
    threads, blas = None, None
    try:
        from threadpoolctl import threadpool_info
        pools = threadpool_info()
        threads = max((i.get("num_threads", 0) for i in pools), default=None)
        libs = [i for i in pools if i.get("user_api") == "blas"]
        if libs:
            b = libs[0]
            blas = "%s %s (%s kernels, %s threads)" % (b.get("internal_api"), b.get("version"),
                                                       b.get("architecture"), b.get("num_threads"))
    except Exception:  # pragma: no cover
        pass
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads or os.cpu_count(),
            "kind": "oracle", "seconds": round(dt, 2), "stage_seconds": stages, "cpu_model": host_cpu_model(),
            "host_logical_cpus": os.cpu_count(), "blas": blas,
            "c0_single_thread_seconds": oracle_c0_single_thread(),
            "sample": "gate projection, first %d tokens x first %d output columns, refresh step "
                      "(decompose + quantise + fwd + bwd), float64 numpy oracle" % (tokens, ncols)}


def _top_right_subspace(m, k):
    """Orthonormal basis (cols x k) of the top-k right singular subspace of m,
    from the eigenvectors of the smaller Gram matrix in float64."""
    import torch
    md = m.double()
    if md.shape[0] >= md.shape[1]:
        _, vec = torch.linalg.eigh(md.T @ md)
        return vec[:, -k:]
    lam, vec = torch.linalg.eigh(md @ md.T)
    v = md.T @ vec[:, -k:]
    return torch.linalg.qr(v)[0]


def _captured(m, basis, best):
    """Share of m's best rank-k energy that the right subspace span(basis)
    captures: ||m Q||_F^2 / ||m Q_best||_F^2 (1 for the top-k subspace)."""
    import torch
    md = m.double()
    q = torch.linalg.qr(basis.double())[0]
    return float((md @ q).pow(2).sum() / (md @ best).pow(2).sum())


# companion: run each operand's rediagonalisation on a second stream beside
# its residual sweeps.  weight_stream: prepare the weight on a stream of its
# own beside X's preparation.  Measured (ms per step): q_proj 3.61 -> 3.47
# with the companion, 3.28 / 3.51 against 3.47 / 3.48 with the weight stream
# as well (no clear gain, not used); GPT-2 0.92 -> 0.95 with the companion
# (its rank-12 Jacobi is short: the fork and join cost more than they hide),
# 0.92 -> 0.85 with the weight stream.
LAYER_CONFIGS = {
    # GPT-2 130M MLP up-projection: X 8192 x 768, W 768 x 3072, k = 12
    "c1_gpt2_130m_mlp_up": dict(tokens=8192, n_in=768, n_out=3072, k=12, s=8, l_k=82, companion=False,
                                weight_stream=True),
    # LLaMA-3 8B q_proj: X 16384 x 4096, W 4096 x 4096, k = 61
    "c2_llama3_8b_q_proj": dict(tokens=16384, n_in=4096, n_out=4096, k=61, s=8, l_k=164, companion=True,
                                weight_stream=False),
}


def measure_layer(dev, name, steps=16, warmup=8, companion=None, weight_stream=None):
    """One split projection on its own (calls in data order on one stream;
    with ``companion`` each operand's rediagonalisation runs on a second
    stream beside its residual sweeps, as metis_prepare_operand allows, and
    with ``weight_stream`` the weight is prepared on a stream of its own):
    decompose + quantise X, W and D (both K orientations), the split GEMM
    forward and backward (dX, dW), the factors refreshed every 8 steps.
    Every step has its own inputs: W drifts, X and D turn their dominant
    subspace 0.01 rad per step.  Reports ms per step, algorithmic TFLOP/s,
    the main GEMM's share, and the decomposition times of X, W and D at a
    refresh step and at a cached step."""
    import torch
    from spectral_split_quantized_amd import metis, synth
    c = LAYER_CONFIGS[name]
    if companion is None:
        companion = c["companion"]
    if weight_stream is None:
        weight_stream = c.get("weight_stream", False)
    l, m, n, k = c["tokens"], c["n_in"], c["n_out"], c["k"]
    cfg = metis.make_config(k=k, s=c["s"], l_k=c["l_k"], refresh=REFRESH, rounding=metis.SR, seed=0)
    shapes = {"X": (l, m, synth.FRAC_X, True, metis.OPERAND_X), "W": (m, n, synth.FRAC_W, False, metis.OPERAND_W),
              "D": (l, n, synth.FRAC_D, True, metis.OPERAND_D)}
    nst = warmup + steps
    seqs = {}
    for op, (r, cc, frac, _, _) in shapes.items():
        seed = 5000 + 10 * synth.OPERAND_ID[op]
        if op == "W":
            master, _ = synth.anisotropic_fast(r, cc, frac, seed, out_dtype=torch.float32, device=dev)
            seq = []
            for t in range(nst):
                seq.append(master.to(torch.bfloat16))
                master = synth.drift_weight(master, seed + 7919 * (t + 1))
        else:
            seq, basis = [], None
            for t in range(nst):
                mt, basis = synth.anisotropic_fast(r, cc, frac, seed + t, device=dev, basis=basis, theta=0.01 * t)
                seq.append(mt)
        seqs[op] = seq
    f = {op: metis.Factors(r, cc, k, dev) for op, (r, cc, _, _, _) in shapes.items()}
    q = {op: metis.QOperand(r, cc, k, metis.AXIS0 | metis.AXIS1, dev) for op, (r, cc, _, _, _) in shapes.items()}
    lib = metis.load()
    import ctypes
    need = max(lib.metis_prepare_operand_workspace(r, cc, ctypes.byref(cfg), int(smp))
               for r, cc, _, smp, _ in shapes.values())
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    side = torch.cuda.Stream(device=dev) if companion else None  # default priority
    wst = torch.cuda.Stream(device=dev) if weight_stream else None
    main = torch.cuda.current_stream(dev)
    w_free = None
    Y = torch.empty(l, n, dtype=torch.float32, device=dev)
    dX = torch.empty(l, m, dtype=torch.float32, device=dev)
    dW = torch.empty(m, n, dtype=torch.float32, device=dev)
    xc, wc, dc = q["X"]._c(), q["W"]._c(), q["D"]._c()
    gwf = torch.empty(lib.metis_gemm_fwd_workspace(ctypes.byref(xc), ctypes.byref(wc)), dtype=torch.uint8, device=dev)
    gwb = torch.empty(lib.metis_gemm_bwd_workspace(ctypes.byref(dc), ctypes.byref(wc), ctypes.byref(xc)),
                      dtype=torch.uint8, device=dev)

    wws = torch.empty(need, dtype=torch.uint8, device=dev) if weight_stream else None

    def step(t):
        nonlocal w_free
        w_ready = None
        if wst is not None:
            # the weight is prepared on its own stream, beside X's preparation
            # (after the previous step's last GEMM reading its codes)
            if w_free is not None:
                wst.wait_event(w_free)
            with torch.cuda.stream(wst):
                metis.prepare_operand(seqs["W"][t], cfg, False, metis.make_tag(9, metis.OPERAND_W), t, f["W"],
                                      metis.AXIS0 | metis.AXIS1, out=q["W"], workspace=wws)
                w_ready = torch.cuda.Event()
                w_ready.record(wst)
        for op, (_, _, _, smp, kind) in shapes.items():
            if op == "W" and wst is not None:
                main.wait_event(w_ready)
            else:
                metis.prepare_operand(seqs[op][t], cfg, smp, metis.make_tag(9, kind), t, f[op],
                                      metis.AXIS0 | metis.AXIS1, out=q[op], workspace=ws, side_stream=side)
            if op == "W":
                metis.gemm_fwd(q["X"], q["W"], Y=Y, workspace=gwf)
        metis.gemm_bwd(q["D"], q["W"], q["X"], dX=dX, dW=dW, workspace=gwb)
        if wst is not None:
            w_free = torch.cuda.Event()
            w_free.record(main)

    for t in range(warmup):
        step(t)
    torch.cuda.synchronize()
    metis.status_sync()
    metis.timing_enable(1024)
    metis.timing_kinds(1)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for t in range(warmup, nst):
        step(t)
    b.record()
    torch.cuda.synchronize()
    total = a.elapsed_time(b)
    recs = metis.timing_read(1024)
    metis.timing_enable(0)
    metis.timing_kinds(-1)
    metis.status_sync()
    flops = 0
    for t in range(warmup, nst):
        refresh = (t % REFRESH) == 0
        for op, (r, cc, _, smp, _) in shapes.items():
            flops += decompose_flops(r, cc, k, c["s"], c["l_k"] if smp else r, refresh) + residual_flops(r, cc, k)
        flops += split_gemm_flops(l, n, m, k, k) + split_gemm_flops(l, m, n, k, k) + split_gemm_flops(m, n, l, k, k)
    g = [r for r in recs if r[0] == 0]
    g_ms = sum(r[1] for r in g) / steps
    g_flops = sum(2 * r[2] * r[3] * r[4] + 2 * r[2] * r[3] * 2 * k for r in g) / steps
    g_tf = g_flops / (g_ms * 1e-3) / 1e12 if g_ms > 0 else 0.0
    # decomposition alone, at a refresh step and at the cached step after it
    rsvd = {}
    for op, (r, cc, _, smp, kind) in shapes.items():
        fo = metis.Factors(r, cc, k, dev)
        t0 = (nst // REFRESH) * REFRESH
        for label, t in (("refresh", t0), ("cached", t0 + 1)):
            total, sketch, proj = decompose_timed(seqs[op][t % nst], cfg, smp, metis.make_tag(9, kind), t, fo,
                                                  workspace=ws)
            rsvd["%s_%s" % (op, label)] = total
            if label == "refresh":
                rsvd["%s_refresh_sketch" % op] = sketch
                rsvd["%s_refresh_project_rediag" % op] = proj
    metis.status_sync()
    del seqs
    torch.cuda.empty_cache()
    return {"workload": name, "shapes": {"X": [l, m], "W": [m, n], "D": [l, n]}, "k": k, "s": c["s"],
            "l_k": c["l_k"], "refresh": REFRESH, "rounding": "sr", "steps": steps, "warmup": warmup,
            "ms_per_step": round(total / steps, 4), "tflops": round(flops / (total * 1e-3) / 1e12, 2),
            "main_gemm": {"ms_per_step": round(g_ms, 4), "launches_per_step": len(g) / steps,
                          "roofline": {"bound": "mfma", "achieved": round(g_tf, 1), "peak": PEAK_F16_TFLOPS,
                                       "unit": "TFLOP/s", "frac": round(g_tf / PEAK_F16_TFLOPS, 4)}},
            "rsvd_ms": rsvd, "streams": 1 + int(bool(companion)) + int(bool(weight_stream))}


def measure_training_loop(dev, steps=48, periods=(1, 8, 32), tokens=8192, lr=2e-5):
    """A GPT-2-130M-shaped MLP block (768 -> 3072 -> GELU -> 768, no bias),
    both linears through the Metis autograd layer, trained with Adam on a
    synthetic teacher-student regression, once per factor refresh period.
    Each step draws new inputs whose dominant right subspace turns by 0.01 rad
    per step.  Reports the relative loss, how well each cached right factor
    still spans its operand's current top-k right singular subspace
    (staleness), how much that subspace moves between adjacent steps, and the
    time per training step.  A float32 run of the same model and data is the
    reference loss."""
    import torch
    import torch.nn.functional as Fn
    from spectral_split_quantized_amd import synth
    from spectral_split_quantized_amd.layer import MetisLinear, set_step
    H, F_, k = 768, 3072, 12

    def weight(r, c, seed):
        w, _ = synth.anisotropic_fast(r, c, synth.FRAC_W, seed, out_dtype=torch.float32, device=dev)
        return w / torch.linalg.matrix_norm(w, ord=2)

    t1, t2 = weight(H, F_, 901), weight(F_, H, 902)
    s1, s2 = weight(H, F_, 903), weight(F_, H, 904)
    _, basis = synth.anisotropic_fast(tokens, H, synth.FRAC_X, 905, device=dev)

    def batch(t):
        x, _ = synth.anisotropic_fast(tokens, H, synth.FRAC_X, 1000 + t, device=dev, basis=basis, theta=0.01 * t)
        with torch.no_grad():
            y = Fn.gelu(x.float() @ t1) @ t2
        return x, y

    def run(period):
        if period is None:
            w1 = torch.nn.Parameter(s1.clone())
            w2 = torch.nn.Parameter(s2.clone())
            params = [w1, w2]
            fwd = lambda x: Fn.gelu(x.float() @ w1) @ w2
        else:
            l1 = MetisLinear(H, F_, k, l_k=82, refresh=period, weight=s1.clone(), layer=0, device=dev)
            l2 = MetisLinear(F_, H, k, l_k=82, refresh=period, weight=s2.clone(), layer=1, device=dev)
            params = [l1.weight, l2.weight]
            fwd = lambda x: l2(Fn.gelu(l1(x.float())))
        opt = torch.optim.Adam(params, lr=lr)
        rec = {"loss": [], "ms": [], "align_w": [], "align_x": [], "drift_w": [], "drift_x": []}
        prev = None
        for t in range(steps):
            x, y = batch(t)
            # the operands' current top-k right subspaces (the weight before this step's update)
            w_now = params[0].detach().clone()
            cur = (_top_right_subspace(w_now, k), _top_right_subspace(x, k))
            if prev is not None:
                rec["drift_w"].append(_captured(w_now, prev[0], cur[0]))
                rec["drift_x"].append(_captured(x, prev[1], cur[1]))
            prev = cur
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            if period is not None:
                set_step(l1, t)
                set_step(l2, t)
            out = fwd(x)
            loss = (out - y).pow(2).mean() / y.pow(2).mean()
            opt.zero_grad(set_to_none=True)
            loss.backward()
            opt.step()
            torch.cuda.synchronize()
            rec["ms"].append(1e3 * (time.perf_counter() - t0))
            rec["loss"].append(float(loss.detach()))
            if period is not None:
                # the right factors this step used: sketched at its last refresh, rotated since
                rec["align_w"].append(_captured(w_now, l1.factors["W"].V, cur[0]))
                rec["align_x"].append(_captured(x, l1.factors["X"].V, cur[1]))
            del out, loss
        return rec

    def mean(v):
        return round(sum(v) / len(v), 5) if v else None

    out = {"model": "GPT-2-130M MLP block 768 -> 3072 -> GELU -> 768, no bias; teacher-student regression",
           "tokens": tokens, "steps": steps, "k": k, "l_k": 82, "optimizer": "Adam lr %g" % lr,
           "input_drift": "dominant right subspace of X turned 0.01 rad per step",
           "loss": "||Y - Y*||^2 / ||Y*||^2 of the step's batch"}
    ref = run(None)
    out["float32"] = {"loss_first": round(ref["loss"][0], 5), "loss_last8": mean(ref["loss"][-8:]),
                      "ms_per_step": mean(ref["ms"][2:])}
    out["previous_step_subspace_energy"] = {"W1": mean(ref["drift_w"]), "X": mean(ref["drift_x"]),
                                      "W1_min": round(min(ref["drift_w"]), 5), "X_min": round(min(ref["drift_x"]), 5)}
    for period in periods:
        r = run(period)
        out["refresh_%d" % period] = {
            "loss_first": round(r["loss"][0], 5), "loss_last8": mean(r["loss"][-8:]),
            "ms_per_step": mean(r["ms"][2:]),
            "cached_factor_energy": {"W1": mean(r["align_w"]), "X": mean(r["align_x"]),
                                        "W1_min": round(min(r["align_w"]), 5), "X_min": round(min(r["align_x"]), 5)}}
    out["energy_note"] = ("share of the operand's best rank-k energy ||M Q||^2 / ||M V_k||^2 that a k-dim right subspace "
                          "captures (1 = as good as the exact top-k): cached_factor_energy for the factor each step used, "
                          "previous_step_subspace_energy for the previous step's exact top-k subspace (the float32 run)")
    return out


# -------------------------------------------------------------------- main --

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=16)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=2048)
    ap.add_argument("--cpu-cols", type=int, default=4096)
    ap.add_argument("--streams", type=int, default=3,
                    help="HIP streams per step (1: every call in order on one stream)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the ceilings, the plain-NVFP4 comparison and the 1M x 4096 activation")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy three times (PMC byte-counter scale)")
    ap.add_argument("--mxfp4-only", action="store_true",
                    help="only the MXFP4 variant at the gate projection's shape (for kernel profiles)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return 0
    if args.mxfp4_only:
        return mxfp4_only()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from spectral_split_quantized_amd import metis

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    metis.load()

    # one input set per step, so the weight drift and the activation rotation
    # continue over the whole run (cycled only past MAX_INPUT_STEPS)
    n_in = min(args.warmup + args.steps, MAX_INPUT_STEPS)
    log("building inputs (%d steps, LLaMA-3-8B MLP shapes)" % n_in)
    t_build = time.time()
    inputs = build_inputs(n_in, dev)
    log("inputs built in %.1f s" % (time.time() - t_build))
    mlp = MetisMLP(dev, streams=args.streams)

    # warmup (untimed), then the timed steps; step index continues so the
    # refresh schedule (every 8 steps) is the same in both
    for t in range(args.warmup):
        mlp.step(t, inputs)
        if t == 0:
            metis.status_sync()
    torch.cuda.synchronize()
    metis.status_sync()
    log("warmup done (%d steps)" % args.warmup)

    # events around the main split GEMMs only: each record adds two packets to
    # its stream, so the quantiser sweeps are timed on their own further down
    metis.timing_enable(4096)
    metis.timing_kinds(1)
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for t in range(args.warmup, args.warmup + args.steps):
        mlp.step(t, inputs)
    if mlp.free_down is not None:
        stream.wait_event(mlp.free_down)  # the last step's side-stream GEMM
    ev1.record(stream)
    torch.cuda.synchronize()
    total_ms = ev0.elapsed_time(ev1)
    recs = metis.timing_read(4096)
    metis.timing_enable(0)
    metis.timing_kinds(-1)
    metis.status_sync()
    ms_per_step = total_ms / args.steps
    flops = sum(mlp.step_flops(t) for t in range(args.warmup, args.warmup + args.steps))
    value = flops / (total_ms * 1e-3) / 1e12
    log("timed %d steps: %.2f ms/step, %.1f TFLOP/s" % (args.steps, ms_per_step, value))

    # roofline of the dominant kernel: the main split-GEMM kernel (kind 0)
    g = [r for r in recs if r[0] == 0]
    g_ms = sum(r[1] for r in g)
    g_flops = sum(2 * r[2] * r[3] * r[4] + 2 * r[2] * r[3] * 2 * K_RANK for r in g)
    g_tflops = g_flops / (g_ms * 1e-3) / 1e12 if g_ms > 0 else 0.0
    traffic = GEMM_TRAFFIC_BYTES if GEMM_TRAFFIC_SHA is not None and gemm_source_sha() == GEMM_TRAFFIC_SHA else None
    roofline = {"bound": "mfma", "achieved": round(g_tflops, 1), "peak": PEAK_F16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(g_tflops / PEAK_F16_TFLOPS, 4), "traffic": traffic,
                "kernel": "gemm_fp4_reg_kernel (main split GEMM)", "launches": len(g),
                "avg_ms": round(g_ms / max(len(g), 1), 4)}
    # per output shape: median, p10 and p90 of the launch times
    by_shape = {}
    for r in g:
        by_shape.setdefault("%dx%dx%d" % (r[2], r[3], r[4]), []).append(r[1])
    roofline["launch_ms_p10_p50_p90"] = {
        k: [round(float(q), 4) for q in np.percentile(v, [10, 50, 90])] for k, v in sorted(by_shape.items())}
    # streaming: both quantiser sweeps (amax + quantise-on-store) of the
    # largest operand, X_down's residual in both orientations with SR, timed
    # alone after the timed steps (median of 5 calls)
    t_last = args.warmup + args.steps - 1
    xd = mlp.ops["X_down"]
    M = inputs["X_down"][t_last % len(inputs["X_down"])]
    metis.timing_enable(64)
    metis.timing_kinds(6)
    for _ in range(6):
        metis.quantize(M, mlp.cfg, xd.tag, t_last, metis.AXIS0 | metis.AXIS1, factors=mlp.factors["X_down"],
                       out=mlp.q["X_down"], workspace=mlp.ws[0])
    qrecs = metis.timing_read(64)
    metis.timing_enable(0)
    metis.timing_kinds(-1)
    # the residual sweeps only (the factor sweeps are recorded too)
    q1 = [r[1] for r in qrecs if r[0] == 1 and r[2] == xd.rows and r[3] == xd.cols][1:]
    q2 = [r[1] for r in qrecs if r[0] == 2 and r[2] == xd.rows and r[3] == xd.cols][1:]
    q_ms = sorted(a + b for a, b in zip(q1, q2))[len(q2) // 2]
    # M read by both sweeps (bf16), codes and scales of two orientations, and
    # the rank-k reconstruction operands
    q_bytes = xd.rows * xd.cols * (2 * 2 + 2 * (0.5 + 1 / 16)) + 2 * (xd.rows + xd.cols) * K_RANK * 4
    q_gbs = q_bytes / (q_ms * 1e-3) / 1e9 if q_ms > 0 else 0.0
    streaming = {"bound": "hbm", "achieved": round(q_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                 "frac": round(q_gbs / PEAK_HBM_GBS, 4),
                 "traffic": QUANT_TRAFFIC_BYTES if source_sha(QUANT_SOURCES) == QUANT_TRAFFIC_SHA else None,
                 "kernel": "qf_amax_kernel + qf_quant_kernel (both quantiser sweeps)",
                 "operand": "X_down residual %d x %d, both orientations, SR" % (xd.rows, xd.cols),
                 "ms": round(q_ms, 4)}

    # rSVD timing at a refresh step and at the cached step after it, on that
    # step's own (drifted) input (outside the timed region); the refresh is
    # also split into the sketch (row sample to V) and the projection with
    # its rediagonalisation, from the library's own event pairs
    rsvd_ms = {}
    for name in ("W_gate", "X_gu", "D_gate"):
        op = mlp.ops[name]
        f = metis.Factors(op.rows, op.cols, K_RANK, dev)
        for label, t in (("refresh", 64), ("cached", 65)):
            M = inputs[name][(t - 64) % len(inputs[name])]
            total, sketch, proj = decompose_timed(M, mlp.cfg, op.sample, op.tag, t, f, workspace=mlp.ws[0])
            rsvd_ms["%s_%s" % (name, label)] = total
            if label == "refresh":
                rsvd_ms["%s_refresh_sketch" % name] = sketch
                rsvd_ms["%s_refresh_project_rediag" % name] = proj
    metis.status_sync()

    extras = {}
    if not args.no_extras:
        log("measuring the copy and vendor-GEMM ceilings")
        extras["ceilings"] = measure_ceilings(dev)
        log("plain NVFP4 (k = 0) on the same workload")
        extras["direct_nvfp4"] = measure_direct(mlp, inputs, args.warmup + args.steps - 1, ms_per_step)
        log("MXFP4 variant on the scaled FP4 matrix instruction")
        t_last = args.warmup + args.steps - 1
        extras["mxfp4_variant"] = measure_mxfp4(mlp.metis, inputs["X_gu"][t_last % len(inputs["X_gu"])],
                                                inputs["W_gate"][t_last % len(inputs["W_gate"])], t_last,
                                                roofline["avg_ms"])
        for name in LAYER_CONFIGS:
            log("single projection %s" % name)
            extras.setdefault("layers", {})[name] = measure_layer(dev, name)
        log("1M x 4096 activation")
        extras["c4_activation"] = measure_c4(dev, extras["ceilings"]["copy_GBps"])
        log("training loop through the autograd layer (refresh periods 1, 8, 32)")
        extras["training_loop"] = measure_training_loop(dev)
        ceil_tf = extras["ceilings"]["hipblaslt_bf16_TFLOPs"]
        roofline["frac_vs_hipblaslt_bf16"] = round(g_tflops / ceil_tf, 4) if ceil_tf else None
        streaming["frac_vs_copy"] = round(streaming["achieved"] / extras["ceilings"]["copy_GBps"], 4)

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        sample = {"X": inputs["X_gu"][0][:args.cpu_tokens].float().cpu().numpy(),
                  "W": inputs["W_gate"][0][:, :args.cpu_cols].float().cpu().numpy(),
                  "D": inputs["D_gate"][0][:args.cpu_tokens, :args.cpu_cols].float().cpu().numpy()}
        cpu = cpu_baseline(sample, args.cpu_tokens, args.cpu_cols)
        log("cpu oracle: %.3g TFLOP/s in %.1f s" % (cpu["value"], cpu["seconds"]))

    out = {"metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 3),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "nvfp4 operands, f16 mfma, f32 accumulate",
           "data": "synthetic",
           "config": {"workload": "llama3_8b_mlp_gate_up_down_16k_tokens_8step_factor_cache",
                      "streams": mlp.nstreams + (1 if mlp.side is not None else 0),
                      "tokens": TOKENS, "hidden": HIDDEN, "ffn": FFN, "k": K_RANK, "s": OVERSAMPLE,
                      "l_k": L_K, "refresh": REFRESH, "rounding": "sr", "input_steps": n_in},
           "dense_equiv_tflops": round(dense_equiv_flops() * args.steps / (total_ms * 1e-3) / 1e12, 2),
           "algorithmic_flop_per_step": round(flops / args.steps),
           "roofline": roofline, "streaming_roofline": streaming, "rsvd_ms": rsvd_ms,
           "cpu_baseline": cpu}
    out.update(extras)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
