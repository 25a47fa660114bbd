"""Python front of the CPU oracle for the Prox two-stage sparse SwiGLU FFN step.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may call this module; the product path (the HIP library and
its Python binding) never imports it, and it never imports them.

The arithmetic lives in ``prox_oracle.c`` (plain C, double accumulation); this
file only marshals numpy arrays and strings the paper's steps together in the
paper's order.  Paper: "Prox: Training-Free FFN Activation Sparsity via
Approximate Intermediate-Channel Salience in LLMs" (arXiv 2607.27591).

Parity status per function (what pins it, see tests/test_oracle_pins.py):
  quantize      round-trip bound, +-7 at the absmax, zero groups
  input_mask    brute force; Gaussian energy closed form of App. A.2
  proxy         full-precision mode reduces to the exact state (oracle-s,
                Sec. 3.1); Gaussian correlation/error closed forms (App. A.2);
                brute force on tiny shapes.  The INT4 proxy values themselves
                have no printed example: beyond the bit-fixed quantizer they
                are "parity unpinned".
  topk          brute-force rank definition; Laplace energy closed form
                (App. A.2); popcount; ties to the lower index
  threshold_mask  equals top-k when tau_s is the k-th largest value (no ties);
                monotone in tau_s; Laplace energy closed form (App. A.2)
  stage2/dense  zero sparsity equals the dense FFN; brute force on tiny shapes
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "prox_oracle.c")
_LIB = os.path.join(_HERE, "libprox_oracle.so")

_lib = None


def build(force: bool = False, cc: str = "gcc", extra_flags=()) -> str:
    """Compile prox_oracle.c (IEEE arithmetic: no fast-math, no contraction).
    cc / extra_flags let the CPU sanitizer run build it with clang and
    -fsanitize=address,undefined."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            [cc, "-O2", "-fno-fast-math", "-ffp-contract=off", "-std=c11", *extra_flags,
             "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.prox_oracle_quantize.argtypes = [P, I, I, I, P, P]
        lib.prox_oracle_quantize.restype = I
        lib.prox_oracle_dequantize.argtypes = [P, P, I, I, I, P]
        lib.prox_oracle_input_mask.argtypes = [P, I, ctypes.c_float, P]
        lib.prox_oracle_input_mask.restype = I
        lib.prox_oracle_proxy.argtypes = [P, P, I, P, P, I, P, P, P, I]
        lib.prox_oracle_topk.argtypes = [P, I, I, P]
        lib.prox_oracle_topk.restype = I
        lib.prox_oracle_threshold_mask.argtypes = [P, I, ctypes.c_float, P]
        lib.prox_oracle_threshold_mask.restype = I
        lib.prox_oracle_stage2.argtypes = [P, I, I, P, P, P, P, I, P, P, I]
        lib.prox_oracle_dense.argtypes = [P, I, I, P, P, P, P, P, I]
        lib.prox_oracle_gate_act.argtypes = [ctypes.c_double, I]
        lib.prox_oracle_gate_act.restype = ctypes.c_double
        lib.prox_oracle_round_bf16.argtypes = [ctypes.c_float]
        lib.prox_oracle_round_bf16.restype = ctypes.c_float
        lib.prox_oracle_round_bf16_array.argtypes = [P, ctypes.c_long]
        lib.prox_oracle_rmsnorm.argtypes = [P, I, ctypes.c_double, I, P]
        _lib = lib
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


# --------------------------------------------------------------------------
# Individual steps, in the paper's order.
# --------------------------------------------------------------------------
def quantize(W, G: int):
    """Symmetric INT4 proxy of one [d_model][d_ff] matrix (Sec. 4.3).

    Returns (q int8 [d_model][d_ff] in [-7, 7], scale float32 [d_model/G][d_ff]).
    """
    W = _f32(W)
    d_model, d_ff = W.shape
    q = np.zeros((d_model, d_ff), dtype=np.int8)
    sc = np.zeros((d_model // G, d_ff), dtype=np.float32)
    rc = _load().prox_oracle_quantize(_p(W), d_model, d_ff, G, _p(q), _p(sc))
    if rc != 0:
        raise ValueError("d_model must be a multiple of the group size")
    return q, sc


def dequantize(q, scale, G: int) -> np.ndarray:
    """Proxy weights W~ = q * scale in double, [d_model][d_ff]."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    scale = _f32(scale)
    d_model, d_ff = q.shape
    out = np.empty((d_model, d_ff), dtype=np.float64)
    _load().prox_oracle_dequantize(_p(q), _p(scale), d_model, d_ff, G, _p(out))
    return out


def input_mask(x, tau: float) -> np.ndarray:
    """Ascending survivors {i : |x_i| >= tau} (Sec. 4.1, m_x equation)."""
    x = _f32(x)
    idx = np.zeros(max(1, x.size), dtype=np.int32)
    n1 = _load().prox_oracle_input_mask(_p(x), x.size, float(np.float32(tau)), _p(idx))
    return idx[:n1].copy()


def gate_act(z: float, act: int = 0) -> float:
    """Gate activation: 0 = SiLU (SwiGLU), 1 = GELU, tanh form (GeGLU)."""
    return float(_load().prox_oracle_gate_act(float(z), int(act)))


def proxy(x, idx, Wt_up, Wt_gate, act: int = 0):
    """Stage 1 proxy state u~, g~ (pre-activation), s~ (Sec. 4.1, u~/h~
    equations; act 1 swaps SiLU for the tanh form of GELU).

    Wt_up / Wt_gate are [d_model][d_ff] proxy weights (dequantized INT4, or the
    original weights for the full-precision proxy)."""
    x = _f32(x)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    Wt_up = np.ascontiguousarray(Wt_up, dtype=np.float64)
    Wt_gate = np.ascontiguousarray(Wt_gate, dtype=np.float64)
    d_ff = Wt_up.shape[1]
    u = np.empty(d_ff)
    g = np.empty(d_ff)
    s = np.empty(d_ff)
    _load().prox_oracle_proxy(_p(x), _p(idx), idx.size, _p(Wt_up), _p(Wt_gate),
                              d_ff, _p(u), _p(g), _p(s), int(act))
    return u, g, s


def topk(z, k: int) -> np.ndarray:
    """k indices of largest |z|, ties to the lower index, ascending (App. A.6)."""
    z = np.ascontiguousarray(z, dtype=np.float64)
    sel = np.zeros(max(1, k), dtype=np.int32)
    rc = _load().prox_oracle_topk(_p(z), z.size, int(k), _p(sel))
    if rc != 0:
        raise ValueError("k out of range")
    return sel[:k].copy()


def threshold_mask(z, tau_s: float) -> np.ndarray:
    """Ascending channels with |z_j| >= tau_s, compared in float32 (Sec. 4.1,
    m_s equation with the calibrated threshold tau_s)."""
    z = np.ascontiguousarray(z, dtype=np.float64)
    sel = np.zeros(max(1, z.size), dtype=np.int32)
    m = _load().prox_oracle_threshold_mask(_p(z), z.size, float(np.float32(tau_s)), _p(sel))
    return sel[:m].copy()


def stage2(x, W_up, W_gate, W_down, sel, act: int = 0):
    """Exact Stage 2 over the selected channels (Sec. 4.1, Stage 2 equations).

    Returns (s_sp [k] double, y [d_model] double)."""
    x = _f32(x)
    W_up, W_gate, W_down = _f32(W_up), _f32(W_gate), _f32(W_down)
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    d_model, d_ff = W_up.shape
    k = sel.size
    s_sp = np.zeros(max(1, k))
    y = np.zeros(d_model)
    _load().prox_oracle_stage2(_p(x), d_model, d_ff, _p(W_up), _p(W_gate),
                               _p(W_down), _p(sel), k, _p(s_sp), _p(y), int(act))
    return s_sp[:k].copy(), y


def dense(x, W_up, W_gate, W_down, act: int = 0):
    """Dense gated FFN (Sec. 2.1; act 0 SwiGLU, 1 GeGLU).  Returns (s [d_ff]
    double, y [d_model] double)."""
    x = _f32(x)
    W_up, W_gate, W_down = _f32(W_up), _f32(W_gate), _f32(W_down)
    d_model, d_ff = W_up.shape
    s = np.empty(d_ff)
    y = np.empty(d_model)
    _load().prox_oracle_dense(_p(x), d_model, d_ff, _p(W_up), _p(W_gate),
                              _p(W_down), _p(s), _p(y), int(act))
    return s, y


def round_bf16(v) -> np.ndarray:
    """Round float32 values to bfloat16 (ties to even), widened back to float32."""
    out = np.array(v, dtype=np.float32, copy=True, order="C")
    _load().prox_oracle_round_bf16_array(_p(out), out.size)
    return out


def rmsnorm(r, eps: float = 1e-5, to_bf16: bool = True) -> np.ndarray:
    """x = cast(r / sqrt(mean(r^2) + eps)), unit gain (stack glue)."""
    r = np.ascontiguousarray(r, dtype=np.float64)
    x = np.empty(r.size, dtype=np.float32)
    _load().prox_oracle_rmsnorm(_p(r), r.size, float(eps), 1 if to_bf16 else 0, _p(x))
    return x


# --------------------------------------------------------------------------
# The whole step.
# --------------------------------------------------------------------------
class Layer:
    """One FFN layer as the oracle sees it: original weights (paper layout,
    float32 values) plus its own INT4 proxy, computed here."""

    def __init__(self, W_up, W_gate, W_down, G: int, full_precision_proxy=False, act: int = 0):
        self.act = int(act)
        self.W_up = _f32(W_up)
        self.W_gate = _f32(W_gate)
        self.W_down = _f32(W_down)
        self.G = int(G)
        self.d_model, self.d_ff = self.W_up.shape
        if full_precision_proxy:
            self.q_up = self.sc_up = self.q_gate = self.sc_gate = None
            self.Wt_up = self.W_up.astype(np.float64)
            self.Wt_gate = self.W_gate.astype(np.float64)
        else:
            self.q_up, self.sc_up = quantize(self.W_up, G)
            self.q_gate, self.sc_gate = quantize(self.W_gate, G)
            self.Wt_up = dequantize(self.q_up, self.sc_up, G)
            self.Wt_gate = dequantize(self.q_gate, self.sc_gate, G)


def forward(layer: Layer, x, tau: float, k: int) -> dict:
    """Prox FFN step for one token: Stage 1 (mask, proxy, top-k) then Stage 2.

    Returns a dict with idx (survivors), u_t/g_t/s_t (proxy), sel, s_sp, y."""
    x = _f32(x)
    idx = input_mask(x, tau)
    u_t, g_t, s_t = proxy(x, idx, layer.Wt_up, layer.Wt_gate, layer.act)
    sel = topk(s_t, k)
    s_sp, y = stage2(x, layer.W_up, layer.W_gate, layer.W_down, sel, layer.act)
    return dict(idx=idx, u_t=u_t, g_t=g_t, s_t=s_t, sel=sel, s_sp=s_sp, y=y)


def forward_ts(layer: Layer, x, tau_x: float, tau_s: float) -> dict:
    """Prox FFN step with the calibrated Stage 2 threshold instead of top-k:
    Stage 1 (input mask, proxy), the mask |s~| >= tau_s, then Stage 2 (Sec. 4.1).
    Same dict as forward(); the number of kept channels is sel.size."""
    x = _f32(x)
    idx = input_mask(x, tau_x)
    u_t, g_t, s_t = proxy(x, idx, layer.Wt_up, layer.Wt_gate, layer.act)
    sel = threshold_mask(s_t, tau_s)
    s_sp, y = stage2(x, layer.W_up, layer.W_gate, layer.W_down, sel, layer.act)
    return dict(idx=idx, u_t=u_t, g_t=g_t, s_t=s_t, sel=sel, s_sp=s_sp, y=y)


def forward_batch(layer: Layer, X, tau: float, k: int) -> list:
    """Batch of independent tokens: each token gets its own masks and its own
    exact result (the union of the masks only decides what a kernel streams)."""
    return [forward(layer, X[b], tau, k) for b in range(np.asarray(X).shape[0])]


def stack_forward(layers, taus, k: int, r0, eps: float = 1e-5, to_bf16=True):
    """Pre-norm residual FFN stack: x_l = cast(RMSNorm(r_l)), y_l = FFN_l(x_l)
    cast to the layer dtype, r_{l+1} = r_l + y_l.  Returns (r_L, per-layer dicts)."""
    r = np.asarray(r0, dtype=np.float64).copy()
    outs = []
    for layer, tau in zip(layers, taus):
        x = rmsnorm(r, eps, to_bf16)
        o = forward(layer, x, tau, k)
        yc = o["y"].astype(np.float32)
        if to_bf16:
            yc = round_bf16(yc)
        r = r + yc.astype(np.float64)
        o["x"] = x
        outs.append(o)
    return r, outs


# --------------------------------------------------------------------------
# Stack with Stage 2 threshold masks, and its sequential calibration
# (App. A.7, Algorithm 1).
# --------------------------------------------------------------------------
def lower_quantile(values, q: float) -> float:
    """Lower empirical quantile: the sorted values at position floor(q (N - 1))."""
    v = np.sort(np.asarray(values, dtype=np.float64).ravel())
    return float(v[int(math.floor(q * (v.size - 1)))])


def stack_forward_ts(layers, taus_x, taus_s, r0, eps: float = 1e-5, to_bf16=True):
    """Pre-norm residual stack with the Stage 2 threshold mask in every layer:
    x_l = cast(RMSNorm(r_l)), y_l = forward_ts(x_l), r_{l+1} = r_l + cast(y_l).
    Returns (r_L, per-layer dicts)."""
    r = np.asarray(r0, dtype=np.float64).copy()
    outs = []
    for layer, tx, ts in zip(layers, taus_x, taus_s):
        x = rmsnorm(r, eps, to_bf16)
        o = forward_ts(layer, x, tx, ts)
        yc = o["y"].astype(np.float32)
        if to_bf16:
            yc = round_bf16(yc)
        r = r + yc.astype(np.float64)
        o["x"] = x
        outs.append(o)
    return r, outs


def calibrate_sequential(layers, calib_r0, s1: float, s2: float, eps: float = 1e-5,
                         to_bf16=True):
    """Algorithm 1 of App. A.7, layer by layer in depth order: the calibration
    tokens' inputs x_l are collected after layers 1..l-1 ran with their final
    thresholds; tau_x,l is the s1 quantile of the pooled |x_l|; s~_l is the
    INT4 proxy state under that input mask; tau_s,l is the s2 quantile of the
    pooled float32 |s~_l|; then the tokens pass layer l with both thresholds.

    calib_r0: [N][d_model] residual-stream tokens.  Returns (taus_x, taus_s,
    per-layer inputs [N][d_model] float32)."""
    R = [np.asarray(r, dtype=np.float64).copy() for r in calib_r0]
    taus_x, taus_s, inputs = [], [], []
    for layer in layers:
        X = np.stack([rmsnorm(r, eps, to_bf16) for r in R])
        tx = lower_quantile(np.abs(X.astype(np.float32)), s1)
        S = []
        for x in X:
            _, _, s_t = proxy(x, input_mask(x, tx), layer.Wt_up, layer.Wt_gate, layer.act)
            S.append(np.abs(s_t).astype(np.float32))
        ts = lower_quantile(np.concatenate(S), s2)
        for t, x in enumerate(X):
            yc = forward_ts(layer, x, tx, ts)["y"].astype(np.float32)
            if to_bf16:
                yc = round_bf16(yc)
            R[t] = R[t] + yc.astype(np.float64)
        taus_x.append(tx)
        taus_s.append(ts)
        inputs.append(X)
    return taus_x, taus_s, inputs
