"""Sequential per-layer threshold calibration for an FFN stack, and the
runtime sparsity it yields.

Paper: "Prox: Training-Free FFN Activation Sparsity ...", App. A.7
(Algorithm 1, sequential threshold calibration): layers are calibrated in
depth order, and layer l's inputs are collected after the calibration tokens
went through layers 1..l-1 with their finalized sparse rules.

- sequential_thresholds: the input threshold tau_x only, for a stack whose
  Stage 2 mask is the per-token top-k.
- sequential_thresholds_ts: both thresholds, tau_x,l at the Stage 1 target
  s1 and tau_s,l at the Stage 2 target s2 (Sec. 4.1 masks), for a stack with
  Stage 2 threshold masks; (s1, s2) come from costmodel.allocate for a target
  effective sparsity e (Sec. 4.2).
- runtime_sparsity: the realized s1, s2 and e on other tokens (App. A.7,
  runtime sparsity), from the mask counts of the GPU path.

Every step runs on the GPU through libprox (normalization, Stage 1, sparse
forward, residual update); only the quantiles are taken on the host, as the
lower empirical quantile sorted[floor(q (N - 1))] of the pooled magnitudes.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import costmodel, prox, synth


def calibrate_layer(L, r, quantile: float, k: int, eps: float = 1e-5, return_input=False):
    """One step of the sequential calibration (top-k Stage 2 mask): tau_x of
    layer L is the `quantile` of the pooled |x| of the calibration tokens'
    inputs x = cast(RMSNorm(r)); then the tokens pass the layer with it
    (r += y, in place).  r: float32 [N][d_model] residual-stream tokens."""
    N = r.shape[0]
    mb = L.shape.max_batch
    x = torch.empty(r.shape, dtype=L.dtype, device=r.device)
    for c in range(0, N, mb):
        prox.prox_rmsnorm(L, r[c:c + mb], eps, x[c:c + mb])
    tau = synth.calibrate_tau(x, quantile)
    for c in range(0, N, mb):
        prox.prox_stack_forward([L], [tau], k, r[c:c + mb], eps)
    return (tau, x) if return_input else tau


def sequential_thresholds(layers, calib_resid, quantile: float, k: int, eps: float = 1e-5):
    """Thresholds tau_x for each layer of a stack.

    calib_resid: float32 [N][d_model] residual-stream calibration tokens (not
    modified).  Returns a list of floats, one per layer."""
    r = calib_resid.detach().clone().contiguous()
    return [calibrate_layer(L, r, quantile, k, eps) for L in layers]


def _abs_proxy_state(L, x_row, tau_x, s_abs, y):
    """|s~| of one token (Stage 1 only: the Stage 2 mask keeps nothing)."""
    dbg = prox.prox_debug(s_abs=ctypes.c_void_p(s_abs.data_ptr()))
    prox._check(prox.load_library().prox_ffn_forward_ts_debug(
        L.handle, prox._ptr(x_row), float(tau_x), float("inf"), prox._ptr(y),
        ctypes.byref(dbg), prox._stream()))


def calibrate_layer_ts(L, r, s1: float, s2: float, eps: float = 1e-5, return_input=False):
    """One step of Algorithm 1 (App. A.7) with both thresholds: x_l =
    cast(RMSNorm(r)) of every token; tau_x,l = the s1 quantile of the pooled
    |x_l|; |s~_l| of every token under that input mask (INT4 proxy); tau_s,l =
    the s2 quantile of the pooled |s~_l|; then every token passes layer l with
    both thresholds (r += y, in place).  Returns (tau_x, tau_s)."""
    N = r.shape[0]
    mb = L.shape.max_batch
    x = torch.empty(r.shape, dtype=L.dtype, device=r.device)
    for c in range(0, N, mb):
        prox.prox_rmsnorm(L, r[c:c + mb], eps, x[c:c + mb])
    tx = synth.calibrate_tau(x, s1)
    S = torch.empty(N, L.d_ff, dtype=torch.float32, device=r.device)
    y = torch.empty(1, L.d_model, dtype=L.dtype, device=r.device)
    for t in range(N):
        _abs_proxy_state(L, x[t:t + 1], tx, S[t], y)
    ts = synth.calibrate_tau(S, s2)
    for t in range(N):
        prox.prox_stack_forward_ts([L], [tx], [ts], r[t], eps)
    return (tx, ts, x) if return_input else (tx, ts)


def sequential_thresholds_ts(layers, calib_resid, s1: float, s2: float, eps: float = 1e-5,
                             return_inputs: bool = False):
    """Algorithm 1 of App. A.7 with both thresholds, layer by layer in depth
    order (calibrate_layer_ts).

    calib_resid: float32 [N][d_model] residual-stream calibration tokens (not
    modified).  Returns (taus_x, taus_s) or, with return_inputs, also the list
    of per-layer inputs x_l [N][d_model]."""
    r = calib_resid.detach().clone().contiguous()
    taus_x, taus_s, inputs = [], [], []
    for L in layers:
        tx, ts, x = calibrate_layer_ts(L, r, s1, s2, eps, return_input=True)
        taus_x.append(tx)
        taus_s.append(ts)
        if return_inputs:
            inputs.append(x)
    return (taus_x, taus_s, inputs) if return_inputs else (taus_x, taus_s)


def runtime_sparsity(layers, taus_x, taus_s, resid_tokens, eps: float = 1e-5,
                     alpha: float = costmodel.ALPHA):
    """Realized sparsities of a threshold-mask stack on tokens it was not
    calibrated on (App. A.7, runtime sparsity): the Stage 1 and Stage 2 mask
    counts of every layer and token are accumulated, then
    e = s2 - 2 alpha (1 - s1) / 3.  Returns a dict with s1, s2, e and the
    per-layer means."""
    n1_tot = nsel_tot = 0
    per_layer = []
    dev = resid_tokens.device
    for t in range(resid_tokens.shape[0]):
        r = resid_tokens[t].detach().clone().float().contiguous()
        for li, L in enumerate(layers):
            x = prox.prox_rmsnorm(L, r[None], eps)
            out = prox.prox_ffn_forward_ts_debug(L, x, taus_x[li], taus_s[li])
            n1 = int(out["n1"][0])
            ns = int(out["n_sel"][0])
            n1_tot += n1
            nsel_tot += ns
            if t == 0:
                per_layer.append([0, 0])
            per_layer[li][0] += n1
            per_layer[li][1] += ns
            prox.prox_stack_forward_ts([L], [taus_x[li]], [taus_s[li]], r, eps)
    T = resid_tokens.shape[0]
    L0 = layers[0]
    s1 = 1.0 - n1_tot / (T * len(layers) * L0.d_model)
    s2 = 1.0 - nsel_tot / (T * len(layers) * L0.d_ff)
    return dict(s1=s1, s2=s2, e=costmodel.effective_sparsity(s1, s2, alpha),
                per_layer=[dict(s1=1.0 - a / (T * L0.d_model), s2=1.0 - b / (T * L0.d_ff))
                           for a, b in per_layer])
