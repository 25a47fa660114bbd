"""Sequential per-layer threshold calibration for an FFN stack.

Paper: "Prox: Training-Free FFN Activation Sparsity ...", App. A.7
(Algorithm 1, sequential threshold calibration): layers are calibrated in
depth order, and layer l's inputs are collected after the calibration tokens
went through layers 1..l-1 with their finalized sparse rules.  Only the input
threshold tau_x is calibrated here (the Stage 2 mask is a per-token top-k);
tau_x,l is the lower empirical quantile of the pooled |x_l|.

Every step runs on the GPU through libprox (normalization, sparse forward,
residual update); only the quantile is taken on the host.
"""
from __future__ import annotations

import torch

from . import prox, synth


def sequential_thresholds(layers, calib_resid, quantile: float, k: int, eps: float = 1e-5):
    """Thresholds tau_x for each layer of a stack.

    calib_resid: float32 [N][d_model] residual-stream calibration tokens (not
    modified).  Returns a list of floats, one per layer."""
    r = calib_resid.detach().clone().contiguous()
    N = r.shape[0]
    mb = min(layer.shape.max_batch for layer in layers)
    taus = []
    for L in layers:
        x = torch.empty(r.shape, dtype=L.dtype, device=r.device)
        for c in range(0, N, mb):
            prox.prox_rmsnorm(L, r[c:c + mb], eps, x[c:c + mb])
        tau = synth.calibrate_tau(x, quantile)
        taus.append(tau)
        for c in range(0, N, mb):
            prox.prox_stack_forward([L], [tau], k, r[c:c + mb], eps)
    return taus
