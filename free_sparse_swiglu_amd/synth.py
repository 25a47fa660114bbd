"""Seeded synthetic workloads for the Prox FFN step.

This module only draws inputs: layer weights, token activations and the
per-layer input threshold calibrated from them.  It holds none of the FFN
arithmetic, and both the HIP path and the CPU oracle consume what it makes.

The real models and the Alpaca calibration text of the paper ("Prox:
Training-Free FFN Activation Sparsity ...", App. A.7) are not available, so
seeded draws of the same shapes stand in for them:

  tiny   d_model 256,  d_ff 688,   fp32, x ~ Laplace(0, 1), G = 64,
         tau = 40th percentile of |x| over 64 calibration inputs
  8b     d_model 4096, d_ff 14336, bf16, G = 128
  14b    d_model 5120, d_ff 17408, bf16, G = 128
  70b    d_model 8192, d_ff 28672, bf16, G = 128

For the bf16 shapes x ~ Student-t(nu = 4); each vector is divided by its own
empirical RMS, then a fixed set of round(0.001 * d_model) outlier channels
(drawn once per layer) is multiplied by 20, then the vector is cast to bf16;
tau is the 50% quantile of |x| over 256 calibration inputs.  Weights are
N(0, 0.02^2) cast to the layer dtype.
"""
from __future__ import annotations

import math
import zlib
from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Config:
    name: str
    d_model: int
    d_ff: int
    group: int
    dtype: str  # "f32" or "bf16"
    x_dist: str  # "laplace" or "student_t"
    tau_quantile: float
    n_calib: int
    sparsities: tuple = field(default=(0.7,))
    batches: tuple = field(default=(1,))
    layers: int = 1


CONFIGS = {
    "tiny": Config("tiny", 256, 688, 64, "f32", "laplace", 0.40, 64, (0.7,)),
    "8b": Config("8b", 4096, 14336, 128, "bf16", "student_t", 0.50, 256, (0.5, 0.6, 0.7)),
    "14b": Config("14b", 5120, 17408, 128, "bf16", "student_t", 0.50, 256, (0.6, 0.7)),
    "stack8b": Config("stack8b", 4096, 14336, 128, "bf16", "student_t", 0.50, 256, (0.7,),
                      layers=32),
    "70b": Config("70b", 8192, 28672, 128, "bf16", "student_t", 0.50, 256, (0.7,),
                  batches=(1, 2, 4, 8)),
}


def k_for(d_ff: int, sparsity: float) -> int:
    """Channels kept at a given FFN sparsity: (1 - P) of d_ff, nearest integer."""
    return int(math.floor((1.0 - sparsity) * d_ff + 0.5))


def torch_dtype(dtype: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def seed_for(*parts) -> int:
    """Stable 63-bit seed from a tuple of labels (config, layer, purpose, ...)."""
    text = "|".join(str(p) for p in parts).encode()
    return (zlib.crc32(text) << 31) ^ zlib.crc32(text[::-1] + b"#")


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_for(*parts))
    return g


def make_layer(cfg: Config, layer: int = 0, device="cpu"):
    """Weights of one FFN layer in the paper's x.W layout:
    W_up, W_gate [d_model][d_ff] and W_down [d_ff][d_model], N(0, 0.02^2)."""
    dt = torch_dtype(cfg.dtype)
    out = []
    for name, shape in (("up", (cfg.d_model, cfg.d_ff)), ("gate", (cfg.d_model, cfg.d_ff)),
                        ("down", (cfg.d_ff, cfg.d_model))):
        w = torch.randn(shape, generator=_gen(device, cfg.name, layer, name), device=device,
                        dtype=torch.float32)
        w.mul_(0.02)
        out.append(w.to(dt))
    return tuple(out)


def outlier_channels(cfg: Config, layer: int = 0) -> torch.Tensor:
    """The fixed outlier input channels of a layer (round(0.001 d_model), >= 1)."""
    n = max(1, int(math.floor(0.001 * cfg.d_model + 0.5)))
    perm = torch.randperm(cfg.d_model, generator=_gen("cpu", cfg.name, layer, "outliers"))
    return torch.sort(perm[:n]).values


def make_inputs(cfg: Config, n: int, purpose: str, layer: int = 0, device="cpu"):
    """n token activations [n][d_model] in the layer dtype.

    purpose is a label ("calib", "test", "bench", ...) so that calibration and
    evaluation inputs are distinct draws."""
    g = _gen(device, cfg.name, layer, purpose, n)
    shape = (n, cfg.d_model)
    if cfg.x_dist == "laplace":
        # Laplace(0, 1) as the difference of two unit exponentials.
        e1 = torch.empty(shape, device=device).exponential_(1.0, generator=g)
        e2 = torch.empty(shape, device=device).exponential_(1.0, generator=g)
        x = e1 - e2
    elif cfg.x_dist == "student_t":
        # Student-t with nu = 4: Z / sqrt(V / 4), V a chi-square with 4 dof.
        z = torch.randn(shape, generator=g, device=device)
        v = torch.zeros(shape, device=device)
        for _ in range(4):
            v.add_(torch.randn(shape, generator=g, device=device).square())
        x = z / torch.sqrt(v / 4.0)
        x = x / torch.sqrt(torch.mean(x.square(), dim=1, keepdim=True))
        oc = outlier_channels(cfg, layer).to(device)
        x[:, oc] *= 20.0
    else:
        raise ValueError(cfg.x_dist)
    return x.to(torch_dtype(cfg.dtype))


def calibrate_tau(xs: torch.Tensor, quantile: float) -> float:
    """Per-layer input threshold: the lower empirical quantile of the pooled
    |x| of the calibration inputs, sorted[floor(q (N - 1))] (no interpolation)."""
    a = xs.detach().abs().float().reshape(-1).cpu().numpy()
    a.sort(kind="stable")
    return float(np.float32(a[int(math.floor(quantile * (a.size - 1)))]))


def layer_tau(cfg: Config, layer: int = 0, device="cpu") -> float:
    """tau for a single layer calibrated on cfg.n_calib seeded inputs."""
    return calibrate_tau(make_inputs(cfg, cfg.n_calib, "calib", layer, device),
                         cfg.tau_quantile)
