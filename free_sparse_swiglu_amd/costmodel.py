"""Normalized cost model and target-aware allocation of the two stages.

Paper: "Prox: Training-Free FFN Activation Sparsity via Approximate
Intermediate-Channel Salience in LLMs", Sec. 4.2 (cost model and effective
sparsity), Sec. 5 (alpha = 1/3), App. A.4 (worked allocations), App. A.7
(runtime effective sparsity from measured mask counts).

Used for reporting the realised Stage 1 / Stage 2 sparsities of a run and the
effective sparsity they imply; the kernels do not depend on it.
"""
from __future__ import annotations

ALPHA = 1.0 / 3.0
S_REF = 0.7
S1_RANGE = (0.0, 0.7)


def prox_cost(s1: float, s2: float, alpha: float = ALPHA) -> float:
    """C_Prox = 2 alpha (1 - s1) + 3 (1 - s2), dense cost being 3 (Sec. 4.2)."""
    return 2.0 * alpha * (1.0 - s1) + 3.0 * (1.0 - s2)


def effective_sparsity(s1: float, s2: float, alpha: float = ALPHA) -> float:
    """e = 1 - C_Prox / 3 = s2 - 2 alpha (1 - s1) / 3 (Sec. 4.2)."""
    return 1.0 - prox_cost(s1, s2, alpha) / 3.0


def allocate(e: float, alpha: float = ALPHA, s_ref: float = S_REF,
             s1_range=S1_RANGE):
    """Target-aware allocation (Sec. 4.2): start from s2 = s_ref, give the rest
    of the budget to Stage 1; if that s1 leaves [s1_min, s1_max], clamp it and
    solve the effective-sparsity relation for s2 instead.  Returns (s1, s2)."""
    s2 = s_ref
    s1 = 1.0 - 3.0 * (s2 - e) / (2.0 * alpha)
    lo, hi = s1_range
    if s1 < lo or s1 > hi:
        s1 = min(max(s1, lo), hi)
        s2 = e + 2.0 * alpha * (1.0 - s1) / 3.0
    return s1, s2
