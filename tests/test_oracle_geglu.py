"""Pins of the oracle's gate activations: SiLU for SwiGLU (the pages' FFN,
Sec. 2.1) and the tanh form of GELU for the GeGLU variant (Gemma-3 style
models, evaluated in Sec. 5; the pages name the model family, not the
formula, so the standard tanh form is the reading adopted).

Pins: the exact erf form of GELU (a textbook function, math.erf) bounds the
tanh form to within 5e-4; both activations satisfy a(z) - a(-z) = z; limits;
and the whole GeGLU step reduces to the dense GeGLU FFN and to the exact
top-k of |s| exactly as the SwiGLU step does.
"""
from __future__ import annotations

import math

import numpy as np

import oracle


def test_gelu_tanh_against_erf_form():
    worst = 0.0
    for z in np.linspace(-8.0, 8.0, 4001):
        exact = 0.5 * z * (1.0 + math.erf(z / math.sqrt(2.0)))
        worst = max(worst, abs(oracle.gate_act(z, 1) - exact))
    assert worst <= 5e-4
    assert worst >= 1e-4  # it is the tanh form, not the erf form


def test_gate_activations_odd_part_and_limits():
    for act in (0, 1):
        assert oracle.gate_act(0.0, act) == 0.0
        for z in (0.1, 0.7, 1.3, 2.9, 6.0):
            assert abs(oracle.gate_act(z, act) - oracle.gate_act(-z, act) - z) <= 1e-14
        assert abs(oracle.gate_act(40.0, act) - 40.0) <= 1e-9
        assert abs(oracle.gate_act(-40.0, act)) <= 1e-9
    # SiLU hand value: z sigma(z) at z = ln 3 is ln(3) * 3/4
    assert abs(oracle.gate_act(math.log(3.0), 0) - 0.75 * math.log(3.0)) <= 1e-15


def _tiny_layer(seed, d_model=64, d_ff=96, G=16):
    rng = np.random.default_rng(seed)
    Wu = rng.normal(0, 0.1, (d_model, d_ff)).astype(np.float32)
    Wg = rng.normal(0, 0.1, (d_model, d_ff)).astype(np.float32)
    Wd = rng.normal(0, 0.1, (d_ff, d_model)).astype(np.float32)
    x = rng.laplace(size=d_model).astype(np.float32)
    return Wu, Wg, Wd, x, G


def test_geglu_zero_sparsity_equals_dense_geglu():
    Wu, Wg, Wd, x, G = _tiny_layer(31)
    out = oracle.forward(oracle.Layer(Wu, Wg, Wd, G, act=1), x, 0.0, Wu.shape[1])
    s_dense, y_dense = oracle.dense(x, Wu, Wg, Wd, act=1)
    assert np.max(np.abs(out["y"] - y_dense)) <= 1e-12 * np.max(np.abs(y_dense))
    # the dense state is u * GELU(g) element by element
    u = x.astype(np.float64) @ Wu.astype(np.float64)
    g = x.astype(np.float64) @ Wg.astype(np.float64)
    ref = np.array([u[j] * oracle.gate_act(g[j], 1) for j in range(u.size)])
    assert np.max(np.abs(s_dense - ref)) <= 1e-12 * np.max(np.abs(ref))
    # and differs from the SwiGLU state
    s_swi, _ = oracle.dense(x, Wu, Wg, Wd, act=0)
    assert np.max(np.abs(s_swi - s_dense)) > 1e-3 * np.max(np.abs(s_dense))


def test_geglu_full_precision_proxy_is_exact_topk():
    Wu, Wg, Wd, x, G = _tiny_layer(32)
    L = oracle.Layer(Wu, Wg, Wd, G, full_precision_proxy=True, act=1)
    s_exact, _ = oracle.dense(x, Wu, Wg, Wd, act=1)
    a = np.abs(s_exact)
    for k in (1, 30, 95):
        out = oracle.forward(L, x, 0.0, k)
        assert np.max(np.abs(out["s_t"] - s_exact)) <= 1e-12 * np.max(a)
        want = sorted(j for j in range(a.size)
                      if sum(1 for i in range(a.size) if a[i] > a[j] or (a[i] == a[j] and i < j)) < k)
        assert out["sel"].tolist() == want
