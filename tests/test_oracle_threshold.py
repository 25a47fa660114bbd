"""Pins of the oracle's Stage 2 threshold mask (Sec. 4.1, m_s equation with a
calibrated tau_s), the alternative to the per-token top-k of App. A.6.

Each pin ties the threshold form to something defined independently of it:
the top-k selection (sort-based, App. A.6), the Laplace energy closed form of
App. A.2, and the dense FFN (Sec. 2.1) at zero thresholds.
"""
from __future__ import annotations

import math

import numpy as np

import oracle


def _distinct_f32(rng, n, scale=1.0):
    """n distinct magnitudes that are exact float32 values (no rounding in the
    float32 comparison), with random signs."""
    while True:
        v = (rng.standard_normal(n) * scale).astype(np.float32)
        if np.unique(np.abs(v)).size == n:
            return v.astype(np.float64)


def test_threshold_at_kth_value_equals_topk():
    """|z| >= (k-th largest |z|) keeps exactly the top-k set when the values
    are distinct (App. A.6 top-k versus Sec. 4.1 threshold)."""
    rng = np.random.default_rng(11)
    z = _distinct_f32(rng, 3001)
    a = np.sort(np.abs(z))[::-1]
    for k in (1, 2, 57, 900, 3000, 3001):
        sel = oracle.threshold_mask(z, float(a[k - 1]))
        assert sel.tolist() == oracle.topk(z, k).tolist()


def test_threshold_limits_and_monotone():
    rng = np.random.default_rng(12)
    z = rng.standard_normal(500)
    assert oracle.threshold_mask(z, 0.0).tolist() == list(range(500))
    assert oracle.threshold_mask(z, -1.0).tolist() == list(range(500))
    assert oracle.threshold_mask(z, float("inf")).size == 0
    prev = None
    for t in np.linspace(0.0, 3.5, 40):
        cur = set(oracle.threshold_mask(z, float(t)).tolist())
        if prev is not None:
            assert cur <= prev
        prev = cur
    # the comparison keeps equality (>=): the exact value of a float32 entry
    zz = np.array([0.5, -0.25, 0.75, 0.25], dtype=np.float64)
    assert oracle.threshold_mask(zz, 0.25).tolist() == [0, 1, 2, 3]
    assert oracle.threshold_mask(zz, 0.5).tolist() == [0, 2]


def test_threshold_laplace_energy_closed_form(golden):
    """App. A.2, q_Lap: a threshold at the 70th percentile of |s| for Laplace
    s keeps ~87.9% of the squared energy."""
    pv = golden("pages_values.json")["laplace_energy_q_lap_0p7"]["value"]
    rng = np.random.default_rng(2025)
    s = rng.laplace(0.0, 0.9, 400_000)
    tau = -0.9 * math.log(1 - 0.7)  # the 0.7 quantile of |s| for scale 0.9
    sel = oracle.threshold_mask(s, tau)
    assert abs(sel.size / s.size - 0.3) < 0.005
    frac = np.sum(s[sel] ** 2) / np.sum(s ** 2)
    assert abs(frac - pv) < 0.006


def _tiny_layer(seed, d_model=64, d_ff=96, G=16):
    rng = np.random.default_rng(seed)
    Wu = rng.normal(0, 0.02, (d_model, d_ff)).astype(np.float32)
    Wg = rng.normal(0, 0.02, (d_model, d_ff)).astype(np.float32)
    Wd = rng.normal(0, 0.02, (d_ff, d_model)).astype(np.float32)
    x = rng.laplace(size=d_model).astype(np.float32)
    return Wu, Wg, Wd, x, G


def test_forward_ts_zero_thresholds_is_dense():
    Wu, Wg, Wd, x, G = _tiny_layer(5)
    out = oracle.forward_ts(oracle.Layer(Wu, Wg, Wd, G), x, 0.0, 0.0)
    _, y_dense = oracle.dense(x, Wu, Wg, Wd)
    assert out["sel"].tolist() == list(range(Wu.shape[1]))
    assert np.max(np.abs(out["y"] - y_dense)) <= 1e-12 * np.max(np.abs(y_dense))


def test_forward_ts_matches_topk_forward_at_kth_proxy_value():
    """With tau_s at the k-th largest float32 |s~| (no float32 ties there), the
    threshold step keeps the top-k channels and gives the top-k step's y."""
    Wu, Wg, Wd, x, G = _tiny_layer(6, d_model=128, d_ff=300, G=32)
    L = oracle.Layer(Wu, Wg, Wd, G)
    tau_x = float(np.sort(np.abs(x))[40])
    s_t = oracle.forward(L, x, tau_x, 1)["s_t"]
    a32 = np.sort(np.abs(s_t).astype(np.float32))[::-1]
    checked = 0
    for k in (5, 90, 150, 299):
        if a32[k - 1] == a32[k] or (k >= 2 and a32[k - 2] == a32[k - 1]):
            continue
        ts = oracle.forward_ts(L, x, tau_x, float(a32[k - 1]))
        tk = oracle.forward(L, x, tau_x, k)
        assert ts["sel"].tolist() == tk["sel"].tolist()
        np.testing.assert_array_equal(ts["y"], tk["y"])
        checked += 1
    assert checked >= 3


# ---------------------------------------------------------------------------
# Sequential calibration (App. A.7, Algorithm 1)
# ---------------------------------------------------------------------------
def test_lower_quantile_counts():
    """With N distinct values, the threshold at quantile q keeps exactly
    N - floor(q (N - 1)) of them under the >= rule: the realized sparsity on
    the calibration set is q up to one part in N."""
    rng = np.random.default_rng(13)
    v = np.abs(_distinct_f32(rng, 1000))
    for q in (0.0, 0.3, 0.5, 0.7, 0.767, 1.0):
        t = oracle.lower_quantile(v, q)
        kept = int(np.sum(v >= t))
        assert kept == 1000 - math.floor(q * 999)
        assert abs((1 - kept / 1000) - q) <= 1 / 1000 + 1e-12


def _stack(nl=3, d_model=64, d_ff=96, G=16, seed=20):
    rng = np.random.default_rng(seed)
    layers = []
    for _ in range(nl):
        Wu = rng.normal(0, 0.05, (d_model, d_ff)).astype(np.float32)
        Wg = rng.normal(0, 0.05, (d_model, d_ff)).astype(np.float32)
        Wd = rng.normal(0, 0.05, (d_ff, d_model)).astype(np.float32)
        layers.append(oracle.Layer(Wu, Wg, Wd, G))
    R0 = rng.standard_t(4, size=(12, d_model))
    return layers, R0


def test_calibration_keeps_everything_at_zero_targets_and_is_dense():
    """s1 = s2 = 0: every threshold is the smallest value seen, nothing is
    pruned on the calibration tokens, and the calibrated stack equals the
    dense stack (k = d_ff, tau_x = 0) on them."""
    layers, R0 = _stack()
    tx, ts, X = oracle.calibrate_sequential(layers, R0, 0.0, 0.0)
    for t in range(R0.shape[0]):
        r_ts, _ = oracle.stack_forward_ts(layers, tx, ts, R0[t])
        r_dense, _ = oracle.stack_forward(layers, [0.0] * len(layers), layers[0].d_ff, R0[t])
        np.testing.assert_allclose(r_ts, r_dense, rtol=0, atol=1e-12 * np.max(np.abs(r_dense)))


def test_calibration_realizes_targets_on_its_tokens():
    """Each layer's thresholds, applied to the inputs that layer saw during
    calibration, prune the target fractions (up to quantile granularity), and
    those inputs are what the calibrated earlier layers produce."""
    layers, R0 = _stack(nl=3)
    s1, s2 = 0.5, 0.7
    tx, ts, X = oracle.calibrate_sequential(layers, R0, s1, s2)
    def quantile_counts(v, t, q):
        # lower empirical quantile t at q: at most floor(q (N-1)) values lie
        # strictly below it and at least floor(q (N-1)) + 1 lie at or below
        m = math.floor(q * (v.size - 1))
        assert np.sum(v < t) <= m < np.sum(v <= t)

    for l in range(len(layers)):
        ax = np.abs(X[l].astype(np.float32)).ravel()
        quantile_counts(ax, np.float32(tx[l]), s1)
        sv, kept_s = [], 0
        for x in X[l]:
            o = oracle.forward_ts(layers[l], x, tx[l], ts[l])
            sv.append(np.abs(o["s_t"]).astype(np.float32))
            kept_s += o["sel"].size
        sv = np.concatenate(sv)
        quantile_counts(sv, np.float32(ts[l]), s2)
        assert kept_s == int(np.sum(sv >= np.float32(ts[l])))
        assert abs((1 - kept_s / sv.size) - s2) <= 0.02
    # depth order: layer l's inputs are the stack's inputs with layers < l calibrated
    for t in range(R0.shape[0]):
        _, outs = oracle.stack_forward_ts(layers, tx, ts, R0[t])
        for l in range(len(layers)):
            np.testing.assert_array_equal(outs[l]["x"], X[l][t])
