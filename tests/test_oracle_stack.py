"""Pins of the oracle's stack composition (normalize, FFN, cast y, add to
the residual) against a hand-derived two-layer stack, not against the
oracle's own other functions."""
import numpy as np

import oracle


def _layers(g):
    return [oracle.Layer(np.array(L["W_up"], np.float32), np.array(L["W_gate"], np.float32),
                         np.array(L["W_down"], np.float32), g["G"]) for L in g["layers"]]


def test_stack_composition_hand_fixture(golden):
    g = golden("stack_hand.json")
    layers = _layers(g)
    taus = [g["tau"]] * 2
    r, outs = oracle.stack_forward(layers, taus, g["k"], np.array(g["r0"]), g["eps"])
    for l, o in enumerate(outs):
        np.testing.assert_array_equal(o["x"], np.array(g["x"][l], np.float32))
        np.testing.assert_allclose(o["y"], g["y_exact"][l], rtol=1e-12, atol=0)
        np.testing.assert_array_equal(oracle.round_bf16(o["y"].astype(np.float32)),
                                      np.array(g["y_cast"][l], np.float32))
    # the residual carries the cast outputs exactly
    np.testing.assert_array_equal(r, np.array(g["r"][-1]))
    r1, _ = oracle.stack_forward(layers[:1], taus[:1], g["k"], np.array(g["r0"]), g["eps"])
    np.testing.assert_array_equal(r1, np.array(g["r"][0]))


def test_stack_ts_composition_hand_fixture(golden):
    """The threshold-mask stack with tau_s = 0 keeps every channel: the same
    residuals."""
    g = golden("stack_hand.json")
    layers = _layers(g)
    r, outs = oracle.stack_forward_ts(layers, [g["tau"]] * 2, [0.0] * 2, np.array(g["r0"]),
                                      g["eps"])
    np.testing.assert_array_equal(r, np.array(g["r"][-1]))
    for l, o in enumerate(outs):
        np.testing.assert_array_equal(o["x"], np.array(g["x"][l], np.float32))


def test_k0_layer_leaves_residual_bits_unchanged():
    rng = np.random.default_rng(7)
    d, f = 64, 96
    L = oracle.Layer(rng.normal(0, 0.02, (d, f)).astype(np.float32),
                     rng.normal(0, 0.02, (d, f)).astype(np.float32),
                     rng.normal(0, 0.02, (f, d)).astype(np.float32), 64)
    r0 = rng.normal(0, 1, d).astype(np.float32).astype(np.float64)
    r, outs = oracle.stack_forward([L, L], [0.1, 0.1], 0, r0)
    assert np.array_equal(r, r0)
    assert outs[0]["sel"].size == 0 and not np.any(outs[0]["y"])
