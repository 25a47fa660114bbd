"""Pins of the CPU oracle against what the paper and the mathematics fix.

None of these compares the oracle with itself: each check is a closed form
printed in the paper, a brute-force definition written differently from the
oracle's, a hand-derived fixture, or an exact reduction (zero sparsity equals
dense; the full-precision proxy equals the exact state).

Paper: "Prox: Training-Free FFN Activation Sparsity via Approximate
Intermediate-Channel Salience in LLMs" (arXiv 2607.27591).
"""
import math

import numpy as np
import pytest

import oracle


def _silu(z):
    return z / (1.0 + math.exp(-z))


# ---------------------------------------------------------------------------
# Quantizer (Sec. 4.3; reading: codes in [-7, 7], scale = absmax / 7)
# ---------------------------------------------------------------------------
def test_quantize_hand_fixture(golden):
    fx = golden("quantize_hand.json")
    W = np.array(fx["W"], dtype=np.float32)
    q, sc = oracle.quantize(W, fx["G"])
    assert sc.shape == (1, W.shape[1])
    np.testing.assert_array_equal(sc[0], np.array(fx["scale"], dtype=np.float32))
    np.testing.assert_array_equal(q, np.array(fx["q"], dtype=np.int8))


@pytest.mark.parametrize("G", [8, 64, 128])
def test_quantize_round_trip_and_absmax(G):
    rng = np.random.default_rng(1234 + G)
    d_model, d_ff = 4 * G, 96
    W = rng.normal(0.0, 0.02, (d_model, d_ff)).astype(np.float32)
    W[:, 5] = 0.0                      # an all-zero column in every group
    W[G:2 * G, 7] = 0.0                # an all-zero group in one column
    W[3, 9] = -0.5                     # a negative absmax
    q, sc = oracle.quantize(W, G)
    assert q.dtype == np.int8 and q.min() >= -7 and q.max() <= 7
    deq = q.astype(np.float64) * np.repeat(sc.astype(np.float64), G, axis=0)
    err = np.abs(W.astype(np.float64) - deq)
    bound = np.repeat(sc.astype(np.float64), G, axis=0) * (0.5 + 2.0 ** -20)
    assert np.all(err <= bound)
    for g in range(d_model // G):
        blk = W[g * G:(g + 1) * G]
        qb = q[g * G:(g + 1) * G]
        for j in range(d_ff):
            a = np.max(np.abs(blk[:, j]))
            if a == 0.0:
                assert sc[g, j] == 0.0 and not qb[:, j].any()
            else:
                i = int(np.argmax(np.abs(blk[:, j])))
                assert abs(int(qb[i, j])) == 7
                assert np.sign(qb[i, j]) == np.sign(blk[i, j])
                assert sc[g, j] == np.float32(a) / np.float32(7.0)


def test_quantize_rejects_ragged_group():
    with pytest.raises(ValueError):
        oracle.quantize(np.zeros((100, 8), np.float32), 64)


# ---------------------------------------------------------------------------
# Stage 1 input mask (Sec. 4.1, m_x equation: |x_i| >= tau keeps)
# ---------------------------------------------------------------------------
def test_input_mask_hand_cases():
    x = np.array([0.5, -0.5, 0.49999997, -2.0, 0.0, 3.0, -0.25], np.float32)
    assert oracle.input_mask(x, 0.5).tolist() == [0, 1, 3, 5]
    assert oracle.input_mask(x, 0.0).tolist() == list(range(7))
    assert oracle.input_mask(x, -1.0).tolist() == list(range(7))
    assert oracle.input_mask(x, float("inf")).tolist() == []
    assert oracle.input_mask(x, 3.0).tolist() == [5]


def test_input_mask_brute_force():
    rng = np.random.default_rng(7)
    for _ in range(20):
        x = rng.laplace(size=300).astype(np.float32)
        tau = float(np.float32(abs(x[rng.integers(300)])))
        want = [i for i in range(300) if not (abs(float(x[i])) < tau)]
        assert oracle.input_mask(x, tau).tolist() == want


# ---------------------------------------------------------------------------
# Top-k (App. A.6, top-k equation; ties to the lower index)
# ---------------------------------------------------------------------------
def _rank_select(z, k):
    """Brute force: j is kept iff fewer than k channels outrank it, where i
    outranks j when |z_i| > |z_j|, or |z_i| == |z_j| and i < j."""
    a = [abs(float(v)) for v in z]
    out = []
    for j in range(len(a)):
        better = sum(1 for i in range(len(a)) if a[i] > a[j] or (a[i] == a[j] and i < j))
        if better < k:
            out.append(j)
    return out


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(11)
    for trial in range(30):
        n = int(rng.integers(1, 40))
        z = rng.choice([-2.0, -1.0, -0.5, 0.0, 0.5, 1.0, 2.0, 3.0], size=n)
        z = z + (trial % 2) * rng.normal(0, 1e-3, n) * (rng.random(n) < 0.3)
        for k in range(n + 1):
            assert oracle.topk(z, k).tolist() == _rank_select(z, k)


def test_topk_sign_insensitive_and_popcount():
    rng = np.random.default_rng(3)
    z = rng.normal(size=500)
    for k in (0, 1, 17, 250, 499, 500):
        sel = oracle.topk(z, k)
        assert sel.size == k and len(set(sel.tolist())) == k
        assert np.all(np.diff(sel) > 0)
        assert sel.tolist() == oracle.topk(-z, k).tolist() == oracle.topk(np.abs(z), k).tolist()


def test_topk_all_zero_takes_lowest_indices():
    for k in (0, 1, 5, 64):
        assert oracle.topk(np.zeros(64), k).tolist() == list(range(k))


def test_topk_rejects_bad_k():
    with pytest.raises(ValueError):
        oracle.topk(np.zeros(4), 5)


def test_topk_rank_preservation_bound():
    """App. A.2: if ||s_i| - |s_j|| > |d_i| + |d_j| the order of i and j under
    |s + d| is the order under |s|; so a perturbation bounded that way cannot
    change the top-k set when every kept/dropped pair is separated enough."""
    rng = np.random.default_rng(5)
    s = rng.laplace(size=400)
    k = 120
    sel = set(oracle.topk(s, k).tolist())
    a = np.sort(np.abs(s))[::-1]
    gap = a[k - 1] - a[k]
    d = rng.uniform(-1, 1, 400) * (0.49 * gap)
    assert set(oracle.topk(s + d, k).tolist()) == sel


def test_laplace_energy_closed_form(golden):
    """App. A.2, q_Lap equation: keeping the largest-magnitude 30% of a Laplace
    sample keeps ~87.9% of its squared energy."""
    pv = golden("pages_values.json")["laplace_energy_q_lap_0p7"]["value"]
    p = 0.7
    a = -math.log(1 - p)
    closed = (1 - p) / 2 * (a * a + 2 * a + 2)
    assert abs(closed - pv) <= 0.0005
    rng = np.random.default_rng(2024)
    n = 400_000
    s = rng.laplace(0.0, 1.7, n)
    sel = oracle.topk(s, int(round((1 - p) * n)))
    frac = np.sum(s[sel] ** 2) / np.sum(s ** 2)
    assert abs(frac - pv) < 0.006


# ---------------------------------------------------------------------------
# Gaussian closed forms (App. A.2): energy, relative error, correlation
# ---------------------------------------------------------------------------
def test_gaussian_closed_forms(golden):
    pv = golden("pages_values.json")
    qg = pv["gaussian_energy_q_g_0p7"]["value"]
    eta = pv["gaussian_rel_rms_error_eta_0p7"]["value"]
    corr = pv["gaussian_corr_0p7"]["value"]
    rng = np.random.default_rng(99)
    d_in, d_out = 3000, 1500
    W = rng.normal(size=(d_in, d_out))
    qs, es, cs = [], [], []
    for _ in range(4):
        x = rng.normal(size=d_in).astype(np.float32)
        tau = float(np.sort(np.abs(x))[int(0.7 * d_in)])
        idx = oracle.input_mask(x, tau)
        assert abs(idx.size - 0.3 * d_in) <= 2
        u_sp, _, _ = oracle.proxy(x, idx, W, W)
        u, _, _ = oracle.proxy(x, np.arange(d_in, dtype=np.int32), W, W)
        qs.append(np.sum(x[idx].astype(np.float64) ** 2) / np.sum(x.astype(np.float64) ** 2))
        es.append(np.linalg.norm(u - u_sp) / np.linalg.norm(u))
        cs.append(np.corrcoef(u, u_sp)[0, 1])
    assert abs(np.mean(qs) - qg) < 0.01
    assert abs(np.mean(es) - eta) < 0.012
    assert abs(np.mean(cs) - corr) < 0.01


# ---------------------------------------------------------------------------
# Whole-step reductions
# ---------------------------------------------------------------------------
def _tiny_layer(seed, d_model=64, d_ff=96, G=16):
    rng = np.random.default_rng(seed)
    Wu = rng.normal(0, 0.02, (d_model, d_ff)).astype(np.float32)
    Wg = rng.normal(0, 0.02, (d_model, d_ff)).astype(np.float32)
    Wd = rng.normal(0, 0.02, (d_ff, d_model)).astype(np.float32)
    x = rng.laplace(size=d_model).astype(np.float32)
    return Wu, Wg, Wd, x, G


def test_zero_sparsity_equals_dense():
    Wu, Wg, Wd, x, G = _tiny_layer(1)
    L = oracle.Layer(Wu, Wg, Wd, G)
    out = oracle.forward(L, x, 0.0, Wu.shape[1])
    _, y_dense = oracle.dense(x, Wu, Wg, Wd)
    assert out["idx"].size == x.size
    assert out["sel"].tolist() == list(range(Wu.shape[1]))
    assert np.max(np.abs(out["y"] - y_dense)) <= 1e-12 * np.max(np.abs(y_dense))


def test_full_precision_proxy_is_oracle_s():
    """Sec. 3.1 oracle-s: with the proxy weights equal to the original weights
    and no input threshold, s~ is the exact state and the mask is the exact
    top-k of |s| (checked with the brute-force rank definition)."""
    Wu, Wg, Wd, x, G = _tiny_layer(2)
    L = oracle.Layer(Wu, Wg, Wd, G, full_precision_proxy=True)
    s_exact, _ = oracle.dense(x, Wu, Wg, Wd)
    for k in (0, 1, 29, 48, 96):
        out = oracle.forward(L, x, 0.0, k)
        assert np.max(np.abs(out["s_t"] - s_exact)) <= 1e-12 * np.max(np.abs(s_exact))
        assert out["sel"].tolist() == _rank_select(s_exact, k)
        np.testing.assert_allclose(out["s_sp"], s_exact[out["sel"]], rtol=1e-12, atol=0)


def test_no_survivors_selects_lowest_indices():
    Wu, Wg, Wd, x, G = _tiny_layer(3)
    L = oracle.Layer(Wu, Wg, Wd, G)
    for k in (0, 7, 50):
        out = oracle.forward(L, x, float("inf"), k)
        assert out["idx"].size == 0
        assert not np.any(out["s_t"])
        assert out["sel"].tolist() == list(range(k))


def test_k_zero_gives_zero_output():
    Wu, Wg, Wd, x, G = _tiny_layer(4)
    out = oracle.forward(oracle.Layer(Wu, Wg, Wd, G), x, 0.5, 0)
    assert out["sel"].size == 0 and not np.any(out["y"])


def _brute_force_step(x, Wt_u, Wt_g, Wu, Wg, Wd, tau, k):
    """Pure-Python transcription of the step in the masked-product form of
    App. A.7 (s~ = W~up^T (m_x . x) . SiLU(W~gate^T (m_x . x))) followed by the
    Stage 2 equations of Sec. 4.1 written with an explicit channel mask."""
    d_model, d_ff = Wu.shape
    m_x = [1.0 if abs(float(x[i])) >= tau else 0.0 for i in range(d_model)]
    xm = [m_x[i] * float(x[i]) for i in range(d_model)]
    st = []
    for j in range(d_ff):
        ut = sum(xm[i] * float(Wt_u[i][j]) for i in range(d_model))
        gt = sum(xm[i] * float(Wt_g[i][j]) for i in range(d_model))
        st.append(ut * _silu(gt))
    keep = set(_rank_select(st, k))
    m_s = [1.0 if j in keep else 0.0 for j in range(d_ff)]
    s = []
    for j in range(d_ff):
        u = sum(float(x[i]) * float(Wu[i][j]) for i in range(d_model))
        g = sum(float(x[i]) * float(Wg[i][j]) for i in range(d_model))
        s.append(m_s[j] * u * _silu(g))
    y = [sum(s[j] * float(Wd[j][c]) for j in range(d_ff)) for c in range(d_model)]
    return sorted(keep), st, y


def test_brute_force_tiny_int4_exact_weights():
    """Weights placed exactly on each group's INT4 grid (absmax = 7 * scale), so
    the INT4 proxy must reproduce them exactly; the whole step then matches the
    pure-Python masked-product transcription for every k."""
    rng = np.random.default_rng(21)
    d_model, d_ff, G = 16, 24, 4

    def grid_matrix():
        codes = rng.integers(-7, 8, (d_model, d_ff)).astype(np.float32)
        codes[::G, :] = 7.0 * np.where(rng.random(d_ff) < 0.5, -1.0, 1.0)
        steps = np.float32(2.0) ** rng.integers(-9, -5, (d_model // G, d_ff)).astype(np.float32)
        return codes * np.repeat(steps, G, axis=0)

    Wu, Wg = grid_matrix(), grid_matrix()
    Wd = rng.normal(0, 0.1, (d_ff, d_model)).astype(np.float32)
    L = oracle.Layer(Wu, Wg, Wd, G)
    np.testing.assert_array_equal(L.Wt_up, Wu.astype(np.float64))
    np.testing.assert_array_equal(L.Wt_gate, Wg.astype(np.float64))
    for trial in range(3):
        x = rng.laplace(size=d_model).astype(np.float32)
        tau = float(np.sort(np.abs(x))[6 + trial])
        for k in range(d_ff + 1):
            out = oracle.forward(L, x, tau, k)
            sel, st, y = _brute_force_step(x, Wu, Wg, Wu, Wg, Wd, tau, k)
            assert out["sel"].tolist() == sel
            np.testing.assert_allclose(out["s_t"], st, rtol=1e-12, atol=1e-15)
            np.testing.assert_allclose(out["y"], y, rtol=1e-10, atol=1e-13)


def test_brute_force_tiny_random_weights():
    """Same transcription with arbitrary weights; the proxy side uses the
    oracle's (separately pinned) quantizer output."""
    rng = np.random.default_rng(22)
    d_model, d_ff, G = 12, 20, 4
    Wu = rng.normal(0, 0.3, (d_model, d_ff)).astype(np.float32)
    Wg = rng.normal(0, 0.3, (d_model, d_ff)).astype(np.float32)
    Wd = rng.normal(0, 0.3, (d_ff, d_model)).astype(np.float32)
    L = oracle.Layer(Wu, Wg, Wd, G)
    Wt_u = [[float(L.q_up[i, j]) * float(L.sc_up[i // G, j]) for j in range(d_ff)]
            for i in range(d_model)]
    Wt_g = [[float(L.q_gate[i, j]) * float(L.sc_gate[i // G, j]) for j in range(d_ff)]
            for i in range(d_model)]
    x = rng.laplace(size=d_model).astype(np.float32)
    tau = float(np.sort(np.abs(x))[4])
    for k in range(d_ff + 1):
        out = oracle.forward(L, x, tau, k)
        sel, st, y = _brute_force_step(x, Wt_u, Wt_g, Wu, Wg, Wd, tau, k)
        assert out["sel"].tolist() == sel
        np.testing.assert_allclose(out["y"], y, rtol=1e-10, atol=1e-13)


# ---------------------------------------------------------------------------
# Stack glue: RMSNorm (unit gain) and the bf16 cast
# ---------------------------------------------------------------------------
def test_round_bf16_hand_values():
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20,
                  -2.5, 65504.0, 3.0e38, 1e-40], np.float32)
    want = np.array([1.0, 1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -2.5, 65536.0,
                     np.float32(3.0e38), np.float32(1e-40)], np.float64)
    got = oracle.round_bf16(v).astype(np.float64)
    assert got[:6].tolist() == want[:6].tolist()
    # 3e38 lies between bf16 neighbours 2.9910e38 and 3.0070e38; nearest is the latter.
    assert got[6] == float(np.frombuffer(np.uint32(0x7F62 << 16).tobytes(), np.float32)[0])
    assert np.frombuffer(got[7:8].astype(np.float32).tobytes(), np.uint32)[0] & 0xFFFF == 0


def test_rmsnorm_closed_form():
    r = np.array([3.0, -4.0, 0.0, 5.0])
    x = oracle.rmsnorm(r, eps=0.0, to_bf16=False)
    np.testing.assert_allclose(x, r / math.sqrt(50.0 / 4.0), rtol=1e-7)
    xb = oracle.rmsnorm(r, eps=1e-5, to_bf16=True)
    assert np.all(np.frombuffer(xb.tobytes(), np.uint32) & 0xFFFF == 0)
