"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars (checked element by element on the same seeded inputs):
  - prepared INT4 codes and scales: bit-exact with the oracle's quantizer;
  - Stage 1 survivors (count and ascending list): bit-exact;
  - |s~|: max |diff| <= 1e-4 * max |s~| (float32 vs double summation);
  - top-k mask: exactly k ascending channels, differing from the oracle's only
    inside the 1e-3 tie band around the k-th value (tests/parity_utils.py);
  - exact s of the selected channels: max |diff| <= 1e-4 * max |s|;
  - y: max |diff| / max |y_ref| <= 2e-2 (bf16 weights, float32 accumulation)
    or <= 1e-5 (float32 layer).
Configurations: the tiny float32 layer, a ragged bf16 layer (several proxy
tiles plus a partial one), and the 8B / 14B / 70B shapes at full size.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from free_sparse_swiglu_amd import prox, synth
from tests.parity_utils import check_mask, check_threshold_mask, expected_y, rel_err

pytestmark = pytest.mark.gpu

DEV = "cuda"
RAGGED = synth.Config("ragged", 1024, 3000, 128, "bf16", "student_t", 0.5, 32, (0.7,))


def _tol(cfg):
    return 1e-5 if cfg.dtype == "f32" else 2e-2


class Case:
    """A layer on both sides: GPU prepared layer + oracle layer (+ dense s)."""

    def __init__(self, cfg, layer=0, gen_device="cpu", max_batch=1, act=0, **choices):
        self.cfg = cfg
        self.act = act
        W = synth.make_layer(cfg, layer, gen_device)
        self.Wg_dev = [w.to(DEV) for w in W]
        self.L = prox.prox_prepare_layer(*self.Wg_dev, cfg.group, max_batch, activation=act,
                                         **choices)
        self.Wnp = [w.float().cpu().numpy() for w in W]
        self.ol = oracle.Layer(*self.Wnp, cfg.group, act=act)
        calib = synth.make_inputs(cfg, cfg.n_calib, "calib", layer, gen_device)
        self.tau = synth.calibrate_tau(calib, cfg.tau_quantile)

    def inputs(self, n, purpose="test"):
        return synth.make_inputs(self.cfg, n, purpose, 0, "cpu")


_CASES = {}


def get_case(cfg, gen_device="cpu", max_batch=1, act=0):
    key = (cfg, gen_device, max_batch, act)
    if key not in _CASES:
        if cfg.d_model >= 4096:  # keep at most one full-size layer alive
            for k2 in [k for k in _CASES if k[0].d_model >= 4096]:
                del _CASES[k2]
        _CASES[key] = Case(cfg, 0, gen_device, max_batch, act)
    return _CASES[key]


def _check_token(case, x_row_dev, x_np, tau, k, out, t=0, stats=None):
    """Compare token t of a debug forward with the oracle."""
    cfg = case.cfg
    # bit 0: a bounded wait of the persistent kernel timed out
    assert (int(out["status"][0]) & 1) == 0, f"status word {int(out['status'][0])}"
    ref = oracle.forward(case.ol, x_np, tau, k)
    n1 = int(out["n1"][t])
    assert n1 == ref["idx"].size
    assert out["idx"][t, :n1].cpu().numpy().tolist() == ref["idx"].tolist()
    y = out["y"][t].float().cpu().numpy().astype(np.float64)
    if k == 0:
        assert not np.any(y)
        return
    s_abs = out["s_abs"][t].cpu().numpy().astype(np.float64)
    e_s = rel_err(s_abs, np.abs(ref["s_t"]))
    if np.max(np.abs(ref["s_t"])) > 0:
        assert e_s <= 1e-4, f"|s~| error {e_s:.3e}"
    else:
        assert not np.any(s_abs)
    sel = out["sel"][t, :k].cpu().numpy()
    m = check_mask(sel, ref["sel"], ref["s_t"], k, case=f"{cfg.name} top-k k={k}")
    if np.array_equal(sel, ref["sel"]):
        # same channels: the oracle's own exact Stage 2 is the reference
        s_ref, y_ref = ref["s_sp"], ref["y"]
    else:
        # swaps inside the tie band: the exact Stage 2 of the GPU's channels
        s_exact, _ = oracle.dense(x_np, *case.Wnp, act=case.act)
        s_ref = s_exact[sel]
        y_ref = expected_y(sel, ref["sel"], ref["y"], s_exact, case.Wnp[2])
    e_y = rel_err(y, y_ref)
    assert e_y <= _tol(cfg), f"y error {e_y:.3e} (k={k}, tau={tau})"
    if out.get("s_sel") is not None and x_row_dev is not None:
        s_sel = out["s_sel"][t, :k].cpu().numpy().astype(np.float64)
        if out["sel"].shape[0] == 1:
            e_ss = rel_err(s_sel, s_ref)
            assert e_ss <= 1e-4, f"exact s error {e_ss:.3e}"
    if stats is not None:
        stats.append(dict(k=k, n1=n1, band=m["band"], diff=m["diff"], e_y=e_y, e_s=e_s))


# ---------------------------------------------------------------------------
# Prepare
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", [synth.CONFIGS["tiny"], RAGGED], ids=lambda c: c.name)
def test_prepare_quantizer_bit_exact(cfg):
    case = get_case(cfg)
    for m, (q_or, sc_or) in enumerate(((case.ol.q_up, case.ol.sc_up),
                                       (case.ol.q_gate, case.ol.sc_gate))):
        codes, scales = prox.prox_export_proxy(case.L, m)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(codes.cpu().numpy(), q_or)
        np.testing.assert_array_equal(scales.cpu().numpy().view(np.uint32),
                                      sc_or.view(np.uint32))


def test_prepare_quantizer_bit_exact_8b():
    cfg = synth.CONFIGS["8b"]
    W = synth.make_layer(cfg, 0, DEV)
    L = prox.prox_prepare_layer(*W, cfg.group, 1)
    for m in (0, 1):
        codes, scales = prox.prox_export_proxy(L, m)
        q_or, sc_or = oracle.quantize(W[m].float().cpu().numpy(), cfg.group)
        torch.cuda.synchronize()
        assert np.array_equal(codes.cpu().numpy(), q_or)
        assert np.array_equal(scales.cpu().numpy().view(np.uint32), sc_or.view(np.uint32))


def test_relayout_is_exact_copy():
    cfg = RAGGED
    W = synth.make_layer(cfg, 0, DEV)
    L = prox.prox_prepare_layer(*W, cfg.group, 1)
    torch.cuda.synchronize()
    d, f = cfg.d_model, cfg.d_ff
    wb = L.weights.view(torch.bfloat16)
    wug = wb[: 2 * d * f].view(f, 2, d)
    assert torch.equal(wug[:, 0, :], W[0].t())
    assert torch.equal(wug[:, 1, :], W[1].t())
    off = ((2 * d * f * 2 + 255) // 256 * 256) // 2
    wd = wb[off: off + f * d].view(d // 256, f, 256).permute(1, 0, 2).reshape(f, d)
    assert torch.equal(wd, W[2])


# ---------------------------------------------------------------------------
# Forward, small shapes (many inputs, edge cases)
# ---------------------------------------------------------------------------
def test_tiny_f32_parity():
    cfg = synth.CONFIGS["tiny"]
    case = get_case(cfg)
    k = synth.k_for(cfg.d_ff, 0.7)
    X = case.inputs(16)
    stats = []
    for t in range(X.shape[0]):
        xd = X[t:t + 1].to(DEV)
        out = prox.prox_ffn_forward_debug(case.L, xd, case.tau, k)
        torch.cuda.synchronize()
        _check_token(case, xd, X[t].numpy(), case.tau, k, out, stats=stats)
    print("tiny:", stats[:3], "max e_y", max(s["e_y"] for s in stats))


@pytest.mark.parametrize("k_frac", [0.0, 1 / 3000, 0.3, 0.5, 0.999, 1.0])
def test_ragged_bf16_parity_k_sweep(k_frac):
    case = get_case(RAGGED)
    k = int(round(k_frac * RAGGED.d_ff))
    X = case.inputs(3)
    for t in range(X.shape[0]):
        xd = X[t:t + 1].to(DEV)
        out = prox.prox_ffn_forward_debug(case.L, xd, case.tau, k)
        torch.cuda.synchronize()
        _check_token(case, xd, X[t].float().numpy(), case.tau, k, out)


@pytest.mark.parametrize("tau", [0.0, -1.0, float("inf"), 1e30, 2.5])
def test_ragged_threshold_edges(tau):
    case = get_case(RAGGED)
    k = synth.k_for(RAGGED.d_ff, 0.7)
    X = case.inputs(2, "edges")
    for t in range(X.shape[0]):
        xd = X[t:t + 1].to(DEV)
        out = prox.prox_ffn_forward_debug(case.L, xd, tau, k)
        torch.cuda.synchronize()
        _check_token(case, xd, X[t].float().numpy(), tau, k, out)
        if math.isinf(tau):
            assert int(out["n1"][0]) == 0
            assert out["sel"][0, :k].cpu().tolist() == list(range(k))


def test_product_entry_matches_debug_entry_and_is_deterministic():
    case = get_case(RAGGED)
    k = synth.k_for(RAGGED.d_ff, 0.7)
    x = case.inputs(1)[0].to(DEV)
    y1 = prox.prox_ffn_forward(case.L, x, case.tau, k)
    y2 = prox.prox_ffn_forward(case.L, x, case.tau, k)
    yd = prox.prox_ffn_forward_debug(case.L, x[None], case.tau, k)["y"][0]
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(y1.view(torch.int16), yd.view(torch.int16))


def test_argument_errors_with_a_layer():
    case = get_case(RAGGED)
    x = case.inputs(1)[0].to(DEV)
    with pytest.raises(prox.ProxError) as e:
        prox.prox_ffn_forward(case.L, x, float("nan"), 10)
    assert e.value.status == prox.PROX_EINVAL
    with pytest.raises(prox.ProxError):
        prox.prox_ffn_forward(case.L, x, 0.5, RAGGED.d_ff + 1)
    with pytest.raises(prox.ProxError):
        prox.prox_ffn_forward(case.L, x, 0.5, -1)
    with pytest.raises(prox.ProxError):
        prox.prox_ffn_forward_batch(case.L, torch.zeros(2, RAGGED.d_model, dtype=torch.bfloat16,
                                                        device=DEV), 0.5, 10)


# ---------------------------------------------------------------------------
# Dense baseline
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", [synth.CONFIGS["tiny"], RAGGED], ids=lambda c: c.name)
def test_dense_parity(cfg):
    case = get_case(cfg)
    X = case.inputs(2, "dense")
    for t in range(X.shape[0]):
        y = prox.prox_dense_ffn_forward(case.L, X[t:t + 1].to(DEV))
        torch.cuda.synchronize()
        _, y_ref = oracle.dense(X[t].float().numpy(), *case.Wnp)
        assert rel_err(y[0].float().cpu().numpy(), y_ref) <= _tol(cfg)


# ---------------------------------------------------------------------------
# Batch path: per-token masks, union-driven streaming
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("B", [2, 3, 8])
def test_batch_equals_independent_tokens(B):
    case = get_case(RAGGED, max_batch=8)
    k = synth.k_for(RAGGED.d_ff, 0.7)
    X = case.inputs(B, "batch")
    xd = X.to(DEV)
    out = prox.prox_ffn_forward_debug(case.L, xd, case.tau, k)
    torch.cuda.synchronize()
    sels = []
    for t in range(B):
        _check_token(case, xd[t], X[t].float().numpy(), case.tau, k, out, t=t)
        sels.append(set(out["sel"][t, :k].cpu().tolist()))
    nu = int(out["n_union"][0])
    uni = out["union_idx"][:nu].cpu().tolist()
    assert uni == sorted(set.union(*sels))
    # exact s by union position: token t's value where its own mask holds
    # the channel, else 0
    for t in range(B):
        s_exact, _ = oracle.dense(X[t].float().numpy(), *case.Wnp, act=case.act)
        want = np.array([s_exact[j] if j in sels[t] else 0.0 for j in uni])
        got = out["s_sel"][t, :nu].cpu().numpy().astype(np.float64)
        assert not np.any(got[want == 0.0])
        assert rel_err(got, want) <= 1e-4
    yb = prox.prox_ffn_forward_batch(case.L, xd, case.tau, k)
    torch.cuda.synchronize()
    assert torch.equal(yb.view(torch.int16), out["y"].view(torch.int16))


@pytest.mark.parametrize("B", [2, 5, 8])
def test_batch_mfma_form_parity(B):
    """The MFMA form of the batched up/gate step (chosen at prepare time)
    against the oracle, token by token, and against the VALU form."""
    case = Case(RAGGED, 0, "cpu", 8, batch_upgate=prox.PROX_FORM_MFMA)
    valu = get_case(RAGGED, max_batch=8)
    k = synth.k_for(RAGGED.d_ff, 0.7)
    X = case.inputs(B, "mfma")
    xd = X.to(DEV)
    out = prox.prox_ffn_forward_debug(case.L, xd, case.tau, k)
    yv = prox.prox_ffn_forward_batch(valu.L, xd, valu.tau, k)
    yd = prox.prox_dense_ffn_forward(case.L, xd)
    torch.cuda.synchronize()
    for t in range(B):
        _check_token(case, xd[t], X[t].float().numpy(), case.tau, k, out, t=t)
        _, y_ref = oracle.dense(X[t].float().numpy(), *case.Wnp)
        assert rel_err(yd[t].float().cpu().numpy(), y_ref) <= _tol(RAGGED)
    assert rel_err(yv.float().cpu().numpy(), out["y"].float().cpu().numpy()) <= _tol(RAGGED)


@pytest.mark.parametrize("B", [3, 8])
def test_batch_stage1_mfma_matches_valu(B):
    """Stage 1 of 3..8 tokens runs on the matrix cores over the 8-row code
    words written at prepare time: its |s~| against the oracle (through the
    mask and output checks) and against the VALU Stage 1 of a layer prepared
    with batch_stage1 = PROX_FORM_VALU (same codes, other summation order)."""
    valu = Case(RAGGED, 0, "cpu", 8, batch_stage1=prox.PROX_FORM_VALU)
    mf = get_case(RAGGED, max_batch=8)
    k = synth.k_for(RAGGED.d_ff, 0.7)
    X = mf.inputs(B, "stage1mfma")
    xd = X.to(DEV)
    out_m = prox.prox_ffn_forward_debug(mf.L, xd, mf.tau, k)
    out_v = prox.prox_ffn_forward_debug(valu.L, xd, valu.tau, k)
    torch.cuda.synchronize()
    for t in range(B):
        _check_token(mf, xd[t], X[t].float().numpy(), mf.tau, k, out_m, t=t)
        sm = out_m["s_abs"][t].cpu().numpy().astype(np.float64)
        sv = out_v["s_abs"][t].cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(sm))
        assert rel_err(sm, sv) <= 1e-5, f"token {t}: {rel_err(sm, sv):.3e}"


def test_batch_split_tie():
    """A zero token has |s~| = 0 everywhere: its mask is the k lowest
    channels (ties to the lower index), the product path (mask words only)
    takes its tie branch and must agree with the list path."""
    case = get_case(RAGGED, max_batch=8)
    k = synth.k_for(RAGGED.d_ff, 0.7)
    X = case.inputs(3, "tie")
    X[1].zero_()
    xd = X.to(DEV)
    out = prox.prox_ffn_forward_debug(case.L, xd, case.tau, k)
    torch.cuda.synchronize()
    assert out["sel"][1, :k].cpu().tolist() == list(range(k))
    assert not torch.any(out["y"][1].float())
    for t in (0, 2):
        _check_token(case, xd[t], X[t].float().numpy(), case.tau, k, out, t=t)
    sels = [set(out["sel"][t, :k].cpu().tolist()) for t in range(3)]
    nu = int(out["n_union"][0])
    assert out["union_idx"][:nu].cpu().tolist() == sorted(set.union(*sels))
    yb = prox.prox_ffn_forward_batch(case.L, xd, case.tau, k)
    torch.cuda.synchronize()
    assert torch.equal(yb.view(torch.int16), out["y"].view(torch.int16))


# ---------------------------------------------------------------------------
# Stack: RMSNorm + FFN + residual over several layers
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("k_frac", [0.3, -1])
def test_stack_parity(k_frac):
    cfg = synth.Config("stacksmall", 1024, 2816, 128, "bf16", "student_t", 0.5, 32, (0.7,))
    nl = 4
    layers, olayers, taus = [], [], []
    ws = None
    for l in range(nl):
        W = synth.make_layer(cfg, l, "cpu")
        L = prox.prox_prepare_layer(*[w.to(DEV) for w in W], cfg.group, 1, workspace=ws)
        ws = L.workspace
        layers.append(L)
        olayers.append(oracle.Layer(*[w.float().numpy() for w in W], cfg.group))
        taus.append(synth.layer_tau(cfg, l, "cpu") * 0.5)
    k = synth.k_for(cfg.d_ff, 0.7) if k_frac > 0 else cfg.d_ff
    R0 = synth.make_inputs(cfg, 3, "stack", 0, "cpu").float()
    for t in range(R0.shape[0]):
        r = R0[t].clone().to(DEV)
        prox.prox_stack_forward(layers, taus, k if k_frac > 0 else -1, r)
        torch.cuda.synchronize()
        r_ref, _ = oracle.stack_forward(olayers, taus, k, R0[t].numpy())
        assert rel_err(r.cpu().numpy(), r_ref) <= 2e-2


@pytest.mark.parametrize("mode", ["topk", "threshold"])
def test_stack_fused_norm_matches_separate_launches(mode):
    """For one token the stack runs one launch per layer: the persistent
    kernel forms x = RMSNorm(r) itself.  Layer by layer, the residual must
    carry the same bits as the separate RMSNorm kernel + forward + add."""
    cfg = synth.Config("stacksmall", 1024, 2816, 128, "bf16", "student_t", 0.5, 32, (0.7,))
    nl = 3
    layers, taus, tss = [], [], []
    ws = None
    for l in range(nl):
        W = synth.make_layer(cfg, l, "cpu")
        L = prox.prox_prepare_layer(*[w.to(DEV) for w in W], cfg.group, 1, workspace=ws)
        ws = L.workspace
        layers.append(L)
        taus.append(synth.layer_tau(cfg, l, "cpu") * 0.5)
    k = synth.k_for(cfg.d_ff, 0.7)
    R0 = synth.make_inputs(cfg, 2, "stacknorm", 0, "cpu").float().to(DEV)
    if mode == "threshold":
        # tau_s per layer: the 0.7 quantile of |s~| on the first token's inputs
        r = R0[0].clone()
        for l in range(nl):
            x = prox.prox_rmsnorm(layers[l], r)
            out = prox.prox_ffn_forward_debug(layers[l], x[None], taus[l], k)
            tss.append(float(torch.quantile(out["s_abs"][0].float(), 0.7)))
            r += out["y"][0].float()
    for t in range(R0.shape[0]):
        ra = R0[t].clone()
        if mode == "topk":
            prox.prox_stack_forward(layers, taus, k, ra)
        else:
            prox.prox_stack_forward_ts(layers, taus, tss, ra)
        rb = R0[t].clone()
        for l in range(nl):
            x = prox.prox_rmsnorm(layers[l], rb)
            if mode == "topk":
                y = prox.prox_ffn_forward(layers[l], x, taus[l], k)
            else:
                y = prox.prox_ffn_forward_ts(layers[l], x, taus[l], tss[l])
            rb += y.float()
        torch.cuda.synchronize()
        assert torch.equal(ra, rb), f"token {t}: max diff {float((ra - rb).abs().max())}"


# ---------------------------------------------------------------------------
# Full-size shapes (8B, 14B, 70B), in the launch configuration bench.py times
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["8b", "14b", "70b"])
def test_full_size_parity(name):
    cfg = synth.CONFIGS[name]
    case = get_case(cfg, DEV, 8 if name == "70b" else 1)
    X = synth.make_inputs(cfg, 2, "test", 0, DEV)
    stats = []
    for sp in cfg.sparsities:
        k = synth.k_for(cfg.d_ff, sp)
        for t in range(X.shape[0]):
            xd = X[t:t + 1]
            out = prox.prox_ffn_forward_debug(case.L, xd, case.tau, k)
            torch.cuda.synchronize()
            _check_token(case, xd, X[t].float().cpu().numpy(), case.tau, k, out, stats=stats)
    print(name, stats)
    # the dense baseline of the same shape
    y = prox.prox_dense_ffn_forward(case.L, X[:1])
    torch.cuda.synchronize()
    _, y_ref = oracle.dense(X[0].float().cpu().numpy(), *case.Wnp)
    assert rel_err(y[0].float().cpu().numpy(), y_ref) <= 2e-2


@pytest.mark.parametrize("B", [2, 4, 8])
def test_70b_batch_parity(B):
    cfg = synth.CONFIGS["70b"]
    case = get_case(cfg, DEV, 8)
    k = synth.k_for(cfg.d_ff, 0.7)
    X = synth.make_inputs(cfg, B, "batch", 0, DEV)
    out = prox.prox_ffn_forward_debug(case.L, X, case.tau, k)
    torch.cuda.synchronize()
    for t in range(B):
        _check_token(case, X[t], X[t].float().cpu().numpy(), case.tau, k, out, t=t)


# ---------------------------------------------------------------------------
# The multi-kernel path (path = PROX_PATH_MULTI at prepare time) against the oracle
# and against the persistent single-launch path of the same layer
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["ragged", "8b"])
def test_multi_kernel_path_parity(name):
    cfg = RAGGED if name == "ragged" else synth.CONFIGS["8b"]
    gen = "cpu" if name == "ragged" else DEV
    fused = get_case(cfg, gen)
    multi = Case(cfg, 0, gen, 1, path=prox.PROX_PATH_MULTI)
    k = synth.k_for(cfg.d_ff, 0.7)
    X = synth.make_inputs(cfg, 2, "paths", 0, gen)
    for t in range(X.shape[0]):
        xd = X[t:t + 1].to(DEV)
        out = prox.prox_ffn_forward_debug(multi.L, xd, multi.tau, k)
        yf = prox.prox_ffn_forward(fused.L, xd[0], fused.tau, k)
        torch.cuda.synchronize()
        _check_token(multi, xd, X[t].float().cpu().numpy(), multi.tau, k, out)
        e = rel_err(yf.float().cpu().numpy(), out["y"][0].float().cpu().numpy())
        assert e <= _tol(cfg), f"paths differ by {e:.3e}"


def test_fused_path_repeated_launches_are_identical():
    """The persistent kernel alternates its flags between two halves of the
    sync words (each launch clears the half it does not use, the last ticket
    draw flips the parity): many back-to-back launches on one stream, an odd
    and an even number, give the same bits."""
    case = get_case(RAGGED)
    k = synth.k_for(RAGGED.d_ff, 0.7)
    x = case.inputs(1, "repeat")[0].to(DEV)
    ys = [prox.prox_ffn_forward(case.L, x, case.tau, k) for _ in range(50)]
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(y.view(torch.int16), ys[0].view(torch.int16))


def test_fused_instances_alternate_halves_on_one_workspace():
    """The persistent kernel keeps its per-launch sync words in two halves,
    one per launch parity (the last ticket draw of a launch flips it), and
    each launch clears the half it does not use.  Its top-k and threshold-mask
    instances interleaved on one layer, in an irregular order and across a
    status read, must give the bits of the same calls on a freshly prepared
    layer (whose sync words are all zero, parity 0)."""
    case = get_case(RAGGED)
    W = [w.to(DEV) for w in synth.make_layer(RAGGED, 0, "cpu")]
    L = prox.prox_prepare_layer(*W, RAGGED.group, 1)
    Xc = synth.make_inputs(RAGGED, 4, "halves", 0, "cpu")
    X = Xc.to(DEV)
    k = synth.k_for(RAGGED.d_ff, 0.7)
    tau = case.tau
    tau_s = float(np.quantile(np.abs(oracle.forward(case.ol, Xc[0].float().numpy(), tau, 1)["s_t"]),
                              0.7))
    order = ["topk", "ts", "ts", "topk", "status", "topk", "ts", "topk", "topk", "ts"]
    for i, op in enumerate(order):
        if op == "status":
            st = prox.prox_read_status(L)
            torch.cuda.synchronize()
            assert int(st[0]) == 0
            continue
        x = X[i % X.shape[0]]
        fresh = prox.prox_prepare_layer(*W, RAGGED.group, 1)
        if op == "topk":
            y = prox.prox_ffn_forward(L, x, tau, k)
            y0 = prox.prox_ffn_forward(fresh, x, tau, k)
        else:
            y = prox.prox_ffn_forward_ts(L, x, tau, tau_s)
            y0 = prox.prox_ffn_forward_ts(fresh, x, tau, tau_s)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y0.view(torch.int16)), f"call {i} ({op})"
        del fresh


@pytest.mark.parametrize("name", ["ragged", "8b"])
def test_fused_cut_guess_changes_no_bits(name):
    """A layer keeps the last call's b* as a guess of the next cut, only to
    start Stage 2 early.  Alternating k moves the cut far from the guess in
    both directions (guess above the cut: a second pass; below: extra
    channels computed); every call must give the bits of the same call on a
    freshly prepared layer (no guess)."""
    cfg = RAGGED if name == "ragged" else synth.CONFIGS["8b"]
    gen = "cpu" if name == "ragged" else DEV
    case = get_case(cfg, gen)
    W = synth.make_layer(cfg, 0, gen)
    Wd = [w.to(DEV) for w in W]
    X = synth.make_inputs(cfg, 6, "guess", 0, gen).to(DEV)
    ks = [synth.k_for(cfg.d_ff, sp) for sp in (0.7, 0.3, 0.9, 0.5, 0.7, 0.7)]
    for t, k in enumerate(ks):
        y = prox.prox_ffn_forward(case.L, X[t], case.tau, k)
        fresh = prox.prox_prepare_layer(*Wd, cfg.group, 1)
        y0 = prox.prox_ffn_forward(fresh, X[t], case.tau, k)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y0.view(torch.int16)), f"call {t}, k={k}"
        del fresh


# ---------------------------------------------------------------------------
# Stage 2 threshold mask (|s~| >= tau_s) instead of top-k
# ---------------------------------------------------------------------------
def _check_ts(case, xd, x_np, tau_x, tau_s, out, stats=None):
    cfg = case.cfg
    assert int(out["status"][0]) == 0
    ref = oracle.forward_ts(case.ol, x_np, tau_x, tau_s)
    n1 = int(out["n1"][0])
    assert out["idx"][0, :n1].cpu().numpy().tolist() == ref["idx"].tolist()
    if np.max(np.abs(ref["s_t"])) > 0:
        assert rel_err(out["s_abs"][0].cpu().numpy(), np.abs(ref["s_t"])) <= 1e-4
    m = int(out["n_sel"][0])
    sel = out["sel"][0, :m].cpu().numpy()
    mk = check_threshold_mask(sel, ref["sel"], ref["s_t"], tau_s, case=f"{cfg.name} tau_s")
    y = out["y"][0].float().cpu().numpy().astype(np.float64)
    if m == 0:
        assert ref["sel"].size == 0 and not np.any(y)
        return
    s_sel = out["s_sel"][0, :m].cpu().numpy().astype(np.float64)
    if np.array_equal(sel, ref["sel"]):
        s_ref, y_ref = ref["s_sp"], ref["y"]
    else:
        s_exact, _ = oracle.dense(x_np, *case.Wnp, act=case.act)
        s_ref = s_exact[sel]
        y_ref = expected_y(sel, ref["sel"], ref["y"], s_exact, case.Wnp[2])
    assert rel_err(s_sel, s_ref) <= 1e-4
    e_y = rel_err(y, y_ref)
    assert e_y <= _tol(cfg), f"y error {e_y:.3e} (tau_s={tau_s})"
    if stats is not None:
        stats.append(dict(m=m, band=mk["band"], diff=mk["diff"], e_y=e_y))


@pytest.mark.parametrize("name", ["tiny", "ragged", "8b"])
def test_threshold_mask_parity(name):
    cfg = RAGGED if name == "ragged" else synth.CONFIGS[name]
    gen = DEV if name == "8b" else "cpu"
    case = get_case(cfg, gen)
    X = synth.make_inputs(cfg, 3, "ts", 0, gen)
    stats = []
    for t in range(X.shape[0]):
        x_np = X[t].float().cpu().numpy()
        s_t = oracle.forward(case.ol, x_np, case.tau, 1)["s_t"]
        for q in (0.5, 0.7, 0.9):
            tau_s = float(np.quantile(np.abs(s_t), q))
            xd = X[t:t + 1].to(DEV)
            out = prox.prox_ffn_forward_ts_debug(case.L, xd, case.tau, tau_s)
            torch.cuda.synchronize()
            _check_ts(case, xd, x_np, case.tau, tau_s, out, stats)
    print(name, stats)
    # the product entry gives the debug entry's bits
    xd = X[:1].to(DEV)
    tau_s = float(np.quantile(np.abs(oracle.forward(case.ol, X[0].float().cpu().numpy(),
                                                    case.tau, 1)["s_t"]), 0.7))
    y1 = prox.prox_ffn_forward_ts(case.L, xd[0], case.tau, tau_s)
    yd = prox.prox_ffn_forward_ts_debug(case.L, xd, case.tau, tau_s)["y"][0]
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), yd.view(torch.int16))


@pytest.mark.parametrize("tau_s", [0.0, float("inf"), 1e30])
def test_threshold_mask_edges(tau_s):
    case = get_case(RAGGED)
    X = case.inputs(2, "ts-edges")
    for t in range(X.shape[0]):
        xd = X[t:t + 1].to(DEV)
        out = prox.prox_ffn_forward_ts_debug(case.L, xd, case.tau, tau_s)
        torch.cuda.synchronize()
        _check_ts(case, xd, X[t].float().numpy(), case.tau, tau_s, out)
        if tau_s == 0.0:
            assert int(out["n_sel"][0]) == RAGGED.d_ff


def test_threshold_mask_rejects_nan_and_multi_path():
    case = get_case(RAGGED)
    x = case.inputs(1)[0].to(DEV)
    with pytest.raises(prox.ProxError) as e:
        prox.prox_ffn_forward_ts(case.L, x, case.tau, float("nan"))
    assert e.value.status == prox.PROX_EINVAL
    multi = Case(RAGGED, 0, "cpu", 1, path=prox.PROX_PATH_MULTI)
    with pytest.raises(prox.ProxError) as e:
        prox.prox_ffn_forward_ts(multi.L, x, case.tau, 0.1)
    assert e.value.status == prox.PROX_EUNSUPPORTED


# ---------------------------------------------------------------------------
# Threshold-mask stack and its sequential calibration (App. A.7, Alg. 1)
# ---------------------------------------------------------------------------
STACK_SMALL = synth.Config("stacksmall", 1024, 2816, 128, "bf16", "student_t", 0.5, 32, (0.7,))


def _small_stack(nl):
    layers, olayers = [], []
    ws = None
    for l in range(nl):
        W = synth.make_layer(STACK_SMALL, l, "cpu")
        L = prox.prox_prepare_layer(*[w.to(DEV) for w in W], STACK_SMALL.group, 8, workspace=ws)
        ws = L.workspace
        layers.append(L)
        olayers.append(oracle.Layer(*[w.float().numpy() for w in W], STACK_SMALL.group))
    return layers, olayers


def test_sequential_calibration_matches_oracle():
    """Both thresholds of every layer, teacher-forced: given the inputs the GPU
    calibration collected for a layer, the oracle's quantiles of |x| and of its
    own |s~| give the same tau_x (bit-equal) and tau_s (float32 vs double
    summation only)."""
    from free_sparse_swiglu_amd import calibrate, costmodel
    s1, s2 = costmodel.allocate(0.7)  # App. A.4: s1 = 0.7, s2 = 0.767
    layers, olayers = _small_stack(3)
    R0 = synth.make_inputs(STACK_SMALL, 24, "calib", 0, "cpu").float()
    tx, ts, X = calibrate.sequential_thresholds_ts(layers, R0.to(DEV), s1, s2,
                                                   return_inputs=True)
    torch.cuda.synchronize()
    for l, L in enumerate(olayers):
        Xl = X[l].float().cpu().numpy()
        assert oracle.lower_quantile(np.abs(Xl), s1) == tx[l]
        S = []
        for x in Xl:
            _, _, s_t = oracle.proxy(x, oracle.input_mask(x, tx[l]), L.Wt_up, L.Wt_gate)
            S.append(np.abs(s_t).astype(np.float32))
        ts_or = oracle.lower_quantile(np.concatenate(S), s2)
        assert abs(ts[l] - ts_or) <= 1e-3 * ts_or, (l, ts[l], ts_or)


def test_stack_ts_parity_and_runtime_sparsity():
    from free_sparse_swiglu_amd import calibrate, costmodel
    s1, s2 = costmodel.allocate(0.7)
    layers, olayers = _small_stack(4)
    R0 = synth.make_inputs(STACK_SMALL, 16, "calib", 0, "cpu").float()
    tx, ts, _ = oracle.calibrate_sequential(olayers, R0.numpy(), s1, s2)
    T = synth.make_inputs(STACK_SMALL, 3, "stack", 0, "cpu").float()
    n1s, nss = 0, 0
    for t in range(T.shape[0]):
        r = T[t].clone().to(DEV)
        prox.prox_stack_forward_ts(layers, tx, ts, r)
        torch.cuda.synchronize()
        r_ref, outs = oracle.stack_forward_ts(olayers, tx, ts, T[t].numpy())
        assert rel_err(r.cpu().numpy(), r_ref) <= 2e-2
        n1s += sum(o["idx"].size for o in outs)
        nss += sum(o["sel"].size for o in outs)
    rs = calibrate.runtime_sparsity(layers, tx, ts, T.to(DEV))
    e_or = costmodel.effective_sparsity(1 - n1s / (3 * 4 * STACK_SMALL.d_model),
                                        1 - nss / (3 * 4 * STACK_SMALL.d_ff))
    assert abs(rs["e"] - e_or) <= 0.01, (rs, e_or)



# ---------------------------------------------------------------------------
# GeGLU (tanh-form GELU gate) instead of SwiGLU
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["tiny", "ragged", "8b"])
def test_geglu_parity(name):
    cfg = RAGGED if name == "ragged" else synth.CONFIGS[name]
    gen = DEV if name == "8b" else "cpu"
    case = get_case(cfg, gen, 1, act=prox.PROX_ACT_GELU_TANH)
    k = synth.k_for(cfg.d_ff, 0.7)
    X = synth.make_inputs(cfg, 3, "geglu", 0, gen)
    for t in range(X.shape[0]):
        xd = X[t:t + 1].to(DEV)
        x_np = X[t].float().cpu().numpy()
        out = prox.prox_ffn_forward_debug(case.L, xd, case.tau, k)
        torch.cuda.synchronize()
        _check_token(case, xd, x_np, case.tau, k, out)
        s_t = oracle.forward(case.ol, x_np, case.tau, 1)["s_t"]
        tau_s = float(np.quantile(np.abs(s_t), 0.7))
        out = prox.prox_ffn_forward_ts_debug(case.L, xd, case.tau, tau_s)
        torch.cuda.synchronize()
        _check_ts(case, xd, x_np, case.tau, tau_s, out)
    y = prox.prox_dense_ffn_forward(case.L, X[:1].to(DEV))
    torch.cuda.synchronize()
    _, y_ref = oracle.dense(X[0].float().cpu().numpy(), *case.Wnp, act=case.act)
    assert rel_err(y[0].float().cpu().numpy(), y_ref) <= _tol(cfg)


# ---------------------------------------------------------------------------
# The alpha measurement pair: Stage 1 alone and the input-sparse bf16 GEMV
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["ragged", "8b"])
def test_sparse_gemv_parity(name):
    """u, g = x_S W_up, x_S W_gate over |x_i| >= tau: the oracle's proxy step
    with the original weights as proxy weights computes exactly that."""
    cfg = RAGGED if name == "ragged" else synth.CONFIGS[name]
    gen = DEV if name == "8b" else "cpu"
    case = get_case(cfg, gen)
    Wu, Wg = case.Wg_dev[0], case.Wg_dev[1]
    Wu64 = case.Wnp[0].astype(np.float64)
    Wg64 = case.Wnp[1].astype(np.float64)
    ws = prox.prox_sparse_gemv_workspace(cfg.d_model, cfg.d_ff)
    X = synth.make_inputs(cfg, 2, "sgemv", 0, gen)
    for t in range(X.shape[0]):
        x_np = X[t].float().cpu().numpy()
        for tau in (case.tau, 0.0, float("inf")):
            for _ in range(2):  # the workspace is left ready for the next call
                u, g = prox.prox_sparse_gemv(Wu, Wg, X[t].to(DEV), tau, ws)
                torch.cuda.synchronize()
            idx = oracle.input_mask(x_np, tau)
            u_r, g_r, _ = oracle.proxy(x_np, idx, Wu64, Wg64)
            if idx.size == 0:
                assert not torch.any(u) and not torch.any(g)
                continue
            assert rel_err(u.cpu().numpy(), u_r) <= 1e-4
            assert rel_err(g.cpu().numpy(), g_r) <= 1e-4


def test_stage1_entry_matches_oracle():
    case = get_case(RAGGED)
    X = case.inputs(2, "stage1")
    out = torch.empty(RAGGED.d_ff, device=DEV)
    for t in range(X.shape[0]):
        prox.prox_stage1(case.L, X[t].to(DEV), case.tau, out)
        torch.cuda.synchronize()
        ref = oracle.forward(case.ol, X[t].float().numpy(), case.tau, 1)["s_t"]
        assert rel_err(out.cpu().numpy(), np.abs(ref)) <= 1e-4


# ---------------------------------------------------------------------------
# Matrix-core Stage 1 of several tokens at three group sizes (128 has its own
# instance with fixed group ends) and a d_model whose last 1024-row chunk is
# partial (1536 = 1024 + 512)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("G", [64, 128, 256])
@pytest.mark.parametrize("B", [3, 8])
def test_batch_stage1_mfma_group_sizes(G, B):
    cfg = synth.Config(f"mfma1536g{G}", 1536, 3000, G, "bf16", "student_t", 0.5, 32, (0.7,))
    mf = Case(cfg, 0, "cpu", 8, batch_stage1=prox.PROX_FORM_MFMA)
    valu = Case(cfg, 0, "cpu", 8, batch_stage1=prox.PROX_FORM_VALU)
    k = synth.k_for(cfg.d_ff, 0.7)
    X = mf.inputs(B, "stage1g")
    xd = X.to(DEV)
    out_m = prox.prox_ffn_forward_debug(mf.L, xd, mf.tau, k)
    out_v = prox.prox_ffn_forward_debug(valu.L, xd, valu.tau, k)
    torch.cuda.synchronize()
    for t in range(B):
        _check_token(mf, xd[t], X[t].float().numpy(), mf.tau, k, out_m, t=t)
        _check_token(valu, xd[t], X[t].float().numpy(), valu.tau, k, out_v, t=t)
        sm = out_m["s_abs"][t].cpu().numpy().astype(np.float64)
        sv = out_v["s_abs"][t].cpu().numpy().astype(np.float64)
        assert rel_err(sm, sv) <= 1e-5, f"token {t}: {rel_err(sm, sv):.3e}"


# ---------------------------------------------------------------------------
# Error surface of the persistent kernel: a bounded wait that gives up is
# reported through the workspace status, and the next call is correct
# ---------------------------------------------------------------------------
def test_status_reports_timed_out_wait_and_recovers():
    """A poll limit of 0 makes the persistent kernel's first unsatisfied wait
    give up at once (every wait is bounded, so the kernel still exits): the
    status word has bit 0 set, prox_read_status clears it and resets the
    synchronisation block, and with the default limit back the same layer
    gives the oracle's result again."""
    case = Case(RAGGED, 0, "cpu", 1)
    k = synth.k_for(RAGGED.d_ff, 0.7)
    X = case.inputs(2, "status")
    st0 = prox.prox_read_status(case.L)
    torch.cuda.synchronize()
    assert int(st0[0]) == 0
    prox.prox_set_wait_limit(case.L, 0)
    prox.prox_ffn_forward(case.L, X[0].to(DEV), case.tau, k)
    st = prox.prox_read_status(case.L)
    torch.cuda.synchronize()
    assert int(st[0]) & 1, f"status {int(st[0])}: no timed-out wait reported"
    prox.prox_set_wait_limit(case.L, 1 << 22)
    st2 = prox.prox_read_status(case.L)
    torch.cuda.synchronize()
    assert int(st2[0]) == 0, "the status read did not clear the word"
    for t in range(X.shape[0]):
        xd = X[t:t + 1].to(DEV)
        out = prox.prox_ffn_forward_debug(case.L, xd, case.tau, k)
        torch.cuda.synchronize()
        _check_token(case, xd, X[t].float().numpy(), case.tau, k, out)
    y = prox.prox_ffn_forward(case.L, X[0].to(DEV), case.tau, k)
    st3 = prox.prox_read_status(case.L)
    yd = prox.prox_ffn_forward_debug(case.L, X[:1].to(DEV), case.tau, k)["y"][0]
    torch.cuda.synchronize()
    assert int(st3[0]) & 1 == 0
    assert torch.equal(y.view(torch.int16), yd.view(torch.int16))


def test_layers_of_different_shapes_share_a_workspace():
    """Two layers of different shapes and max_batch on one workspace (the
    synchronisation block sits at a fixed place): alternating calls give the
    bits of the same calls on layers with workspaces of their own."""
    cfg_b = synth.Config("ragged2", 1536, 2000, 64, "bf16", "student_t", 0.5, 32, (0.7,))
    Wa = [w.to(DEV) for w in synth.make_layer(RAGGED, 0, "cpu")]
    Wb = [w.to(DEV) for w in synth.make_layer(cfg_b, 0, "cpu")]
    La = prox.prox_prepare_layer(*Wa, RAGGED.group, 8)
    Lb = prox.prox_prepare_layer(*Wb, cfg_b.group, 1, workspace=La.workspace)
    assert Lb.workspace.data_ptr() == La.workspace.data_ptr()
    Ra = prox.prox_prepare_layer(*Wa, RAGGED.group, 8)
    Rb = prox.prox_prepare_layer(*Wb, cfg_b.group, 1)
    # a multi-kernel layer on the same workspace: its kernels write the s and
    # partial-sum buffers that the persistent kernel marks and polls
    Lc = prox.prox_prepare_layer(*Wb, cfg_b.group, 1, workspace=La.workspace,
                                 path=prox.PROX_PATH_MULTI)
    Rc = prox.prox_prepare_layer(*Wb, cfg_b.group, 1, path=prox.PROX_PATH_MULTI)
    xa = synth.make_inputs(RAGGED, 3, "share", 0, "cpu").to(DEV)
    xb = synth.make_inputs(cfg_b, 3, "share", 0, "cpu").to(DEV)
    ka, kb = synth.k_for(RAGGED.d_ff, 0.7), synth.k_for(cfg_b.d_ff, 0.7)
    for t in range(3):
        ya = prox.prox_ffn_forward(La, xa[t], 0.5, ka)
        yab = prox.prox_ffn_forward_batch(La, xa, 0.5, ka)
        yb = prox.prox_ffn_forward(Lb, xb[t], 0.5, kb)
        yc = prox.prox_ffn_forward(Lc, xb[t], 0.5, kb)
        yd = prox.prox_dense_ffn_forward(La, xa[t])
        ya2 = prox.prox_ffn_forward(La, xa[t], 0.5, ka)
        ra = prox.prox_ffn_forward(Ra, xa[t], 0.5, ka)
        rab = prox.prox_ffn_forward_batch(Ra, xa, 0.5, ka)
        rb = prox.prox_ffn_forward(Rb, xb[t], 0.5, kb)
        rc = prox.prox_ffn_forward(Rc, xb[t], 0.5, kb)
        rd = prox.prox_dense_ffn_forward(Ra, xa[t])
        torch.cuda.synchronize()
        assert torch.equal(ya.view(torch.int16), ra.view(torch.int16))
        assert torch.equal(ya2.view(torch.int16), ra.view(torch.int16))
        assert torch.equal(yab.view(torch.int16), rab.view(torch.int16))
        assert torch.equal(yb.view(torch.int16), rb.view(torch.int16))
        assert torch.equal(yc.view(torch.int16), rc.view(torch.int16))
        assert torch.equal(yd.view(torch.int16), rd.view(torch.int16))
    st = prox.prox_read_status(La)
    torch.cuda.synchronize()
    assert int(st[0]) & 1 == 0
