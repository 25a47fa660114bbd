"""The no-allocation entry point, prox_ffn_forward_noalloc, through the C ABI:
its output must be the bits of prox_ffn_forward (the same kernels, with the
per-call scratch in the library's static device array instead of the layer's
workspace), on two calls in a row for each of two layers, the second layer
smaller than the first; a layer whose scratch would not fit is rejected
before anything is launched."""
from __future__ import annotations

import ctypes

import pytest
import torch

from free_sparse_swiglu_amd import prox, synth

pytestmark = pytest.mark.gpu

DEV = "cuda"
RAGGED = synth.Config("ragged", 1024, 3000, 128, "bf16", "student_t", 0.5, 32, (0.7,))


def _noalloc(L, x, tau, k, y):
    lib = prox.load_library()
    return lib.prox_ffn_forward_noalloc(L.handle, prox._ptr(x), float(tau), int(k), prox._ptr(y),
                                        prox._stream())


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_matches_product_entry(order):
    cfgs = [synth.CONFIGS["8b"], RAGGED, synth.CONFIGS["tiny"]]
    for cfg in cfgs:
        gen = DEV if cfg.d_model >= 4096 else "cpu"
        W = [w.to(DEV) for w in synth.make_layer(cfg, 0, gen)]
        L = prox.prox_prepare_layer(*W, cfg.group, 1)
        tau = synth.layer_tau(cfg, 0, gen)
        k = synth.k_for(cfg.d_ff, 0.7)
        X = synth.make_inputs(cfg, 2, "noalloc", 0, gen).to(DEV)
        for t in range(X.shape[0]):  # two calls in a row on this layer
            y_ref = prox.prox_ffn_forward(L, X[t], tau, k)
            y = torch.full_like(y_ref, float("nan"))
            st = _noalloc(L, X[t], tau, k, y)
            assert st == prox.PROX_OK, prox.prox_last_error()
            torch.cuda.synchronize()
            bits = torch.int16 if y.dtype == torch.bfloat16 else torch.int32
            assert torch.equal(y.view(bits), y_ref.view(bits)), f"{cfg.name} call {t}"
        # k = 0 gives y = 0 on this path too
        y = torch.full_like(X[0], 1.0)
        assert _noalloc(L, X[0], tau, 0, y) == prox.PROX_OK
        torch.cuda.synchronize()
        assert not torch.any(y.float())
        del L, W


def test_noalloc_rejects_a_layer_too_large_for_the_scratch():
    d_model, d_ff, G = 16384, 32768, 256  # batch-1 scratch above 8 MiB
    w = torch.zeros(d_model, d_ff, dtype=torch.bfloat16, device=DEV)
    wd = torch.zeros(d_ff, d_model, dtype=torch.bfloat16, device=DEV)
    L = prox.prox_prepare_layer(w, w, wd, G, 1)
    x = torch.zeros(d_model, dtype=torch.bfloat16, device=DEV)
    y = torch.zeros_like(x)
    assert _noalloc(L, x, 0.5, 10, y) == prox.PROX_EUNSUPPORTED
    assert "scratch" in prox.prox_last_error()
    torch.cuda.synchronize()
