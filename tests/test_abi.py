"""The C ABI library without a GPU: it loads, exports every function
include/prox.h declares, and rejects bad arguments on the host before any
HIP call (no kernel is launched by these tests)."""
import ctypes
import math

import pytest

from free_sparse_swiglu_amd import prox


@pytest.fixture(scope="module")
def lib():
    return prox.load_library()


def test_header_declares_the_boundary():
    names = prox.header_symbols()
    for want in ("prox_query_sizes", "prox_prepare_layer", "prox_ffn_forward",
                 "prox_ffn_forward_batch", "prox_ffn_forward_debug",
                 "prox_dense_ffn_forward", "prox_stack_forward", "prox_export_proxy",
                 "prox_destroy_layer", "prox_last_error"):
        assert want in names


def test_library_exports_every_declared_symbol(lib):
    for name in prox.header_symbols():
        assert hasattr(lib, name), f"{name} declared in prox.h but not exported"


def _q(d_model, d_ff, G, dtype, mb=1):
    sh = prox.prox_shape(d_model, d_ff, G, dtype, mb)
    w, p, ws = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    st = prox.load_library().prox_query_sizes(ctypes.byref(sh), ctypes.byref(w),
                                              ctypes.byref(p), ctypes.byref(ws))
    return st, w.value, p.value, ws.value


def test_query_sizes_values(lib):
    st, w, p, ws = _q(4096, 14336, 128, prox.PROX_BF16)
    assert st == prox.PROX_OK
    assert w >= 3 * 4096 * 14336 * 2
    # packed codes (one byte per input row per column pair, up+gate) + fp32 scales
    assert p >= 4096 * 14336 + 2 * (4096 // 128) * 14336 * 4
    assert ws > 0
    st, w1, p1, ws1 = _q(256, 688, 64, prox.PROX_F32)
    assert st == prox.PROX_OK and w1 >= 3 * 256 * 688 * 4
    # ragged last proxy tile: 688 = 2 * 256 + 176 columns
    assert p1 >= 3 * 256 * 256


@pytest.mark.parametrize("args,status", [
    ((4096, 14336, 100, prox.PROX_BF16), prox.PROX_EINVAL),       # d_model % G
    ((4096, 14336, 32, prox.PROX_BF16), prox.PROX_EUNSUPPORTED),  # G not 64/128/256
    ((0, 14336, 128, prox.PROX_BF16), prox.PROX_EINVAL),
    ((4096, 0, 128, prox.PROX_BF16), prox.PROX_EINVAL),
    ((4096, 14336, 128, 7), prox.PROX_EINVAL),                    # dtype
    ((256 * 3, 1000, 64, prox.PROX_BF16), prox.PROX_EUNSUPPORTED), # d_model % 512 (bf16)
    ((4096, 40000, 128, prox.PROX_BF16), prox.PROX_EUNSUPPORTED), # d_ff above 32768
])
def test_query_sizes_rejects(lib, args, status):
    assert _q(*args)[0] == status
    assert prox.prox_last_error() != ""


def test_query_sizes_activation(lib):
    for act in (prox.PROX_ACT_SILU, prox.PROX_ACT_GELU_TANH):
        sh = prox.prox_shape(1024, 2816, 128, prox.PROX_BF16, 1, act)
        w, p, ws = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
        assert lib.prox_query_sizes(ctypes.byref(sh), ctypes.byref(w), ctypes.byref(p),
                                    ctypes.byref(ws)) == prox.PROX_OK
    sh = prox.prox_shape(1024, 2816, 128, prox.PROX_BF16, 1, 2)
    w, p, ws = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.prox_query_sizes(ctypes.byref(sh), ctypes.byref(w), ctypes.byref(p),
                                ctypes.byref(ws)) == prox.PROX_EINVAL
    assert "activation" in prox.prox_last_error()


def test_query_sizes_rejects_batch(lib):
    assert _q(4096, 14336, 128, prox.PROX_BF16, 9)[0] == prox.PROX_EUNSUPPORTED
    assert _q(4096, 14336, 128, prox.PROX_BF16, 0)[0] == prox.PROX_EINVAL


def test_null_arguments_rejected_before_any_launch(lib):
    P = ctypes.c_void_p
    assert lib.prox_ffn_forward(None, P(16), 0.5, 3, P(16), None) == prox.PROX_EINVAL
    assert lib.prox_ffn_forward_batch(None, P(16), 1, 0.5, 3, P(16), None) == prox.PROX_EINVAL
    assert lib.prox_dense_ffn_forward(None, P(16), 1, P(16), None) == prox.PROX_EINVAL
    h = ctypes.c_void_p()
    sh = prox.prox_shape(512, 1024, 128, prox.PROX_BF16, 1)
    assert lib.prox_prepare_layer(ctypes.byref(sh), None, None, None, None, None, None,
                                  None, ctypes.byref(h)) == prox.PROX_EINVAL
    assert lib.prox_prepare_layer(None, P(256), P(256), P(256), P(256), P(256), P(256),
                                  None, ctypes.byref(h)) == prox.PROX_EINVAL
    # misaligned buffers
    assert lib.prox_prepare_layer(ctypes.byref(sh), P(256), P(256), P(256), P(258),
                                  P(256), P(256), None, ctypes.byref(h)) == prox.PROX_EINVAL
    assert lib.prox_stack_forward(None, 0, None, 3, None, 1, 1e-5, None) == prox.PROX_EINVAL
    arr = (ctypes.c_void_p * 1)(None)
    th = (ctypes.c_float * 1)(math.nan)
    assert lib.prox_stack_forward(arr, 1, th, 3, P(256), 1, 1e-5, None) == prox.PROX_EINVAL
    lib.prox_destroy_layer(None)  # no-op


def test_costmodel_effective_sparsity_of_configs():
    """Effective sparsity (Sec. 4.2 cost model) of the k choices used here:
    k = 30% of d_ff with half the inputs kept gives e = 0.7 - 2/9 * 0.5."""
    from free_sparse_swiglu_amd import costmodel, synth
    k = synth.k_for(14336, 0.7)
    assert k == 4301
    s2 = 1 - k / 14336
    e = costmodel.effective_sparsity(0.5, s2)
    assert abs(e - (s2 - 1 / 9)) < 1e-12
    assert [synth.k_for(14336, p) for p in (0.5, 0.6, 0.7)] == [7168, 5734, 4301]
    assert [synth.k_for(17408, p) for p in (0.6, 0.7)] == [6963, 5222]
    assert synth.k_for(28672, 0.7) == 8602 and synth.k_for(688, 0.7) == 206


def _qs(sh):
    w, p, ws = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    st = prox.load_library().prox_query_sizes(ctypes.byref(sh), ctypes.byref(w),
                                              ctypes.byref(p), ctypes.byref(ws))
    return st, w.value, p.value, ws.value


def test_kernel_choices_are_declared_shape_fields(lib):
    """The kernel path and the batched forms are prox_shape fields, checked
    like the sizes (no environment variable is read)."""
    base = dict(d_model=1024, d_ff=2816, group_size=128, dtype=prox.PROX_BF16, max_batch=8)
    ok = [dict(path=prox.PROX_PATH_MULTI), dict(batch_stage1=prox.PROX_FORM_VALU),
          dict(batch_stage1=prox.PROX_FORM_MFMA), dict(batch_upgate=prox.PROX_FORM_MFMA),
          dict(batch_upgate=prox.PROX_FORM_VALU)]
    for extra in ok:
        assert _qs(prox.prox_shape(**base, **extra))[0] == prox.PROX_OK, extra
    for extra in (dict(path=2), dict(batch_stage1=3), dict(batch_upgate=-1)):
        assert _qs(prox.prox_shape(**base, **extra))[0] == prox.PROX_EINVAL, extra
    f32 = dict(base, dtype=prox.PROX_F32)
    assert _qs(prox.prox_shape(**f32, batch_upgate=prox.PROX_FORM_MFMA))[0] == \
        prox.PROX_EUNSUPPORTED
    assert _qs(prox.prox_shape(**f32, batch_stage1=prox.PROX_FORM_MFMA))[0] == \
        prox.PROX_EUNSUPPORTED
    # the matrix-core Stage 1 keeps a second copy of the codes: the automatic
    # choice holds it from 2 tokens, the VALU form never
    auto = _qs(prox.prox_shape(**base))[2]
    valu = _qs(prox.prox_shape(**base, batch_stage1=prox.PROX_FORM_VALU))[2]
    assert auto - valu >= 1024 * 2816 // 2
    two = dict(base, max_batch=2)
    assert _qs(prox.prox_shape(**two))[2] == _qs(prox.prox_shape(**two, batch_stage1=2))[2]
    assert _qs(prox.prox_shape(**two, batch_stage1=1))[2] < _qs(prox.prox_shape(**two))[2]
    one = dict(base, max_batch=1)
    assert _qs(prox.prox_shape(**one))[2] == _qs(prox.prox_shape(**one, batch_stage1=1))[2]


def test_workspace_sync_block_is_shape_independent(lib):
    """Every workspace starts with the same fixed-size synchronisation block,
    so layers of different shapes (or max_batch) can share one workspace:
    each one's scratch starts past the block whatever its shape."""
    hdr = lib.prox_sync_block_bytes()
    assert hdr > 0 and hdr % 256 == 0
    shapes = [(4096, 14336, 128, prox.PROX_BF16, 1), (4096, 14336, 128, prox.PROX_BF16, 8),
              (256, 688, 64, prox.PROX_F32, 1), (8192, 28672, 128, prox.PROX_BF16, 8),
              (16384, 32768, 256, prox.PROX_BF16, 1)]
    for sh in shapes:
        st, _, _, ws = _q(*sh)
        assert st == prox.PROX_OK
        d_model, d_ff, _, dt, mb = sh
        esz = 2 if dt == prox.PROX_BF16 else 4
        # at least |s~|, s, x and y scratch past the block
        assert ws >= hdr + mb * d_ff * 4 + d_ff * 4 + 2 * mb * d_model * esz
    assert lib.prox_sync_block_bytes() == hdr


def test_status_entries_reject_null(lib):
    P = ctypes.c_void_p
    assert lib.prox_read_status(None, P(256), None) == prox.PROX_EINVAL
    assert lib.prox_set_wait_limit(None, 5) == prox.PROX_EINVAL
