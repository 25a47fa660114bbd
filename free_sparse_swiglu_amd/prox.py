"""Thin Python binding of libprox (C ABI in include/prox.h).

Argument marshalling only: every step of the FFN runs in the HIP kernels of
libprox.so.  PyTorch provides device memory and the current stream.  The
functions keep the C names; tensors stand in for device pointers.

The library is loaded on first use and a missing or unloadable library
raises immediately: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libprox.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "prox.h")

PROX_OK, PROX_EINVAL, PROX_EUNSUPPORTED, PROX_EHIP = 0, -1, -2, -3
PROX_F32, PROX_BF16 = 0, 1
PROX_ACT_SILU, PROX_ACT_GELU_TANH = 0, 1
PROX_PATH_PERSISTENT, PROX_PATH_MULTI = 0, 1
PROX_FORM_AUTO, PROX_FORM_VALU, PROX_FORM_MFMA = 0, 1, 2
_STATUS = {0: "PROX_OK", -1: "PROX_EINVAL", -2: "PROX_EUNSUPPORTED", -3: "PROX_EHIP"}


class ProxError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class prox_shape(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int), ("d_ff", ctypes.c_int),
                ("group_size", ctypes.c_int), ("dtype", ctypes.c_int),
                ("max_batch", ctypes.c_int), ("activation", ctypes.c_int),
                ("path", ctypes.c_int), ("batch_stage1", ctypes.c_int),
                ("batch_upgate", ctypes.c_int)]


class prox_debug(ctypes.Structure):
    _fields_ = [("n1", ctypes.c_void_p), ("idx", ctypes.c_void_p),
                ("s_abs", ctypes.c_void_p), ("sel", ctypes.c_void_p),
                ("s_sel", ctypes.c_void_p), ("n_union", ctypes.c_void_p),
                ("union_idx", ctypes.c_void_p), ("status", ctypes.c_void_p),
                ("n_sel", ctypes.c_void_p)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libprox.so and declare its signatures (raises if absent)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ProxError(PROX_EHIP, f"libprox.so not built ({path}); run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    S = ctypes.POINTER(prox_shape)
    Z = ctypes.POINTER(ctypes.c_size_t)
    sig = {
        "prox_query_sizes": ([S, Z, Z, Z], I),
        "prox_prepare_layer": ([S, P, P, P, P, P, P, P, ctypes.POINTER(P)], I),
        "prox_export_proxy": ([P, I, P, P, P], I),
        "prox_ffn_forward": ([P, P, F, I, P, P], I),
        "prox_ffn_forward_noalloc": ([P, P, F, I, P, P], I),
        "prox_ffn_forward_batch": ([P, P, I, F, I, P, P], I),
        "prox_ffn_forward_debug": ([P, P, I, F, I, P, ctypes.POINTER(prox_debug), P], I),
        "prox_dense_ffn_forward": ([P, P, I, P, P], I),
        "prox_stack_forward": ([ctypes.POINTER(P), I, ctypes.POINTER(F), I, P, I, F, P], I),
        "prox_ffn_forward_profiled": ([P, P, I, F, I, P, ctypes.POINTER(P), I,
                                       ctypes.POINTER(I), P], I),
        "prox_dense_ffn_forward_profiled": ([P, P, I, P, ctypes.POINTER(P), I,
                                             ctypes.POINTER(I), P], I),
        "prox_ffn_forward_traced": ([P, P, F, I, P, P, I, ctypes.POINTER(I), P], I),
        "prox_ffn_forward_ts": ([P, P, F, F, P, P], I),
        "prox_stage1": ([P, P, F, P, P], I),
        "prox_sparse_gemv_workspace_bytes": ([I, I], ctypes.c_size_t),
        "prox_sparse_gemv": ([P, P, I, I, P, F, P, P, P, P], I),
        "prox_stack_forward_ts": ([ctypes.POINTER(P), I, ctypes.POINTER(F), ctypes.POINTER(F), P,
                                   F, P], I),
        "prox_ffn_forward_ts_debug": ([P, P, F, F, P, ctypes.POINTER(prox_debug), P], I),
        "prox_rmsnorm": ([P, P, I, F, P, P], I),
        "prox_read_status": ([P, P, P], I),
        "prox_sync_block_bytes": ([], ctypes.c_size_t),
        "prox_set_wait_limit": ([P, ctypes.c_uint32], I),
        "prox_destroy_layer": ([P], None),
        "prox_last_error": ([], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def header_symbols(path: str = HEADER_PATH):
    """Names of the functions include/prox.h declares."""
    with open(path) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:prox_status|void|size_t|const char \*)\s*(prox_\w+)\s*\(",
                                 text, re.M)))


def _check(st: int):
    if st != PROX_OK:
        msg = load_library().prox_last_error()
        raise ProxError(st, msg.decode() if msg else "")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(dt) -> int:
    if dt == torch.bfloat16:
        return PROX_BF16
    if dt == torch.float32:
        return PROX_F32
    raise ProxError(PROX_EINVAL, f"unsupported dtype {dt}")


def prox_last_error() -> str:
    msg = load_library().prox_last_error()
    return msg.decode() if msg else ""


def prox_query_sizes(d_model: int, d_ff: int, group_size: int, dtype, max_batch: int = 1,
                     activation: int = 0, path: int = 0, batch_stage1: int = 0,
                     batch_upgate: int = 0):
    """(weights_bytes, proxy_bytes, workspace_bytes) for a layer shape."""
    sh = prox_shape(d_model, d_ff, group_size, _dtype_code(dtype), max_batch, activation, path,
                    batch_stage1, batch_upgate)
    w, p, ws = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(load_library().prox_query_sizes(ctypes.byref(sh), ctypes.byref(w),
                                           ctypes.byref(p), ctypes.byref(ws)))
    return w.value, p.value, ws.value


class Layer:
    """A prepared layer: the opaque handle plus the device buffers it uses."""

    def __init__(self, handle, shape, weights, proxy, workspace):
        self.handle = handle
        self.shape = shape
        self.weights, self.proxy, self.workspace = weights, proxy, workspace

    @property
    def d_model(self):
        return self.shape.d_model

    @property
    def d_ff(self):
        return self.shape.d_ff

    @property
    def dtype(self):
        return torch.bfloat16 if self.shape.dtype == PROX_BF16 else torch.float32

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.prox_destroy_layer(self.handle)
            self.handle = None


def prox_prepare_layer(w_up, w_gate, w_down, group_size: int, max_batch: int = 1,
                       workspace=None, activation: int = 0, path: int = 0,
                       batch_stage1: int = 0, batch_upgate: int = 0) -> Layer:
    """Relayout and quantize one layer (weights in the x.W layout, on the GPU).

    A workspace tensor may be shared by layers that run on one stream.
    activation: PROX_ACT_SILU (SwiGLU, default) or PROX_ACT_GELU_TANH (GeGLU);
    path: PROX_PATH_PERSISTENT (default) or PROX_PATH_MULTI for batch-1 calls;
    batch_stage1 / batch_upgate: PROX_FORM_* of the batched kernels."""
    d_model, d_ff = w_up.shape
    dt = _dtype_code(w_up.dtype)
    for t in (w_up, w_gate, w_down):
        if not (t.is_cuda and t.is_contiguous() and t.dtype == w_up.dtype):
            raise ProxError(PROX_EINVAL, "weights must be contiguous CUDA tensors of one dtype")
    if tuple(w_gate.shape) != (d_model, d_ff) or tuple(w_down.shape) != (d_ff, d_model):
        raise ProxError(PROX_EINVAL, "weight shapes do not match")
    wb, pb, wsb = prox_query_sizes(d_model, d_ff, group_size, w_up.dtype, max_batch, activation,
                                   path, batch_stage1, batch_upgate)
    dev = w_up.device
    weights = torch.empty(wb, dtype=torch.uint8, device=dev)
    proxy = torch.empty(pb, dtype=torch.uint8, device=dev)
    if workspace is None or workspace.numel() < wsb:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=dev)
    sh = prox_shape(d_model, d_ff, group_size, dt, max_batch, activation, path, batch_stage1,
                    batch_upgate)
    h = ctypes.c_void_p()
    _check(load_library().prox_prepare_layer(
        ctypes.byref(sh), _ptr(w_up), _ptr(w_gate), _ptr(w_down), _ptr(weights),
        _ptr(proxy), _ptr(workspace), _stream(), ctypes.byref(h)))
    return Layer(h, sh, weights, proxy, workspace)


def prox_read_status(layer: Layer, out=None):
    """The workspace status word (bit 0: a bounded wait timed out, results
    invalid; bit 1: the select's slow exact path), read and cleared on the
    current stream.  Returns a device int32 tensor [1]."""
    if out is None:
        out = torch.zeros(1, dtype=torch.int32, device=layer.weights.device)
    _check(load_library().prox_read_status(layer.handle, _ptr(out), _stream()))
    return out


def prox_set_wait_limit(layer: Layer, polls: int):
    """Polls before a bounded wait of the persistent kernel gives up."""
    _check(load_library().prox_set_wait_limit(layer.handle, int(polls)))


def prox_export_proxy(layer: Layer, matrix: int):
    """INT4 codes (int8 [d_model][d_ff]) and scales ([d_model/G][d_ff]) of a layer."""
    dev = layer.weights.device
    codes = torch.empty((layer.d_model, layer.d_ff), dtype=torch.int8, device=dev)
    scales = torch.empty((layer.d_model // layer.shape.group_size, layer.d_ff),
                         dtype=torch.float32, device=dev)
    _check(load_library().prox_export_proxy(layer.handle, matrix, _ptr(codes),
                                            _ptr(scales), _stream()))
    return codes, scales


def _out_like(x, y):
    return torch.empty_like(x) if y is None else y


def prox_ffn_forward(layer: Layer, x, threshold: float, k: int, y=None):
    y = _out_like(x, y)
    _check(load_library().prox_ffn_forward(layer.handle, _ptr(x), float(threshold), int(k),
                                           _ptr(y), _stream()))
    return y


def prox_ffn_forward_batch(layer: Layer, x, threshold: float, k: int, y=None):
    y = _out_like(x, y)
    _check(load_library().prox_ffn_forward_batch(layer.handle, _ptr(x), int(x.shape[0]),
                                                 float(threshold), int(k), _ptr(y), _stream()))
    return y


def _debug_buffers(layer: Layer, x):
    B = int(x.shape[0])
    dev = x.device
    out = dict(
        y=torch.empty_like(x),
        n1=torch.zeros(B, dtype=torch.int32, device=dev),
        idx=torch.full((B, layer.d_model), -1, dtype=torch.int32, device=dev),
        s_abs=torch.full((B, layer.d_ff), float("nan"), device=dev),
        sel=torch.full((B, layer.d_ff), -1, dtype=torch.int32, device=dev),
        s_sel=torch.full((B, layer.d_ff), float("nan"), device=dev),
        n_union=torch.zeros(1, dtype=torch.int32, device=dev),
        union_idx=torch.full((layer.d_ff,), -1, dtype=torch.int32, device=dev),
        status=torch.zeros(1, dtype=torch.int32, device=dev),
        n_sel=torch.full((1,), -1, dtype=torch.int32, device=dev),
    )
    dbg = prox_debug(*(ctypes.c_void_p(out[k].data_ptr()) for k in
                       ("n1", "idx", "s_abs", "sel", "s_sel", "n_union", "union_idx", "status",
                        "n_sel")))
    return out, dbg


def prox_ffn_forward_debug(layer: Layer, x, threshold: float, k: int):
    """Forward for x [batch][d_model] plus its intermediate results."""
    out, dbg = _debug_buffers(layer, x)
    _check(load_library().prox_ffn_forward_debug(layer.handle, _ptr(x), int(x.shape[0]),
                                                 float(threshold), int(k), _ptr(out["y"]),
                                                 ctypes.byref(dbg), _stream()))
    return out


def prox_ffn_forward_ts(layer: Layer, x, threshold_x: float, threshold_s: float, y=None):
    """Batch-1 forward with the Stage 2 threshold mask |s~| >= threshold_s."""
    y = _out_like(x, y)
    _check(load_library().prox_ffn_forward_ts(layer.handle, _ptr(x), float(threshold_x),
                                              float(threshold_s), _ptr(y), _stream()))
    return y


def prox_ffn_forward_ts_debug(layer: Layer, x, threshold_x: float, threshold_s: float):
    """prox_ffn_forward_ts for x [1][d_model] plus its intermediate results
    (n_sel holds the number of kept channels)."""
    out, dbg = _debug_buffers(layer, x)
    _check(load_library().prox_ffn_forward_ts_debug(layer.handle, _ptr(x), float(threshold_x),
                                                    float(threshold_s), _ptr(out["y"]),
                                                    ctypes.byref(dbg), _stream()))
    return out


def prox_dense_ffn_forward(layer: Layer, x, y=None):
    y = _out_like(x, y)
    B = 1 if x.dim() == 1 else int(x.shape[0])
    _check(load_library().prox_dense_ffn_forward(layer.handle, _ptr(x), B, _ptr(y), _stream()))
    return y


def prox_rmsnorm(layer: Layer, resid, eps: float = 1e-5, x=None):
    """cast(RMSNorm(resid)) for resid [batch][d_model] float32 (batch <= 8)."""
    B = 1 if resid.dim() == 1 else int(resid.shape[0])
    if x is None:
        x = torch.empty(resid.shape, dtype=layer.dtype, device=resid.device)
    _check(load_library().prox_rmsnorm(layer.handle, _ptr(resid), B, float(eps), _ptr(x),
                                       _stream()))
    return x


def _event_array(events):
    for e in events:  # torch creates the underlying hipEvent on first record()
        if not e.cuda_event:
            e.record()
    return (ctypes.c_void_p * len(events))(*[ctypes.c_void_p(e.cuda_event) for e in events])


def prox_ffn_forward_profiled(layer: Layer, x, threshold: float, k: int, events, y=None):
    """Forward of x [batch][d_model] with torch.cuda.Event objects recorded
    before the first kernel and after each kernel; returns (y, n_recorded)."""
    y = _out_like(x, y)
    n = ctypes.c_int()
    B = 1 if x.dim() == 1 else int(x.shape[0])
    _check(load_library().prox_ffn_forward_profiled(
        layer.handle, _ptr(x), B, float(threshold), int(k), _ptr(y),
        _event_array(events), len(events), ctypes.byref(n), _stream()))
    return y, n.value


def prox_dense_ffn_forward_profiled(layer: Layer, x, events, y=None):
    y = _out_like(x, y)
    n = ctypes.c_int()
    B = 1 if x.dim() == 1 else int(x.shape[0])
    _check(load_library().prox_dense_ffn_forward_profiled(
        layer.handle, _ptr(x), B, _ptr(y), _event_array(events), len(events),
        ctypes.byref(n), _stream()))
    return y, n.value


def prox_ffn_forward_traced(layer: Layer, x, threshold: float, k: int, y=None):
    """Batch-1 forward on the persistent kernel with its per-ticket timeline.

    Returns (y, trace, counts): trace is an int64 tensor [tickets][4] of
    (start, wait end, end, work-group | phase << 32), times in 100 MHz clock
    ticks, phase 1..4 = Stage 1, select, up/gate, down; counts gives the
    tickets of each phase."""
    y = _out_like(x, y)
    counts = (ctypes.c_int * 4)()
    lib = load_library()
    _check(lib.prox_ffn_forward_traced(layer.handle, _ptr(x), float(threshold), int(k), _ptr(y),
                                       None, 0, counts, _stream()))
    total = sum(counts)
    trace = torch.zeros(total, 4, dtype=torch.int64, device=x.device)
    _check(lib.prox_ffn_forward_traced(layer.handle, _ptr(x), float(threshold), int(k), _ptr(y),
                                       _ptr(trace), total, counts, _stream()))
    return y, trace, list(counts)


def prox_stack_forward(layers, thresholds, k: int, resid, eps: float = 1e-5):
    """Run the FFN stack on the float32 residual stream `resid` in place."""
    n = len(layers)
    arr = (ctypes.c_void_p * n)(*[L.handle for L in layers])
    th = (ctypes.c_float * n)(*[float(t) for t in thresholds]) if thresholds is not None else None
    B = 1 if resid.dim() == 1 else int(resid.shape[0])
    _check(load_library().prox_stack_forward(arr, n, th, int(k), _ptr(resid), B, float(eps),
                                             _stream()))
    return resid


def prox_stack_forward_ts(layers, thresholds_x, thresholds_s, resid, eps: float = 1e-5):
    """Run the FFN stack with Stage 2 threshold masks on the float32 residual
    resid [d_model] (one token) in place."""
    n = len(layers)
    arr = (ctypes.c_void_p * n)(*[L.handle for L in layers])
    tx = (ctypes.c_float * n)(*[float(t) for t in thresholds_x])
    ts = (ctypes.c_float * n)(*[float(t) for t in thresholds_s])
    _check(load_library().prox_stack_forward_ts(arr, n, tx, ts, _ptr(resid), float(eps), _stream()))
    return resid


def prox_stage1(layer: Layer, x, threshold: float, s_abs=None):
    """Stage 1 alone for one token; returns s_abs (or None when not asked)."""
    _check(load_library().prox_stage1(layer.handle, _ptr(x), float(threshold), _ptr(s_abs),
                                      _stream()))
    return s_abs


def prox_sparse_gemv_workspace(d_model: int, d_ff: int, device="cuda"):
    n = load_library().prox_sparse_gemv_workspace_bytes(int(d_model), int(d_ff))
    return torch.zeros(n, dtype=torch.uint8, device=device)


def prox_sparse_gemv(w_up, w_gate, x, threshold: float, workspace, u=None, g=None):
    """Input-sparse bf16 GEMV: (u, g) = x_S W_up, x_S W_gate over |x_i| >= threshold."""
    d_model, d_ff = w_up.shape
    if u is None:
        u = torch.empty(d_ff, dtype=torch.float32, device=x.device)
    if g is None:
        g = torch.empty(d_ff, dtype=torch.float32, device=x.device)
    _check(load_library().prox_sparse_gemv(_ptr(w_up), _ptr(w_gate), int(d_model), int(d_ff),
                                           _ptr(x), float(threshold), _ptr(u), _ptr(g),
                                           _ptr(workspace), _stream()))
    return u, g
