#!/usr/bin/env python3
"""Benchmark of the Prox two-stage sparse SwiGLU FFN decode step on one GPU.

Default workload: one 8B-shaped FFN layer (d_model 4096, d_ff 14336, bf16,
INT4 proxy with G = 128) at 70% FFN sparsity (k = 4301 of 14336 channels),
batch 1.  A step is one full forward of the layer (Stage 1 threshold +
compaction + INT4 proxy, top-k mask, Stage 2 exact up/gate + SwiGLU, Stage 2
down projection) for one token.  Steps rotate over a ring of distinct seeded
layers (8 x 415 MB by default) and inputs so that the 256 MB last-level cache
cannot serve a repeated layer: the bytes come from HBM.

Printed: one JSON line.  value = achieved GB/s on the algorithmic bytes of a
step (weights actually needed, x, y) over the measured step time; also
microseconds per layer, the duration of the step's one persistent kernel (HIP
events recorded by the library around it, on the launch stream), the same
step on the multi-kernel path with its per-kernel breakdown, the dense bf16
baseline on the same relaid weights, and the CPU oracle timed on the host
cores.

Other workloads (--workload): 14b (k at 70%), 70b (batch 1/2/4/8), stack8b
(32 layers x 128 sequential tokens, tokens/s; top-k and the calibrated
threshold mode), alpha (INT4 proxy GEMV over bf16 input-sparse GEMV time, the
alpha of the allocation model), copy (a plain device copy of known size, used
to scale rocprofv3 byte counters).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
KERNEL_NAMES = ["stage1_proxy", "topk", "stage2_upgate", "stage2_down"]  # multi-kernel path
FUSED_KERNEL = "ffn_fused_kernel"


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("prox_kernels.hip", "prox_fused.hip", "prox_api.hip", "prox_internal.h",
              "prox_device.h"):
        with open(os.path.join(ROOT, "free_sparse_swiglu_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    """HBM traffic per launch of the dominant kernel from committed rocprofv3
    counter summaries, if they were taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t


def algorithmic_bytes(cfg, n1, groups_touched, k, batch=1, union=None):
    """Bytes the step must move: proxy codes of surviving rows and scales of
    touched groups (Stage 1), up+gate rows and down rows of the selected
    channels (Stage 2), x and y."""
    import math
    ntile = math.ceil(cfg.d_ff / 256)
    esz = 2 if cfg.dtype == "bf16" else 4
    stage1 = n1 * ntile * 256 + groups_touched * 2 * cfg.d_ff * 4
    m = k if union is None else union
    upgate = m * 2 * cfg.d_model * esz
    down = m * cfg.d_model * esz
    io = 2 * batch * cfg.d_model * esz
    return dict(stage1=stage1, upgate=upgate, down=down, io=io,
                total=stage1 + upgate + down + io)


def saved_thresholds(name, recipe, compute):
    """The thresholds of a workload from its saved calibration artifact
    (calib/<name>.json) when its recipe matches; otherwise calibrated now and
    saved (also under gpurun_out/calib/).  Returns (thresholds, source, path)."""
    from free_sparse_swiglu_amd import thresholds
    th = thresholds.load(name, recipe)
    if th is not None:
        return th, "loaded", thresholds.path_for(name)
    th = compute()
    p = thresholds.save(name, recipe, th)
    try:
        thresholds.save(name, recipe, th, out_dir=os.path.join(ROOT, "gpurun_out", "calib"))
    except OSError:
        pass
    return th, "calibrated", p


def ring_recipe(cfg, ring):
    return dict(workload=cfg.name, d_model=cfg.d_model, d_ff=cfg.d_ff, dtype=cfg.dtype,
                x_dist=cfg.x_dist, quantile=cfg.tau_quantile, n_calib=cfg.n_calib, ring=ring,
                inputs="synth.make_inputs(cfg, n_calib, 'calib', layer, 'cuda')",
                rule="tau_x = sorted |x| at floor(q (N - 1))")


def ring_taus(cfg, ring):
    """Per-layer input thresholds of a ring of seeded layers (saved artifact)."""
    from free_sparse_swiglu_amd import synth
    th, src, path = saved_thresholds(
        f"{cfg.name}_ring{ring}", ring_recipe(cfg, ring),
        lambda: dict(tau_x=[synth.layer_tau(cfg, l, "cuda") for l in range(ring)]))
    return th["tau_x"], dict(source=src, path=os.path.relpath(path, ROOT))


def build_ring(cfg, ring, max_batch=1, path=0, activation=0, batch_upgate=0, taus=None):
    """Prepare `ring` seeded layers sharing one workspace.  path=1
    (PROX_PATH_MULTI) prepares them for the multi-kernel path (one kernel per
    phase); activation 1 makes them GeGLU layers; batch_upgate is the
    prox_form of the batched up/gate step."""
    import torch

    from free_sparse_swiglu_amd import prox, synth
    layers = []
    ws = None
    if taus is None:
        taus, _ = ring_taus(cfg, ring)
    for l in range(ring):
        W = synth.make_layer(cfg, l, "cuda")
        L = prox.prox_prepare_layer(*W, cfg.group, max_batch, workspace=ws,
                                    activation=activation, path=path,
                                    batch_upgate=batch_upgate)
        ws = L.workspace
        torch.cuda.synchronize()
        del W
        layers.append(L)
    return layers, list(taus)


def torch_dense_ms(cfg, X, steps, warmup, ring=4):
    """The dense SwiGLU FFN step in plain PyTorch (torch.matmul on the bf16
    weights in their x.W layout, i.e. the vendor BLAS, plus SiLU and the
    product), over a ring of `ring` freshly generated layers: context for the
    library's own dense path, not part of the product."""
    import torch
    from free_sparse_swiglu_amd import synth
    W = [synth.make_layer(cfg, l, "cuda") for l in range(ring)]
    nx = X[0].shape[0]

    def step(i):
        wu, wg, wd = W[i % ring]
        x = X[i % len(X)][(i // ring) % nx][None]
        u = torch.matmul(x, wu)
        g = torch.matmul(x, wg)
        torch.matmul(u * torch.nn.functional.silu(g), wd)
    ms = time_loop(step, steps, warmup)
    del W
    torch.cuda.synchronize()
    return ms


def time_loop(fn, steps, warmup):
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        fn(i)
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps  # ms per step


def time_repeats(fn, steps, warmup, repeats):
    """`repeats` timed loops of exactly `steps` steps each (the warm-up runs
    once, before the first); returns the list of ms per step."""
    out = [time_loop(fn, steps, warmup)]
    for _ in range(repeats - 1):
        out.append(time_loop(fn, steps, 0))
    return out


def spread(ms_list):
    import numpy as np
    a = np.asarray(ms_list) * 1e3
    return dict(repeats=len(a), median_us=round(float(np.median(a)), 3),
                min_us=round(float(a.min()), 3), max_us=round(float(a.max()), 3))


def measured_copy_peak(steps=20):
    """Device-to-device copy of 1 GiB (bytes read + bytes written per second):
    the streaming rate this GPU sustains, reported beside the published peak."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    ms = min(time_loop(lambda i: b.copy_(a), steps, 3) for _ in range(3))
    del a, b
    torch.cuda.synchronize()
    return round(2 * n / (ms * 1e-3) / 1e9, 1)


def profile_kernels(call, steps, n_events):
    """Average per-kernel milliseconds from library-recorded events."""
    import torch
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_events)] for _ in range(steps)]
    nrec = 0
    for i in range(steps):
        nrec = call(i, evs[i])
    torch.cuda.synchronize()
    sums = [0.0] * (nrec - 1)
    for i in range(steps):
        for j in range(nrec - 1):
            sums[j] += evs[i][j].elapsed_time(evs[i][j + 1])
    return [s / steps for s in sums]


def cpu_baseline(cfg, k, tau, budget_s, bytes_per_step):
    """The oracle as it stands, single-threaded C, on a bounded sample."""
    import numpy as np
    import torch

    import oracle
    from free_sparse_swiglu_amd import synth
    W = [w.float().cpu().numpy() for w in synth.make_layer(cfg, 0, "cuda")]
    ol = oracle.Layer(*W, cfg.group)  # prepare (quantize), not timed
    X = synth.make_inputs(cfg, 512, "cpu-sample", 0, "cuda").float().cpu().numpy()
    n, t_total = 0, 0.0
    while n < X.shape[0] and (t_total < budget_s or n == 0):
        t0 = time.perf_counter()
        oracle.forward(ol, X[n], tau, k)
        t_total += time.perf_counter() - t0
        n += 1
    sec = t_total / n
    return dict(value=round(bytes_per_step / sec / 1e9, 4), unit="GB/s",
                us_per_layer=round(sec * 1e6, 1), cores=1, kind="oracle",
                sample=f"oracle forward (input mask, INT4 proxy, top-k, exact Stage 2) of "
                       f"{n} tokens on layer 0 of the {cfg.name} ring, single-threaded C "
                       f"(host has {os.cpu_count()} logical CPUs)")


def bench_single_layer(args, name):
    import numpy as np
    import torch

    from free_sparse_swiglu_amd import costmodel, prox, synth
    cfg = synth.CONFIGS[name]
    k = synth.k_for(cfg.d_ff, args.sparsity)
    taus0, tsrc = ring_taus(cfg, args.ring)
    layers, taus = build_ring(cfg, args.ring, taus=taus0)
    R = len(layers)
    NX = 16
    X = [synth.make_inputs(cfg, NX, "bench", l, "cuda") for l in range(R)]
    y = torch.empty(cfg.d_model, dtype=X[0].dtype, device="cuda")

    # Survivor counts of the bench inputs, from the library's own compaction.
    n1s, gts = [], []
    for l in range(R):
        for t in range(NX):
            out = prox.prox_ffn_forward_debug(layers[l], X[l][t:t + 1], taus[l], k)
            idx = out["idx"][0, :int(out["n1"][0])].cpu().numpy()
            n1s.append(idx.size)
            gts.append(np.unique(idx // cfg.group).size)
    torch.cuda.synchronize()
    n1m, gtm = float(np.mean(n1s)), float(np.mean(gts))
    ab = algorithmic_bytes(cfg, n1m, gtm, k)

    def step(i):
        l = i % R
        prox.prox_ffn_forward(layers[l], X[l][(i // R) % NX], taus[l], k, y)

    srep = time_repeats(step, args.steps, args.warmup, args.repeats)
    import numpy as _np
    ms = float(_np.median(srep))

    def pstep(i, evs):
        l = i % R
        return prox.prox_ffn_forward_profiled(layers[l], X[l][(i // R) % NX][None], taus[l], k,
                                              evs, y[None])[1]
    kms = profile_kernels(pstep, min(args.steps, 200), 6)

    def dstep(i):
        l = i % R
        prox.prox_dense_ffn_forward(layers[l], X[l][(i // R) % NX], y)
    drep = time_repeats(dstep, args.steps, args.warmup, args.repeats)
    dms = float(_np.median(drep))
    tdms = torch_dense_ms(cfg, X, args.steps, args.warmup)

    def dpstep(i, evs):
        l = i % R
        return prox.prox_dense_ffn_forward_profiled(layers[l], X[l][(i // R) % NX][None], evs,
                                                    y[None])[1]
    dkms = profile_kernels(dpstep, min(args.steps, 100), 3)

    # Graph-launched step (same kernels, one replay per ring pass).
    graph_ms = None
    try:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(R):
                step(i)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(R):
                step(i)
        reps = max(1, args.steps // R)
        graph_ms = time_loop(lambda i: g.replay(), reps, 2) / R
    except Exception as e:  # capture unsupported: report eager numbers only
        print(f"graph capture skipped: {e}", file=sys.stderr)

    # Other sparsities of the same shape (shorter loops).
    others = {}
    for sp in cfg.sparsities:
        if abs(sp - args.sparsity) < 1e-9:
            continue
        kk = synth.k_for(cfg.d_ff, sp)

        def ostep(i, kk=kk):
            l = i % R
            prox.prox_ffn_forward(layers[l], X[l][(i // R) % NX], taus[l], kk, y)
        oms = time_loop(ostep, max(20, args.steps // 2), 5)
        ob = algorithmic_bytes(cfg, n1m, gtm, kk)["total"]
        others[f"{int(round(sp * 100))}%"] = dict(k=kk, us_per_layer=round(oms * 1e3, 2),
                                                  GBps=round(ob / (oms * 1e-3) / 1e9, 1),
                                                  speedup_vs_dense=round(dms / oms, 3))

    # The same step on the multi-kernel path (one kernel per phase), for the
    # per-phase breakdown.
    mlayers, _ = build_ring(cfg, R, path=prox.PROX_PATH_MULTI)

    def mstep(i):
        l = i % R
        prox.prox_ffn_forward(mlayers[l], X[l][(i // R) % NX], taus[l], k, y)
    mms = time_loop(mstep, args.steps, args.warmup)

    def mpstep(i, evs):
        l = i % R
        return prox.prox_ffn_forward_profiled(mlayers[l], X[l][(i // R) % NX][None], taus[l], k,
                                              evs, y[None])[1]
    mkms = profile_kernels(mpstep, min(args.steps, 200), 6)
    del mlayers
    torch.cuda.synchronize()
    # The Stage 2 threshold mask (Sec. 4.1) instead of top-k: tau_s per layer
    # is the 0.7 quantile of |s~| over 32 calibration inputs of the layer, so
    # about 30% of the channels are kept, as with k = 30% of d_ff.
    from free_sparse_swiglu_amd import calibrate
    tss = []
    for l in range(R):
        xc = synth.make_inputs(cfg, 32, "calib", l, "cuda")
        S = torch.empty(32, cfg.d_ff, device="cuda")
        for t in range(32):
            calibrate._abs_proxy_state(layers[l], xc[t:t + 1], taus[l], S[t], y[None])
        tss.append(synth.calibrate_tau(S, 0.7))

    def tstep(i):
        l = i % R
        prox.prox_ffn_forward_ts(layers[l], X[l][(i // R) % NX], taus[l], tss[l], y)
    tms = time_loop(tstep, args.steps, args.warmup)
    kept = []
    for l in range(R):
        for t in range(NX):
            o = prox.prox_ffn_forward_ts_debug(layers[l], X[l][t:t + 1], taus[l], tss[l])
            kept.append(int(o["n_sel"][0]))
    mkept = float(np.mean(kept))
    tbytes = algorithmic_bytes(cfg, n1m, gtm, mkept)["total"]

    # The same step on GeGLU layers (tanh-form GELU gate), same weights.
    glayers, _ = build_ring(cfg, R, activation=1)

    def gstep(i):
        l = i % R
        prox.prox_ffn_forward(glayers[l], X[l][(i // R) % NX], taus[l], k, y)
    gms = time_loop(gstep, args.steps, args.warmup)
    del glayers
    torch.cuda.synchronize()
    kbytes = dict(stage1_proxy=ab["stage1"] + cfg.d_model * 2, topk=None,
                  stage2_upgate=ab["upgate"] + cfg.d_model * 2, stage2_down=ab["down"])
    mkern = {}
    for nm, t in zip(KERNEL_NAMES, mkms):
        b = kbytes.get(nm)
        mkern[nm] = dict(us=round(t * 1e3, 2),
                         GBps=round(b / (t * 1e-3) / 1e9, 1) if b else None)

    # The default path is one persistent kernel: the library records an
    # event before and after it, so kms has one entry (that bracket adds the
    # event overhead to the kernel).
    kern = {FUSED_KERNEL: dict(us=round(kms[0] * 1e3, 2),
                               GBps=round(ab["total"] / (kms[0] * 1e-3) / 1e9, 1))}
    dom = FUSED_KERNEL
    # A step is exactly one launch of the persistent kernel on the launch
    # stream, so the timed loop gives its average launch duration (launch to
    # launch, dispatch gap included).
    dom_us = ms * 1e3
    achieved = ab["total"] / (dom_us * 1e-6) / 1e9
    traffic = load_traffic(name)
    copy_peak = measured_copy_peak()
    roof = dict(bound="hbm", kernel=dom, launch_us=round(dom_us, 2),
                achieved=round(achieved, 1), peak=HBM_PEAK_GBPS,
                unit="GB/s", frac=round(achieved / HBM_PEAK_GBPS, 4),
                bytes_per_launch=int(ab["total"]),
                traffic=(traffic or {}).get("bytes_per_launch") if traffic else None,
                measured_peak=copy_peak,
                measured_peak_kind="1 GiB device copy, bytes read + written per second",
                frac_of_measured=round(achieved / copy_peak, 4))

    s1 = 1.0 - n1m / cfg.d_model
    s2 = 1.0 - k / cfg.d_ff
    res = dict(
        metric="us/FFN layer and achieved HBM GB/s at 70% sparsity, 8B-shaped, batch 1"
        if name == "8b" else f"us/FFN layer and achieved HBM GB/s, {name}-shaped, batch 1",
        value=round(ab["total"] / (ms * 1e-3) / 1e9, 1),
        unit="GB/s",
        n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=round(ms, 5),
        us_per_layer=round(ms * 1e3, 2),
        repeats=spread(srep),
        us_per_layer_graph=round(graph_ms * 1e3, 2) if graph_ms else None,
        hbm_frac=round(ab["total"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype="bf16", data="synthetic",
        config=dict(workload=f"{name}-shaped single FFN layer, batch 1",
                    threshold_artifact=tsrc,
                    d_model=cfg.d_model, d_ff=cfg.d_ff, group=cfg.group, k=k,
                    sparsity=args.sparsity, ring_layers=R, tau_quantile=cfg.tau_quantile,
                    mean_n1=round(n1m, 1), realised_s1=round(s1, 4), s2=round(s2, 4),
                    effective_sparsity=round(costmodel.effective_sparsity(s1, s2), 4),
                    bytes_per_step=int(ab["total"])),
        kernels=kern,
        multi_kernel_path=dict(us_per_layer=round(mms * 1e3, 2), kernels=mkern),
        threshold_mask=dict(us_per_layer=round(tms * 1e3, 2), mean_kept=round(mkept, 1),
                            GBps=round(tbytes / (tms * 1e-3) / 1e9, 1),
                            speedup_vs_dense=round(dms / tms, 3)),
        geglu=dict(us_per_layer=round(gms * 1e3, 2),
                   GBps=round(ab["total"] / (gms * 1e-3) / 1e9, 1)),
        dense=dict(us_per_layer=round(dms * 1e3, 2), repeats=spread(drep),
                   GBps=round(3 * cfg.d_model * cfg.d_ff * 2 / (dms * 1e-3) / 1e9, 1),
                   kernels=dict(upgate_us=round(dkms[0] * 1e3, 2),
                                down_us=round(dkms[1] * 1e3, 2)),
                   torch_matmul_us_per_layer=round(tdms * 1e3, 2)),
        speedup_vs_dense=round(dms / ms, 3),
        other_sparsities=others,
        roofline=roof,
    )
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, k, taus[0], args.cpu_seconds, ab["total"])
    else:
        res["cpu_baseline"] = None
    return res


def bench_batch(args):
    import numpy as np
    import torch

    from free_sparse_swiglu_amd import prox, synth
    cfg = synth.CONFIGS["70b"]
    k = synth.k_for(cfg.d_ff, args.sparsity)
    form = prox.PROX_FORM_MFMA if args.batch_gemv == "mfma" else prox.PROX_FORM_AUTO
    layers, taus = build_ring(cfg, args.ring, max_batch=8, batch_upgate=form)
    R = len(layers)
    out = {}
    for B in cfg.batches:
        X = [synth.make_inputs(cfg, B, f"bench{B}", l, "cuda") for l in range(R)]
        y = torch.empty_like(X[0])
        unions = []
        for l in range(R):
            o = prox.prox_ffn_forward_debug(layers[l], X[l], taus[l], k)
            unions.append(int(o["n_union"][0]) if B > 1 else k)
        ms = time_loop(lambda i: prox.prox_ffn_forward_batch(layers[i % R], X[i % R], taus[i % R],
                                                             k, y), args.steps, args.warmup)
        dms = time_loop(lambda i: prox.prox_dense_ffn_forward(layers[i % R], X[i % R], y),
                        args.steps, args.warmup)
        out[f"B{B}"] = dict(us_per_step=round(ms * 1e3, 2), dense_us=round(dms * 1e3, 2),
                            speedup_vs_dense=round(dms / ms, 3),
                            mean_union=float(np.mean(unions)),
                            union_frac=round(float(np.mean(unions)) / cfg.d_ff, 4))
    return dict(metric="us per batched FFN step, 70B-shaped, 70% sparsity", unit="us",
                batch_gemv=args.batch_gemv,
                n_gpus=1, steps=args.steps, warmup=args.warmup, dtype="bf16",
                data="synthetic", config=dict(workload="70B-shaped single FFN layer, "
                                                       "batch 1/2/4/8", k=k, ring_layers=R),
                batches=out)


def bench_stack(args):
    import torch

    from free_sparse_swiglu_amd import calibrate, prox, synth
    cfg = synth.CONFIGS["stack8b"]
    k = synth.k_for(cfg.d_ff, args.sparsity)
    layers = []
    ws = None
    for l in range(cfg.layers):
        W = synth.make_layer(cfg, l, "cuda")
        L = prox.prox_prepare_layer(*W, cfg.group, 8, workspace=ws)
        ws = L.workspace
        torch.cuda.synchronize()
        del W
        layers.append(L)
    from free_sparse_swiglu_amd import costmodel
    s1, s2 = costmodel.allocate(0.7)
    recipe = dict(workload=cfg.name, layers=cfg.layers, d_model=cfg.d_model, d_ff=cfg.d_ff,
                  k=k, quantile=cfg.tau_quantile, n_calib=cfg.n_calib, n_calib_ts=64,
                  s1=round(s1, 6), s2=round(s2, 6), eps=1e-5,
                  inputs="synth.make_inputs(cfg, n_calib, 'calib', 0, 'cuda') as residuals",
                  rule="sequential in depth order (Algorithm 1, App. A.7)")

    def calibrate_stack():
        calib = synth.make_inputs(cfg, cfg.n_calib, "calib", 0, "cuda").float()
        taus = calibrate.sequential_thresholds(layers, calib, cfg.tau_quantile, k)
        tx, ts = calibrate.sequential_thresholds_ts(layers, calib[:64], s1, s2)
        return dict(tau_x_topk=taus, tau_x=tx, tau_s=ts)
    th, tsrc, tpath = saved_thresholds(f"{cfg.name}", recipe, calibrate_stack)
    taus, tx, ts = th["tau_x_topk"], th["tau_x"], th["tau_s"]
    ntok = 128
    R0 = synth.make_inputs(cfg, ntok, "stack", 0, "cuda").float()
    r = R0.clone()

    def run_tokens(kk):
        r.copy_(R0)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(ntok):
            prox.prox_stack_forward(layers, taus, kk, r[t])
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    run_tokens(k)
    sec = run_tokens(k)
    dsec = run_tokens(-1)

    # The same 32-layer step captured once as a HIP graph (torch.cuda.graph
    # around one prox_stack_forward call on a fixed residual buffer) and
    # replayed 128 times: launch overhead of graph replay against stream
    # launches of the same kernels.
    graph_tps = None
    try:
        rg = R0[0].clone()
        gs = torch.cuda.Stream()
        gs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(gs):
            prox.prox_stack_forward(layers, taus, k, rg)
        torch.cuda.current_stream().wait_stream(gs)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            prox.prox_stack_forward(layers, taus, k, rg)
        for _ in range(4):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(ntok):
            g.replay()
        torch.cuda.synchronize()
        graph_tps = round(ntok / (time.perf_counter() - t0), 1)
    except Exception as e:  # capture unsupported: stream numbers only
        print(f"graph capture skipped: {e}", file=sys.stderr)

    # The pages' own operating mode: calibrated thresholds for both stages
    # (Sec. 4.1 masks), allocated for a 70% effective sparsity target (Sec. 4.2:
    # s1 = 0.7, s2 = 0.767), calibrated sequentially (App. A.7, Algorithm 1)
    # on 64 tokens, timed on the same 128 tokens, runtime sparsity measured on
    # 16 other tokens.
    def run_tokens_ts():
        r.copy_(R0)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(ntok):
            prox.prox_stack_forward_ts(layers, tx, ts, r[t])
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    run_tokens_ts()
    tsec = run_tokens_ts()
    held = synth.make_inputs(cfg, 16, "held-out", 0, "cuda").float()
    rs = calibrate.runtime_sparsity(layers, tx, ts, held)
    threshold_mode = dict(
        target_e=0.7, s1=round(s1, 4), s2=round(s2, 4),
        tokens_per_s=round(ntok / tsec, 1), speedup_vs_dense=round(dsec / tsec, 3),
        us_per_layer=round(tsec / ntok / cfg.layers * 1e6, 2),
        runtime=dict(s1=round(rs["s1"], 4), s2=round(rs["s2"], 4), e=round(rs["e"], 4)),
        thresholds_x=[round(t, 5) for t in tx], thresholds_s=[float("%.5g" % t) for t in ts])
    return dict(metric="tokens/s of a 32-layer 8B-shaped FFN stack, batch 1, 70% sparsity",
                value=round(ntok / sec, 1), unit="tokens/s", n_gpus=1, dtype="bf16",
                data="synthetic", higher_is_better=True,
                config=dict(workload="32 x 8B-shaped FFN layers + RMSNorm + residual, "
                                     "128 sequential tokens", k=k, layers=cfg.layers),
                graph_tokens_per_s=graph_tps,
                threshold_artifact=dict(source=tsrc, path=os.path.relpath(tpath, ROOT)),
                dense_tokens_per_s=round(ntok / dsec, 1), speedup_vs_dense=round(dsec / sec, 3),
                us_per_layer=round(sec / ntok / cfg.layers * 1e6, 2),
                thresholds=[round(t, 5) for t in taus],
                threshold_mode=threshold_mode)


def bench_alpha(args):
    """alpha of the allocation model (Sec. 4.2; App. A.3 measures it on NVIDIA
    GPUs): the INT4 proxy GEMV time over the bf16 input-sparse GEMV time at
    the same input sparsity s1, both for the up and gate projections of one
    token.  INT4: prox_stage1 (Stage 1 kernel, activation epilogue included);
    bf16: prox_sparse_gemv on the layer's row-major bf16 weights."""
    import numpy as np
    import torch

    from free_sparse_swiglu_amd import prox, synth
    out = {}
    R = 4
    for name in ("8b", "14b", "70b"):
        cfg = synth.CONFIGS[name]
        Ws, layers = [], []
        ws = None
        for l in range(R):
            W = synth.make_layer(cfg, l, "cuda")
            L = prox.prox_prepare_layer(*W, cfg.group, 1, workspace=ws)
            ws = L.workspace
            Ws.append((W[0], W[1]))
            del W
            layers.append(L)
        torch.cuda.synchronize()
        gws = prox.prox_sparse_gemv_workspace(cfg.d_model, cfg.d_ff)
        u = torch.empty(cfg.d_ff, device="cuda")
        g = torch.empty(cfg.d_ff, device="cuda")
        X = [synth.make_inputs(cfg, 8, "bench", l, "cuda") for l in range(R)]
        calib = [synth.make_inputs(cfg, 64, "calib", l, "cuda") for l in range(R)]
        rows = {}
        for s1 in (0.4, 0.5, 0.6, 0.7):
            taus = [synth.calibrate_tau(calib[l], s1) for l in range(R)]
            n1 = [float((X[l].abs() >= taus[l]).sum(dim=1).float().mean()) for l in range(R)]

            def i4(i):
                prox.prox_stage1(layers[i % R], X[i % R][(i // R) % 8], taus[i % R])

            def bf(i):
                l = i % R
                prox.prox_sparse_gemv(Ws[l][0], Ws[l][1], X[l][(i // R) % 8], taus[l], gws, u, g)
            t4 = time_loop(i4, args.steps, args.warmup)
            tb = time_loop(bf, args.steps, args.warmup)
            m = float(np.mean(n1))
            rows[f"s1={s1}"] = dict(
                realized_s1=round(1 - m / cfg.d_model, 4),
                int4_us=round(t4 * 1e3, 2), bf16_us=round(tb * 1e3, 2),
                alpha=round(t4 / tb, 3),
                int4_GBps=round(m * cfg.d_ff / (t4 * 1e-3) / 1e9, 1),
                bf16_GBps=round(m * cfg.d_ff * 4 / (tb * 1e-3) / 1e9, 1))
        out[name] = rows
        del layers, Ws, X, calib
        torch.cuda.synchronize()
    alphas = [r["alpha"] for rows in out.values() for r in rows.values()]
    return dict(metric="alpha = INT4 proxy GEMV time / bf16 input-sparse GEMV time, "
                       "batch 1, same input sparsity",
                value=round(float(np.mean(alphas)), 3), unit="ratio", n_gpus=1,
                steps=args.steps, warmup=args.warmup, higher_is_better=False, dtype="bf16",
                data="synthetic",
                config=dict(workload="up+gate GEMVs of 8B/14B/70B-shaped layers at s1 = 0.4, "
                                     "0.5, 0.6, 0.7", ring_layers=R),
                pages_alpha=dict(model_value=1 / 3, measured_range=[0.234, 0.351],
                                 pooled_mean=0.285),
                shapes=out)


def bench_timeline(args):
    """Per-phase timeline of the persistent kernel at the 8B shape (k at the
    requested sparsity): each traced call records, per work item, its start,
    the end of its wait for earlier items and its end (100 MHz GPU clock).
    Reported per phase, in microseconds from the call's first item start:
    the median over calls of the first start, the median start, the last end
    and the median wait."""
    import numpy as np
    import torch

    from free_sparse_swiglu_amd import prox, synth
    cfg = synth.CONFIGS["8b"]
    k = synth.k_for(cfg.d_ff, args.sparsity)
    layers, taus = build_ring(cfg, min(args.ring, 4))
    R = len(layers)
    X = [synth.make_inputs(cfg, 8, "bench", l, "cuda") for l in range(R)]
    y = torch.empty(cfg.d_model, dtype=X[0].dtype, device="cuda")
    for i in range(args.warmup):
        prox.prox_ffn_forward(layers[i % R], X[i % R][i % 8], taus[i % R], k, y)
    names = {1: "stage1", 2: "select", 3: "upgate", 4: "down"}
    # "mid" is the item's middle stamp: the end of its wait for earlier items;
    # for a Stage 1 item the end of its code loop, for the select the moment
    # b* is published
    per = {n: dict(first_start=[], med_start=[], med_mid=[], last_mid=[], last_end=[],
                   med_dur=[]) for n in names.values()}
    spans = []
    ncalls = max(4, min(args.steps, 40))
    for i in range(ncalls):
        l = i % R
        _, tr, counts = prox.prox_ffn_forward_traced(layers[l], X[l][i % 8], taus[l], k, y)
        torch.cuda.synchronize()
        t = tr.cpu().numpy()
        t0 = t[:, 0].min()
        spans.append((t[:, 2].max() - t0) / 100.0)
        ph = (t[:, 3] >> 32)
        for code, nm in names.items():
            m = ph == code
            if not m.any():
                continue
            st = (t[m, 0] - t0) / 100.0
            we = (t[m, 1] - t0) / 100.0
            en = (t[m, 2] - t0) / 100.0
            per[nm]["first_start"].append(st.min())
            per[nm]["med_start"].append(np.median(st))
            per[nm]["med_mid"].append(np.median(we - st))
            per[nm]["last_mid"].append(we.max())
            per[nm]["last_end"].append(en.max())
            per[nm]["med_dur"].append(np.median(en - st))
    out = {nm: {key: round(float(np.median(v)), 2) for key, v in d.items() if v}
           for nm, d in per.items()}
    if args.dump:
        # the raw per-ticket records of the last call, for offline analysis
        np.save(args.dump, tr.cpu().numpy())
    return dict(metric="per-phase timeline of the persistent kernel, 8B-shaped, batch 1",
                unit="us", n_gpus=1, calls=ncalls, k=k, counts=counts,
                item_span_us=round(float(np.median(spans)), 2), phases=out)


def bench_copy(args):
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    ms = time_loop(lambda i: b.copy_(a), args.steps, args.warmup)
    return dict(metric="device copy", bytes_read=n, bytes_written=n, ms=round(ms, 4),
                GBps=round(2 * n / (ms * 1e-3) / 1e9, 1))


def other_workloads(args):
    """Short runs of the 70B-shaped batch step (1/2/4/8 tokens, 4-layer ring,
    50 timed steps per point), of the 32-layer 8B-shaped stack and of the
    14B-shaped layer (100 timed steps, no CPU leg), summarised
    beside the 8B line so that one default run reports every workload."""
    import copy
    import gc

    import torch
    gc.collect()
    torch.cuda.empty_cache()
    a = copy.copy(args)
    a.steps, a.warmup, a.ring = 50, 5, 4
    b = bench_batch(a)
    batch = {k: dict(us_per_step=v["us_per_step"], dense_us=v["dense_us"],
                     speedup_vs_dense=v["speedup_vs_dense"], union_frac=v["union_frac"])
             for k, v in b["batches"].items()}
    gc.collect()
    torch.cuda.empty_cache()
    st = bench_stack(args)
    tm = st["threshold_mode"]
    stack = dict(tokens_per_s=st["value"], us_per_layer=st["us_per_layer"],
                 dense_tokens_per_s=st["dense_tokens_per_s"],
                 speedup_vs_dense=st["speedup_vs_dense"], graph_tokens_per_s=st["graph_tokens_per_s"],
                 threshold_mask=dict(tokens_per_s=tm["tokens_per_s"], target_e=tm["target_e"],
                                     speedup_vs_dense=tm["speedup_vs_dense"]),
                 threshold_artifact=st["threshold_artifact"])
    gc.collect()
    torch.cuda.empty_cache()
    a = copy.copy(args)
    a.steps, a.warmup, a.no_cpu_baseline = 100, 10, True
    r = bench_single_layer(a, "14b")
    l14 = dict(steps=a.steps, us_per_layer=r["us_per_layer"], k=r["config"]["k"],
               hbm_frac=r["roofline"]["frac"], dense_us=r["dense"]["us_per_layer"],
               speedup_vs_dense=r["speedup_vs_dense"])
    gc.collect()
    torch.cuda.empty_cache()
    return {"14b": l14, "70b_batch": dict(steps=a.steps, ring_layers=a.ring, k=b["config"]["k"], batches=batch),
            "stack8b": stack}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="8b",
                    choices=["8b", "14b", "70b", "stack8b", "alpha", "copy", "timeline"])
    ap.add_argument("--sparsity", type=float, default=0.7)
    ap.add_argument("--repeats", type=int, default=5,
                    help="timed loops of --steps steps each; the median is reported")
    ap.add_argument("--ring", type=int, default=8)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="8b only: skip the 70B batch and 32-layer stack summaries appended "
                         "to the line")
    ap.add_argument("--dump", default=None,
                    help="timeline workload: save the last call's raw trace (.npy) here")
    ap.add_argument("--batch-gemv", choices=["valu", "mfma"], default="valu",
                    help="form of the batched up/gate step the layers are prepared with")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: one GPU only; --gpus {args.gpus} is not supported (the library "
              "runs one layer on one GPU; splitting a layer over GPUs is not implemented)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.workload in ("8b", "14b"):
        res = bench_single_layer(args, args.workload)
        if args.workload == "8b" and not args.no_other_workloads:
            res["other_workloads"] = other_workloads(args)
    elif args.workload == "70b":
        res = bench_batch(args)
    elif args.workload == "stack8b":
        res = bench_stack(args)
    elif args.workload == "alpha":
        res = bench_alpha(args)
    elif args.workload == "timeline":
        res = bench_timeline(args)
    else:
        res = bench_copy(args)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
