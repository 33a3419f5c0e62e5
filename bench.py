#!/usr/bin/env python3
"""Benchmark of one GPU's routed-expert MoE layer (forward + backward).

One step is the whole path over one batch of synthetic tokens, as a sequence
of C-ABI calls on one stream: route -> permute -> grouped GEMM forward (fc1 +
SwiGLU, fc2) [+ shared expert] -> weighted combine -> combine backward
(scaled permute of dY) -> grouped GEMM backward (dgrad fc2 + SwiGLU backward,
dgrad fc1, wgrad fc2, wgrad fc1) [+ shared expert] -> un-permute of dXp.
With --router-grad the step also computes the load-balancing loss after the
permutation, and the combine backward also writes the probability gradient,
followed by the router backward (dlogits).
Inputs are resident in HBM before timing starts.

Prints one JSON line.  `value` is the layer's algorithmic GEMM TFLOP/s over
the whole step (18*d*f per routed row, plus the shared expert).  `roofline`
is for the grouped-GEMM kernel (all its launches in a step): algorithmic
flop / their summed duration, measured with HIP events on the launch stream.
Every step is timed on its own with HIP events (median and min reported);
a 512 MiB write between steps, outside the events, leaves nothing of the
previous step in L2 or the MALL.  `cpu_baseline` times the CPU oracle on a
bounded sample of the same workload (fp32 and fp64 runs of the same code).
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3, "e4m3": 5000.0, "mxfp8": 5000.0}
HBM_PEAK_GBS = 8000.0
FLUSH_BYTES = 512 << 20
METRIC = "MoE layer fwd+bwd TFLOPS/GPU & % MFMA peak; permute/combine HBM GB/s"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# The source file of each dtype's grouped-GEMM kernels.
GEMM_SOURCE = {"bf16": ["gemm_bf16.hip"], "f32": ["gemm_f32.hip"],
               "e4m3": ["gemm_fp8.hip"],
               "mxfp8": ["gemm_fp8.hip"]}


def kernel_sources_sha256(dtype: str) -> str:
    """Hash of the grouped-GEMM kernel sources of `dtype` and of every header of
    the library: a traffic record taken from hardware counters is valid only
    for the kernel sources it was taken on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "token_routed_expert_amd", "csrc")
    for path in sorted([os.path.join(csrc, n) for n in GEMM_SOURCE[dtype]] +
                       glob.glob(os.path.join(csrc, "*.h"))):
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def gemm_traffic(wl):
    """HBM bytes per step of the grouped-GEMM launches, from the counter record
    under profiles/ (FETCH_SIZE and WRITE_SIZE, each scaled by what the same
    counter reads for a device copy of known size), or None when there is no
    record or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_gemm_{wl.name}.txt")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.loads("".join(ln for ln in fh if not ln.startswith("#")))
    if rec.get("kernel_sources_sha256") != kernel_sources_sha256(wl.dtype):
        log(f"bench: {os.path.basename(path)} was taken on other kernel sources; traffic = null")
        return None
    return int(rec["hbm_bytes_per_step"])


def copy_calibration():
    """Two device copies of 1 GiB each, so that a counter run records what its
    FETCH_SIZE / WRITE_SIZE read for a known number of bytes."""
    import torch
    src = torch.empty(1 << 29, dtype=torch.int16, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


# Event marks of one step, in order; segment i runs from mark i to mark i + 1.
MARKS = ("start", "route", "permute", "aux_loss", "gemm_fwd", "combine", "combine_bwd",
         "route_bwd", "gemm_bwd", "unpermute", "quantize_weights")


def mfma_probe(iters: int = 4096):
    """The matrix-core rate and clock this GPU sustains under MFMAs alone
    (moe_probe_mfma), bf16 and e4m3: context for the roofline, whose peak
    stays the published figure."""
    import torch
    import token_routed_expert_amd as tre
    ticks = torch.zeros(2, dtype=torch.int64, device="cuda")
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    out = {"kernel": "8 independent MFMA chains per wavefront, 32 wavefronts per CU, no memory traffic"}
    for dt in ("bf16", "e4m3"):
        tre.moe_probe_mfma(dt, iters // 8, ticks, sink)     # warm-up
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        flops, khz = tre.moe_probe_mfma(dt, iters, ticks, sink)
        stop.record()
        torch.cuda.synchronize()
        sec = start.elapsed_time(stop) * 1e-3
        cyc, wall = (int(v) for v in ticks.cpu())
        out[f"{dt}_tflops"] = round(flops / sec / 1e12, 1)
        out[f"{dt}_frac_of_published"] = round(flops / sec / 1e12 / MFMA_PEAK_TFLOPS[dt], 4)
        out[f"{dt}_clock_ghz"] = round(cyc / (wall / (khz * 1e3)) / 1e9, 3) if wall > 0 else None
    return out


def router_grad_calls(wl, sh, b, ws_aux):
    """(aux loss after the permutation, combine backward with dprob, router
    backward, routing) as four callables: the routing is moe_route_aux, which
    also writes the loss's column sums, and the loss is then formed from them
    and the counts."""
    import token_routed_expert_amd as tre

    def route():
        tre.moe_route_aux(b["logits"], wl.k, b["topk_idx"], b["topk_prob"], ws_aux)

    def aux():
        tre.moe_aux_loss_final(ws_aux, wl.T, wl.E, wl.k, b["counts"], b["aux_alpha"], b["aux_loss"])

    def comb_bwd():
        tre.moe_combine_bwd(sh, b["dY"], b["o"], b["row_of"], b["topk_prob"], b["dO"], b["dprob"])

    def route_bwd():
        tre.moe_route_bwd(b["logits"], wl.k, b["topk_idx"], b["topk_prob"], b["dprob"], b["counts"],
                          b["aux_alpha"], 1.0, b["dlogits"])

    return aux, comb_bwd, route_bwd, route


def build_step(wl, inp, router_grad=False, memory_efficient=False, fused=False):
    import torch
    import token_routed_expert_amd as tre
    from token_routed_expert_amd import _native as N
    from token_routed_expert_amd.buffers import layer_buffers

    sh, b, wsf, wsb = layer_buffers(wl.T, wl.d, wl.E, wl.k, wl.f, wl.f_shared, wl.dtype, "cuda", inp,
                                    router_grad=router_grad, memory_efficient=memory_efficient,
                                    fused_permute=fused)
    rg = None
    if router_grad:
        base = tre.moe_workspace_bytes(sh, N.MOE_WS_LAYER_FWD)
        rg = router_grad_calls(wl, sh, b, wsf[base:])
    if wl.dtype in ("e4m3", "mxfp8"):
        if memory_efficient:
            return build_step_layer(wl, inp, sh, b, wsf, wsb)
        return build_step_e4m3(wl, inp, sh, b, wsf, wsb, rg)
    shared = None
    if wl.f_shared:
        fs = wl.f_shared
        sh_s = tre.make_shape(wl.T, wl.d, 1, 1, fs, 0, wl.dtype)
        off_s = torch.tensor([0, wl.T], dtype=torch.int32, device="cuda")
        shared = (sh_s, off_s)

    if memory_efficient:
        return build_step_rowscaled(wl, sh, b, wsf, wsb, shared, rg, memory_efficient)
    # the fused permutation builds the map alone; fc1 reads x through token_of
    xp = None if fused else b["xp"]

    def gemm_fwd():
        if fused:
            tre.moe_grouped_gemm_fwd_gather(sh, b["offsets"], b["token_of"], b["x"], b["W1"],
                                            b["W3"], b["W2"], b["ab"], b["h"], b["o"])
        else:
            tre.moe_grouped_gemm_fwd(sh, b["offsets"], xp, b["W1"], b["W3"], b["W2"], b["ab"],
                                     b["h"], b["o"])

    def gemm_bwd():
        if fused:
            tre.moe_grouped_gemm_bwd_gather(sh, b["offsets"], b["token_of"], b["x"], b["ab"],
                                            b["h"], b["dO"], b["W1"], b["W3"], b["W2"], b["dab"],
                                            b["dXp"], b["dW1"], b["dW3"], b["dW2"])
        else:
            tre.moe_grouped_gemm_bwd(sh, b["offsets"], xp, b["ab"], b["h"], b["dO"], b["W1"],
                                     b["W3"], b["W2"], b["dab"], b["dXp"], b["dW1"], b["dW3"],
                                     b["dW2"])

    def step(ev):
        ev["start"].record()
        if rg:
            rg[3]()
        else:
            tre.moe_route(b["logits"], wl.k, b["topk_idx"], b["topk_prob"])
        ev["route"].record()
        tre.moe_permute(sh, None if fused else b["x"], b["topk_idx"], None, 1, b["counts"],
                        b["offsets"], b["row_of"], b["token_of"], xp, wsf)
        ev["permute"].record()
        if rg:
            rg[0]()
        ev["aux_loss"].record()
        gemm_fwd()
        if shared:
            tre.moe_grouped_gemm_fwd(shared[0], shared[1], b["x"], b["Ws1"], b["Ws3"], b["Ws2"],
                                     b["s_ab"], b["s_h"], b["ys"])
        ev["gemm_fwd"].record()
        tre.moe_unpermute(sh, b["o"], b["row_of"], b["topk_prob"], b.get("ys"), b["y"])
        ev["combine"].record()
        if rg:
            rg[1]()
        else:
            tre.moe_permute(sh, b["dY"], None, b["topk_prob"], 0, None, None, b["row_of"], None,
                            b["dO"], None)
        ev["combine_bwd"].record()
        if rg:
            rg[2]()
        ev["route_bwd"].record()
        gemm_bwd()
        if shared:
            tre.moe_grouped_gemm_bwd(shared[0], shared[1], b["x"], b["s_ab"], b["s_h"], b["dY"],
                                     b["Ws1"], b["Ws3"], b["Ws2"], b["s_dab"], b["dXs"], b["dWs1"],
                                     b["dWs3"], b["dWs2"])
        ev["gemm_bwd"].record()
        tre.moe_unpermute(sh, b["dXp"], b["row_of"], None, b.get("dXs"), b["dX"])
        ev["unpermute"].record()
        ev["quantize_weights"].record()

    return step


def build_step_layer(wl, inp, sh, b, wsf, wsb):
    """The fp8 memory-efficient step through the layer entry points (its
    row-scaled fp8 products have no stand-alone calls): moe_layer_fwd, then
    moe_layer_bwd, then the weights' re-quantisation; the forward and backward
    are timed as wholes (gemm_fwd / gemm_bwd marks)."""
    import token_routed_expert_amd as tre
    from token_routed_expert_amd.buffers import requantize_weights

    wq = b["wmx"] if wl.dtype == "mxfp8" else b["wq"]
    W = (inp["W1"], inp["W3"], inp["W2"])

    def step(ev):
        ev["start"].record()
        for m in ("route", "permute", "aux_loss"):
            ev[m].record()
        tre.moe_layer_fwd(sh, b, wsf)
        for m in ("gemm_fwd", "combine", "combine_bwd", "route_bwd"):
            ev[m].record()
        tre.moe_layer_bwd(sh, b, wsb)
        for m in ("gemm_bwd", "unpermute"):
            ev[m].record()
        requantize_weights(wq, *W)
        ev["quantize_weights"].record()

    return step


def build_step_rowscaled(wl, sh, b, wsf, wsb, shared, rg, memory_efficient):
    """The memory-efficient step: probabilities applied to h before W2, an
    unweighted combine, the unscaled permutation of dY, and the row-scaled
    expert backward (which also yields dprob when the router gradient is on)."""
    import token_routed_expert_amd as tre

    def step(ev):
        ev["start"].record()
        if rg:
            rg[3]()
        else:
            tre.moe_route(b["logits"], wl.k, b["topk_idx"], b["topk_prob"])
        ev["route"].record()
        tre.moe_permute(sh, b["x"], b["topk_idx"], None, 1, b["counts"], b["offsets"], b["row_of"],
                        b["token_of"], b["xp"], wsf)
        tre.moe_row_probs(sh, b["row_of"], b["topk_prob"], b["row_prob"])
        ev["permute"].record()
        if rg:
            rg[0]()
        ev["aux_loss"].record()
        tre.moe_grouped_gemm_fwd_rowscaled(sh, b["offsets"], b["xp"], b["W1"], b["W3"], b["W2"],
                                           b["row_prob"], b["ab"], b["h"], b["o"])
        if shared:
            tre.moe_grouped_gemm_fwd(shared[0], shared[1], b["x"], b["Ws1"], b["Ws3"], b["Ws2"],
                                     b["s_ab"], b["s_h"], b["ys"])
        ev["gemm_fwd"].record()
        tre.moe_unpermute(sh, b["o"], b["row_of"], None, b.get("ys"), b["y"])
        ev["combine"].record()
        tre.moe_permute(sh, b["dY"], None, None, 0, None, None, b["row_of"], None, b["dO"], None)
        ev["combine_bwd"].record()
        ev["route_bwd"].record()
        tre.moe_grouped_gemm_bwd_rowscaled(sh, b["offsets"], b["xp"], b["ab"], b["h"], b["dO"],
                                           b["W1"], b["W3"], b["W2"], b["row_prob"], b["dab"],
                                           b["dXp"], b["dW1"], b["dW3"], b["dW2"],
                                           b["row_of"] if rg else None,
                                           b["dprob"] if rg else None, wsb,
                                           recompute_h=memory_efficient == 2)
        if shared:
            tre.moe_grouped_gemm_bwd(shared[0], shared[1], b["x"], b["s_ab"], b["s_h"], b["dY"],
                                     b["Ws1"], b["Ws3"], b["Ws2"], b["s_dab"], b["dXs"], b["dWs1"],
                                     b["dWs3"], b["dWs2"])
        if rg:
            rg[2]()
        ev["gemm_bwd"].record()
        tre.moe_unpermute(sh, b["dXp"], b["row_of"], None, b.get("dXs"), b["dX"])
        ev["unpermute"].record()
        ev["quantize_weights"].record()

    return step


def build_step_e4m3(wl, inp, sh, b, wsf, wsb, rg=None):
    """The fp8 step (e4m3 or MXFP8): the expert weights are re-quantised from
    their fp32 masters (as after an optimizer step), x is quantised (1 x 128
    blocks, MXFP8: 1 x 32) and its codes permuted; the GEMM calls quantise h,
    dO, [da|db] and the weight-gradient token blocks themselves."""
    import token_routed_expert_amd as tre
    from token_routed_expert_amd.buffers import requantize_weights
    from token_routed_expert_amd import _native as N

    mx = wl.dtype == "mxfp8"
    wq = b["wmx"] if mx else b["wq"]
    quant_rows = tre.moe_quantize_rows_mx if mx else tre.moe_quantize_rows
    permute8 = tre.moe_permute_mx if mx else tre.moe_permute_e4m3
    gemm_fwd8 = tre.moe_grouped_gemm_fwd_mx if mx else tre.moe_grouped_gemm_fwd_e4m3
    gemm_bwd8 = tre.moe_grouped_gemm_bwd_mx if mx else tre.moe_grouped_gemm_bwd_e4m3
    pws = tre.moe_workspace_bytes(sh, N.MOE_WS_PERMUTE)
    ws_perm = wsf[:max(256, pws)]
    ws_gf = wsf[pws:]
    W = (inp["W1"], inp["W3"], inp["W2"])

    def step(ev):
        ev["start"].record()
        if rg:
            rg[3]()
        else:
            tre.moe_route(b["logits"], wl.k, b["topk_idx"], b["topk_prob"])
        ev["route"].record()
        quant_rows(b["x"], b["xq"], b["xs"])
        permute8(sh, b["xq"], b["xs"], b["topk_idx"], 1, b["counts"], b["offsets"],
                             b["row_of"], b["token_of"], b["xpq"], b["xps"], ws_perm)
        ev["permute"].record()
        if rg:
            rg[0]()
        ev["aux_loss"].record()
        gemm_fwd8(sh, b["offsets"], b["xpq"], b["xps"], wq, b["ab"], b["h"],
                                      b["o"], ws_gf)
        ev["gemm_fwd"].record()
        tre.moe_unpermute(sh, b["o"], b["row_of"], b["topk_prob"], None, b["y"])
        ev["combine"].record()
        if rg:
            rg[1]()
        else:
            tre.moe_permute(sh, b["dY"], None, b["topk_prob"], 0, None, None, b["row_of"], None,
                            b["dO"], None)
        ev["combine_bwd"].record()
        if rg:
            rg[2]()
        ev["route_bwd"].record()
        gemm_bwd8(sh, b["offsets"], b["token_of"], b["x"], b["ab"], b["h"],
                                      b["dO"], wq, b["dab"], b["dXp"], b["dW1"], b["dW3"],
                                      b["dW2"], wsb)
        ev["gemm_bwd"].record()
        tre.moe_unpermute(sh, b["dXp"], b["row_of"], None, None, b["dX"])
        ev["unpermute"].record()
        requantize_weights(wq, *W)
        ev["quantize_weights"].record()

    return step


def mx_expert_fwd_bwd(oracle, X, dO, W1, W3, W2):
    """One expert's MXFP8 forward and backward with the oracle's functions."""
    import numpy as np
    one = np.array([0, X.shape[0]])
    Wq = [oracle.quant_mx_weights(W[None]) for W in (W1, W3, W2)]
    rowd = [oracle.dequant_mx_weights(q[0], q[1]) for q in Wq]
    cold = [oracle.dequant_mx_weights(q[2], q[3]) for q in Wq]
    xq, xs = oracle.quant_mx_rows(X)
    a, b = oracle.fc1_fwd_mx(xq, xs, one, cold[0], cold[1])
    h = oracle.silu(a) * b
    oracle.fc2_fwd_mx(h, one, cold[2])
    da, db = oracle.fc2_dgrad_mx(dO, a, b, one, rowd[2])
    dab = np.concatenate([da, db], axis=1)
    oracle.fc1_dgrad_mx(dab, one, rowd[0], rowd[1])
    oracle.wgrad_mx(h, dO, one)
    oracle.wgrad_mx(X, dab, one)


def e4m3_expert_fwd_bwd(oracle, X, dO, W1, W3, W2):
    """One expert's e4m3 forward and backward with the oracle's functions:
    weight tiles and activation rows quantised, products in fp64."""
    import numpy as np
    one = np.array([0, X.shape[0]])
    Wd = [oracle.dequant_expert_weights(*oracle.quant_expert_weights(W[None])) for W in (W1, W3, W2)]
    xq, xs = oracle.quant_rows(X)
    a, b = oracle.fc1_fwd_e4m3(xq, xs, one, Wd[0], Wd[1])
    h = oracle.silu(a) * b
    oracle.fc2_fwd_e4m3(h, one, Wd[2])
    da, db = oracle.fc2_dgrad_e4m3(dO, a, b, one, Wd[2])
    dab = np.concatenate([da, db], axis=1)
    oracle.fc1_dgrad_e4m3(dab, one, Wd[0], Wd[1])
    oracle.wgrad_e4m3(h, dO, one)
    oracle.wgrad_e4m3(X, dab, one)


def _oracle_sample(wl, inp, budget_s: float, dtype):
    """Routing and the permutation map of all T tokens, then the SwiGLU
    forward and backward of whole experts in index order until `budget_s`
    seconds of expert compute, with the oracle's functions on `dtype` arrays
    (np.float64: the correctness oracle; np.float32: the same code in fp32;
    fp8 workloads: the oracle's e4m3 / MXFP8 chain, fp64 only)."""
    import numpy as np
    import torch

    import oracle
    from moe_workloads import to_f64
    L = inp["logits"].cpu().numpy()
    t0 = time.perf_counter()
    idx, p = oracle.route(L, wl.k)
    counts, offsets, row_of, token_of = oracle.permute_map(idx, wl.E)
    t_route = time.perf_counter() - t0
    p_rows = p.reshape(-1)[np.argsort(row_of.reshape(-1))]
    flops = 0.0
    t_exp = 0.0
    n_exp = 0
    rows_done = 0
    for e in range(wl.E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        toks = torch.from_numpy(token_of[r0:r1]).to(inp["x"].device)
        X = to_f64(inp["x"][toks])
        dO = p_rows[r0:r1, None] * to_f64(inp["dY"][toks])
        if wl.dtype in ("e4m3", "mxfp8"):
            Wm = [inp[n][e].cpu().numpy() for n in ("W1", "W3", "W2")]
            t0 = time.perf_counter()
            (mx_expert_fwd_bwd if wl.dtype == "mxfp8" else e4m3_expert_fwd_bwd)(oracle, X, dO, *Wm)
            t_exp += time.perf_counter() - t0
        else:
            X, dO = X.astype(dtype), dO.astype(dtype)
            W1, W3, W2 = (to_f64(inp[n][e]).astype(dtype) for n in ("W1", "W3", "W2"))
            t0 = time.perf_counter()
            a, b, h, o = oracle.swiglu_fwd(X, W1, W3, W2)
            oracle.swiglu_bwd(X, a, b, h, dO, W1, W3, W2)
            t_exp += time.perf_counter() - t0
        flops += 18.0 * wl.d * wl.f * (r1 - r0)
        n_exp += 1
        rows_done += r1 - r0
        if t_exp >= budget_s:
            break
    return (round(flops / t_exp / 1e12, 6) if t_exp > 0 else None), t_route, n_exp, rows_done, t_exp


def cpu_baseline(wl, inp, budget_s: float):
    """The oracle, unchanged, on a bounded sample of the workload (see
    _oracle_sample): for bf16 / fp32 workloads the same code on fp32 arrays
    (the reported value) and on fp64 arrays (the correctness oracle as the
    tests run it); for fp8 workloads the fp64 e4m3 / MXFP8 chain."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    fp8 = wl.dtype in ("e4m3", "mxfp8")
    runs = [("fp64", np.float64)] if fp8 else [("fp32", np.float32), ("fp64", np.float64)]
    res = {}
    for name, dt in runs:
        res[name] = _oracle_sample(wl, inp, budget_s / len(runs), dt)
    head = runs[0][0]
    val, t_route, n_exp, rows, t_exp = res[head]
    out = {
        "value": val,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{head} NumPy oracle{f' ({wl.dtype} chain: quantise, dequantise, fp64 products)' if fp8 else ''}: "
                   f"route + permutation map of all {wl.T} tokens "
                   f"({t_route:.2f} s), then SwiGLU fwd+bwd of experts 0..{n_exp - 1} "
                   f"({rows} of {wl.P} routed rows) in {t_exp:.1f} s; host has "
                   f"{len(os.sched_getaffinity(0))} usable cores"),
    }
    if "fp64" in res and head != "fp64":
        v64, _, n64, r64, t64 = res["fp64"]
        out["fp64"] = {"value": v64, "unit": "TFLOP/s",
                       "sample": f"the same code on fp64 arrays: experts 0..{n64 - 1} ({r64} rows) in {t64:.1f} s"}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3_bf16")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mfma-probe", action="store_true",
                    help="skip the MFMA-only probe of the sustained matrix-core rate and clock")
    ap.add_argument("--router-grad", action="store_true",
                    help="also the load-balancing loss, dprob and the router backward (dlogits)")
    ap.add_argument("--memory-efficient", action="store_true",
                    help="probabilities applied before W2 (bf16 workloads)")
    ap.add_argument("--recompute-h", action="store_true",
                    help="with --memory-efficient: recompute p*h in the backward instead of keeping it")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run two 1 GiB device copies first (for hardware-counter runs)")
    ap.add_argument("--fused-permute", action="store_true",
                    help="bf16 / fp32: the permutation fused into fc1's operand loads (no xp)")
    ap.add_argument("--no-flush", action="store_true",
                    help="time the steps back to back, without the 512 MiB write between them")
    args = ap.parse_args()
    if args.gpus != 1:
        log(f"bench.py: this library is one GPU's share of the layer; --gpus {args.gpus} is not "
            "supported (run with --gpus 1)")
        sys.exit(2)

    import torch

    from moe_workloads import VARIANTS, WORKLOADS, make_inputs

    wl = {**WORKLOADS, **VARIANTS}[args.workload]
    if wl.dtype not in MFMA_PEAK_TFLOPS:
        log(f"bench.py: workload {wl.name} ({wl.dtype}) is not supported by this build")
        sys.exit(2)
    log(f"bench: {wl}")
    if args.copy_calibration:
        copy_calibration()
    inp = make_inputs(wl, seed=0, device="cuda")
    if args.memory_efficient and wl.dtype not in ("bf16", "e4m3", "mxfp8"):
        log("bench.py: --memory-efficient needs a bf16, e4m3 or mxfp8 workload")
        sys.exit(2)
    me = (2 if args.recompute_h else 1) if args.memory_efficient else 0
    if args.fused_permute and (wl.dtype not in ("bf16", "f32") or args.memory_efficient):
        log("bench.py: --fused-permute needs a bf16 or fp32 workload without --memory-efficient")
        sys.exit(2)
    step = build_step(wl, inp, args.router_grad, me, args.fused_permute)

    def marks():
        return {m: torch.cuda.Event(enable_timing=True) for m in MARKS}

    ev = [marks() for _ in range(args.steps)]
    warm = marks()
    # a write larger than the 256 MB last-level cache between timed steps, so
    # that no step reads what the previous one left in L2 / MALL; it runs
    # outside each step's events
    flush = None if args.no_flush else torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    for i in range(args.warmup):
        if flush is not None:
            flush.fill_(i & 0x7f)
        step(warm)
    torch.cuda.synchronize()
    log(f"bench: warmup done ({args.warmup} steps)")
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        if flush is not None:
            flush.fill_(i & 0x7f)
        step(ev[i])
    stop.record()
    torch.cuda.synchronize()
    per_step = sorted(e[MARKS[0]].elapsed_time(e[MARKS[-1]]) for e in ev)
    ms_step = statistics.median(per_step)
    ms_wall = start.elapsed_time(stop) / args.steps          # incl. the flushes
    log(f"bench: timed {args.steps} steps, median {ms_step:.3f} ms/step, min {per_step[0]:.3f}, "
        f"{ms_wall:.3f} ms per step incl. the flush")

    def seg(i):
        return statistics.median(e[MARKS[i]].elapsed_time(e[MARKS[i + 1]]) for e in ev)

    (t_route, t_perm, t_aux, t_gf, t_comb, t_permb, t_rbwd, t_gb, t_unp,
     t_wq) = (seg(i) for i in range(len(MARKS) - 1))
    s = 4 if wl.dtype == "f32" else 2
    flops = wl.flops_fwd_bwd()
    # the grouped-GEMM launches of one step (forward and backward segments),
    # median over the timed steps
    gemm_ms = statistics.median(e["aux_loss"].elapsed_time(e["gemm_fwd"]) +
                                e["route_bwd"].elapsed_time(e["gemm_bwd"]) for e in ev)
    peak = MFMA_PEAK_TFLOPS[wl.dtype]
    achieved = flops / (gemm_ms * 1e-3) / 1e12
    move_bytes = (wl.T * wl.d + wl.P * wl.d) * s          # bf16 / fp32 rows in and out
    perm_bytes = move_bytes
    if wl.dtype in ("e4m3", "mxfp8"):
        # quantise x (read bf16, write codes + scales), then move codes + scales
        # (fp32 per 128 values or one byte per 32: the same count)
        qx = wl.T * wl.d * (2 + 1) + wl.T * (wl.d // 128) * 4
        perm_bytes = qx + (wl.T + wl.P) * (wl.d + (wl.d // 128) * 4)
    perm_gbs = (perm_bytes + 16 * wl.P) / (t_perm * 1e-3) / 1e9
    comb_gbs = (move_bytes + 8 * wl.P + (wl.T * wl.d * s if wl.f_shared else 0)) / (t_comb * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(flops / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) logits and activations, N(0,1/fan_in) weights)",
        "config": {"workload": wl.name, "T": wl.T, "d": wl.d, "E": wl.E, "k": wl.k, "f": wl.f,
                   "f_shared": wl.f_shared},
        "roofline": {"kernel": ("grouped GEMM (all fwd+bwd launches of a step)"
                                if wl.dtype not in ("e4m3", "mxfp8")
                                else f"{wl.dtype} grouped-GEMM calls (fwd+bwd, with the h, dO, dab and "
                                     "token-block quantisations they run)"), "bound": "mfma",
                     "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": gemm_traffic(wl),
                     "traffic_unit": "bytes per step (all grouped-GEMM launches)"},
        "breakdown_ms": {"route": round(t_route, 4), "permute": round(t_perm, 4),
                         "gemm_fwd": round(t_gf, 4), "combine": round(t_comb, 4),
                         "combine_bwd_permute": round(t_permb, 4), "gemm_bwd": round(t_gb, 4),
                         "unpermute": round(t_unp, 4),
                         "quantize_weights": round(t_wq, 4)},
        "hbm": {"permute_GBps": round(perm_gbs, 1), "combine_GBps": round(comb_gbs, 1),
                "permute_frac": round(perm_gbs / HBM_PEAK_GBS, 4),
                "combine_frac": round(comb_gbs / HBM_PEAK_GBS, 4), "peak_GBps": HBM_PEAK_GBS,
                "permute_us_per_call": round(t_perm * 1e3, 1),
                "combine_us_per_call": round(t_comb * 1e3, 1)},
        "timing": {"per_step": "HIP events around each step; median over the timed steps",
                   "median_ms": round(ms_step, 4), "min_ms": round(per_step[0], 4),
                   "mean_ms": round(statistics.fmean(per_step), 4),
                   "wall_ms_per_step_incl_flush": round(ms_wall, 4),
                   "flush_between_steps_bytes": 0 if args.no_flush else FLUSH_BYTES},
    }
    if args.fused_permute:
        # the permute segment builds the map alone (no rows move): no GB/s figure
        out["config"]["fused_permute"] = True
        out["hbm"].update(permute_GBps=None, permute_frac=None,
                          permute_note="map only: fc1 reads x rows through token_of")
        # the gathered fc1 kernels run here; the counters were taken on the plain ones
        out["roofline"]["traffic"] = None
    if args.memory_efficient:
        out["config"]["memory_efficient"] = "recompute_h" if me == 2 else True
        if wl.dtype in ("e4m3", "mxfp8"):
            # timed through moe_layer_fwd / moe_layer_bwd: the "GEMM" figure is the whole layer's
            out["roofline"]["kernel"] = (f"{wl.dtype} layer calls (moe_layer_fwd + moe_layer_bwd, "
                                         "all steps)")
            # permute and combine run inside the layer calls: no separate times
            out["hbm"] = None
        # the row-scaled GEMM variants run here; the counters were taken on the plain ones
        out["roofline"]["traffic"] = None
        out["breakdown_ms"]["combine_bwd_permute"] = round(t_permb, 4)
    if args.router_grad and args.memory_efficient:
        # dprob comes out of the expert backward; the router backward is timed with it
        out["config"]["router_grad"] = True
        out["breakdown_ms"].update(aux_loss=round(t_aux, 4))
    elif args.router_grad:
        # combine backward with dprob: read dY once and the k rows of o, write dO
        cb_bytes = (wl.T * wl.d + 2 * wl.P * wl.d) * s + 12 * wl.P
        cb_gbs = cb_bytes / (t_permb * 1e-3) / 1e9
        del out["breakdown_ms"]["combine_bwd_permute"]
        out["config"]["router_grad"] = True
        out["breakdown_ms"].update(aux_loss=round(t_aux, 4), combine_bwd=round(t_permb, 4),
                                   route_bwd=round(t_rbwd, 4))
        out["hbm"].update(combine_bwd_GBps=round(cb_gbs, 1),
                          combine_bwd_frac=round(cb_gbs / HBM_PEAK_GBS, 4))
    if not args.no_mfma_probe:
        out["mfma_probe"] = mfma_probe()
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
