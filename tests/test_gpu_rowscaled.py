"""Memory-efficient permutation (probabilities applied before W2) on the GPU
against the oracle, through the C ABI.

The layer's results are the plain layer's (the oracle is unchanged: p (h W2)
= (p h) W2 by linearity), within the bf16 tolerance of the other layer tests;
h and o now hold p-scaled rows.  The probability gradient comes from the fc2
data-gradient epilogue as <silu(a) b, dO W2^T> with a, b the stored bf16
pre-activations, so it carries bf16 rounding of h:
|dprob - exact| <= 2e-2 * sum_f |h_f (dY W2^T)_f|.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_workloads import WORKLOADS, Workload, make_inputs, to_f64

from gpu_common import TOL, announce, assert_close, host_inputs, need_gpu, oracle_layer, run_layer
from test_gpu_parity import SMALL, check_routing_and_map, full_size_sampled

pytestmark = pytest.mark.gpu
BF16 = [w for w in SMALL if w.dtype == "bf16"]


@pytest.fixture(autouse=True)
def _gpu(request):
    need_gpu()
    announce(request.node.nodeid)
    yield
    torch.cuda.synchronize()


def permuted_probs(st):
    """p of every permuted row (the oracle's map)."""
    return st["p"].reshape(-1)[np.argsort(st["row_of"].reshape(-1))]


def check_dprob(wl, st, h, dp):
    """|dp - exact| <= 2e-2 * sum_f |h_f (dY W2^T)_f| for every (t, j)."""
    dp_ref = oracle.combine_dprob(h["dY"], st["o"], st["row_of"])
    toks = np.repeat(np.arange(wl.T), wl.k)
    idx = st["idx"].reshape(-1)
    dhp = np.empty((wl.T * wl.k, wl.f))
    for e in range(wl.E):
        sel = idx == e
        if sel.any():
            dhp[sel] = h["dY"][toks[sel]] @ h["W2"][e].T
    hh = st["h"][st["row_of"].reshape(-1)]
    mag = np.abs(hh * dhp).sum(1).reshape(wl.T, wl.k)
    err = np.abs(dp - dp_ref)
    assert (err <= 2e-2 * mag).all(), f"dprob: worst |err|/sum|terms| {(err / mag).max():.3e}"


@pytest.mark.parametrize("mode", [1, 2], ids=["keep_h", "recompute_h"])
@pytest.mark.parametrize("wl", BF16, ids=lambda w: w.name)
def test_layer_memory_efficient(wl, mode):
    inp = make_inputs(wl, seed=0, device="cuda")
    b = run_layer(wl, inp, memory_efficient=mode)
    h = host_inputs(inp)
    st, g = oracle_layer(wl, h)
    check_routing_and_map(wl, b, inp, st)
    tol = TOL[wl.dtype]
    pr = permuted_probs(st)
    assert np.abs(b["row_prob"].cpu().numpy() - pr).max() <= 1e-4 * pr.max()
    assert_close("ab", to_f64(b["ab"]), np.concatenate([st["a"], st["b"]], 1), tol)
    assert_close("p h", to_f64(b["h"]), pr[:, None] * st["h"], tol)
    assert_close("p o", to_f64(b["o"]), pr[:, None] * st["o"], tol)
    assert_close("y", to_f64(b["y"]), st["y"], tol)
    assert_close("dXp", to_f64(b["dXp"]), g["dXp"], tol)
    assert_close("dX", to_f64(b["dX"]), g["dX"], tol)
    for n in ("dW1", "dW3", "dW2") + (("dWs1", "dWs3", "dWs2") if wl.f_shared else ()):
        assert_close(n, to_f64(b[n]), g[n], tol)
    for e in np.nonzero(st["counts"] == 0)[0]:
        assert not b["dW1"][e].any() and not b["dW3"][e].any() and not b["dW2"][e].any()


@pytest.mark.parametrize("mode", [1, 2], ids=["keep_h", "recompute_h"])
@pytest.mark.parametrize("wl", [Workload("me_rg_bf16", T=777, d=256, E=16, k=4, f=384),
                                Workload("me_rg_skew_bf16", T=500, d=384, E=16, k=4, f=256,
                                         skew=True)],
                         ids=lambda w: w.name)
def test_memory_efficient_router_grad(wl, mode):
    """dprob from the fc2 dgrad epilogue, dlogits and the loss; the backward
    does not read o, nor h when it recomputes it (poisoned between forward
    and backward)."""
    import token_routed_expert_amd as tre
    from token_routed_expert_amd.buffers import layer_buffers
    inp = make_inputs(wl, seed=4, device="cuda")
    sh, b, wsf, wsb = layer_buffers(wl.T, wl.d, wl.E, wl.k, wl.f, 0, "bf16", "cuda", inp,
                                    router_grad=True, aux_alpha=0.01, memory_efficient=mode)
    tre.moe_layer_fwd(sh, b, wsf)
    b["o"].fill_(float("nan"))
    if mode == 2:
        b["h"].fill_(float("nan"))
    tre.moe_layer_bwd(sh, b, wsb)
    torch.cuda.synchronize()
    h = host_inputs(inp)
    st, g = oracle_layer(wl, h)
    tol = TOL["bf16"]
    for n in ("dX", "dW1", "dW3", "dW2"):
        assert torch.isfinite(b[n]).all(), n
        assert_close(n, to_f64(b[n]), g[n], tol)
    dp = b["dprob"].cpu().numpy().astype(np.float64)
    check_dprob(wl, st, h, dp)
    idx = st["idx"]
    ref = oracle.router_bwd(dp, st["p"], idx, wl.E) + oracle.aux_loss(h["logits"], st["counts"],
                                                                      wl.k, 0.01)[1]
    assert_close("dlogits", b["dlogits"].cpu().numpy().astype(np.float64), ref, 1e-4)
    ref_loss = oracle.aux_loss(h["logits"], st["counts"], wl.k, 0.01)[0]
    assert abs(float(b["aux_loss"].item()) - ref_loss) <= 5e-5 * ref_loss


@pytest.mark.parametrize("mode", [1, 2], ids=["keep_h", "recompute_h"])
def test_memory_efficient_is_deterministic(mode):
    wl = Workload("me_det_bf16", T=900, d=256, E=16, k=4, f=256)
    inp = make_inputs(wl, seed=2, device="cuda")
    b1 = run_layer(wl, inp, memory_efficient=mode, router_grad=True)
    b2 = run_layer(wl, inp, memory_efficient=mode, router_grad=True)
    for n in ("y", "dX", "dW1", "dW3", "dW2", "h", "o", "dprob", "dlogits"):
        assert torch.equal(b1[n], b2[n]), n


def test_rowscaled_entry_points():
    """moe_row_probs, the row-scaled GEMM forward and backward (dprob_rows)
    called directly, against the plain entry points' results scaled by p."""
    import token_routed_expert_amd as tre
    from token_routed_expert_amd import _native as N
    wl = Workload("me_ep_bf16", T=600, d=256, E=8, k=2, f=256)
    inp = make_inputs(wl, seed=5, device="cuda")
    b = run_layer(wl, inp)                      # plain layer: routing, map, xp, ab, h, o
    sh = tre.make_shape(wl.T, wl.d, wl.E, wl.k, wl.f, 0, "bf16")
    P = wl.P
    rp = torch.empty(P, device="cuda")
    tre.moe_row_probs(sh, b["row_of"], b["topk_prob"], rp)
    h = host_inputs(inp)
    st, g = oracle_layer(wl, h)
    pr = permuted_probs(st)
    assert np.abs(rp.cpu().numpy() - pr).max() <= 1e-4 * pr.max()
    ab = torch.empty_like(b["ab"]); hs = torch.empty_like(b["h"]); os_ = torch.empty_like(b["o"])
    tre.moe_grouped_gemm_fwd_rowscaled(sh, b["offsets"], b["xp"], inp["W1"], inp["W3"], inp["W2"],
                                       rp, ab, hs, os_)
    assert torch.equal(ab, b["ab"])             # the pre-activations are not scaled
    assert_close("p h", to_f64(hs), pr[:, None] * st["h"], TOL["bf16"])
    assert_close("p o", to_f64(os_), pr[:, None] * st["o"], TOL["bf16"])
    dO = torch.empty_like(b["dO"])
    tre.moe_permute(sh, inp["dY"], None, None, 0, None, None, b["row_of"], None, dO, None)
    out = {n: torch.empty_like(b[n]) for n in ("dab", "dXp", "dW1", "dW3", "dW2")}
    dpr = torch.empty(P, device="cuda")
    ws = torch.empty(tre.moe_workspace_bytes(sh, N.MOE_WS_GEMM_BWD_ROWSCALED), dtype=torch.uint8,
                     device="cuda")
    tre.moe_grouped_gemm_bwd_rowscaled(sh, b["offsets"], b["xp"], ab, hs, dO, inp["W1"], inp["W3"],
                                       inp["W2"], rp, out["dab"], out["dXp"], out["dW1"],
                                       out["dW3"], out["dW2"], None, dpr, ws)
    for n in ("dXp", "dW1", "dW3", "dW2"):
        assert_close(n, to_f64(out[n]), g[n], TOL["bf16"])
    check_dprob(wl, st, h, dpr.cpu().numpy().astype(np.float64)[st["row_of"]])
    dtk = torch.empty(wl.T, wl.k, device="cuda")     # the [T][k] form through row_of
    tre.moe_grouped_gemm_bwd_rowscaled(sh, b["offsets"], b["xp"], ab, hs, dO, inp["W1"], inp["W3"],
                                       inp["W2"], rp, out["dab"], out["dXp"], out["dW1"],
                                       out["dW3"], out["dW2"], b["row_of"], dtk, ws)
    assert torch.equal(dtk, dpr[b["row_of"].long()])
    # recompute_h: h is refilled from ab before fc2 wgrad reads it
    out2 = {n: torch.empty_like(b[n]) for n in ("dab", "dXp", "dW1", "dW3", "dW2")}
    hr = torch.full_like(hs, float("nan"))
    tre.moe_grouped_gemm_bwd_rowscaled(sh, b["offsets"], b["xp"], ab, hr, dO, inp["W1"], inp["W3"],
                                       inp["W2"], rp, out2["dab"], out2["dXp"], out2["dW1"],
                                       out2["dW3"], out2["dW2"], None, None, ws, recompute_h=True)
    assert_close("recomputed p h", to_f64(hr), pr[:, None] * st["h"], TOL["bf16"])
    for n in ("dab", "dXp", "dW1", "dW3"):
        assert torch.equal(out2[n], out[n]), n          # h enters only fc2 wgrad
    assert_close("dW2 (recomputed h)", to_f64(out2["dW2"]), g["dW2"], TOL["bf16"])


@pytest.mark.parametrize("wl", [WORKLOADS["qwen3_bf16"], WORKLOADS["deepseek_v3_bf16"]],
                         ids=lambda w: w.name)
def test_memory_efficient_full_size_sampled(wl):
    full_size_sampled(wl, memory_efficient=2)


# ---------------------------------------------------------------- e4m3 and MXFP8 layers
def fp8_ops(dtype):
    """The oracle's product functions of one fp8 recipe and the dequantised
    weights (forward orientation, data-gradient orientation) of the device's
    quantised weights, which the quantiser tests prove equal to the oracle's."""
    if dtype == "e4m3":
        return (oracle.quant_rows, oracle.dequant_rows, oracle.fc1_fwd_e4m3, oracle.fc2_fwd_e4m3,
                oracle.fc2_dgrad_e4m3, oracle.fc1_dgrad_e4m3, oracle.wgrad_e4m3)
    return (oracle.quant_mx_rows, oracle.dequant_mx_rows, oracle.fc1_fwd_mx, oracle.fc2_fwd_mx,
            oracle.fc2_dgrad_mx, oracle.fc1_dgrad_mx, oracle.wgrad_mx)


def fp8_weights(dtype, inp):
    fwd, bwd = {}, {}
    for n in ("W1", "W3", "W2"):
        W = inp[n].cpu().numpy()
        if dtype == "e4m3":
            q, s_ = oracle.quant_expert_weights(W)
            fwd[n] = bwd[n] = oracle.dequant_expert_weights(q, s_)
        else:
            q, s_, qt, st_ = oracle.quant_mx_weights(W)
            bwd[n] = oracle.dequant_mx_weights(q, s_)
            fwd[n] = oracle.dequant_mx_weights(qt, st_)
    return fwd, bwd


FP8_ME = [Workload("me_e4m3", T=700, d=384, E=16, k=4, f=256, dtype="e4m3", skew=True),
          Workload("me_mxfp8", T=700, d=384, E=16, k=4, f=256, dtype="mxfp8", skew=True),
          Workload("me_mxfp8_ragged", T=301, d=256, E=8, k=2, f=384, dtype="mxfp8")]


@pytest.mark.parametrize("mode", [1, 2], ids=["keep_h", "recompute_h"])
@pytest.mark.parametrize("wl", FP8_ME, ids=lambda w: w.name)
def test_fp8_layer_memory_efficient(wl, mode):
    """Each product of the memory-efficient fp8 layer against the oracle on the
    device's own stored intermediates: h = p silu(a) b, o = Q(h) W2, y the
    unweighted combine, dO the unscaled permutation of dY, [da|db] p times the
    SwiGLU backward of Q(dO) W2^T, dXp, dX, the weight gradients, and dprob
    = <silu(a) b, Q(dO) W2^T> (o poisoned between forward and backward)."""
    import token_routed_expert_amd as tre
    from token_routed_expert_amd.buffers import layer_buffers
    from test_gpu_e4m3 import TOL8
    inp = make_inputs(wl, seed=6, device="cuda")
    sh, b, wsf, wsb = layer_buffers(wl.T, wl.d, wl.E, wl.k, wl.f, 0, wl.dtype, "cuda", inp,
                                    router_grad=True, aux_alpha=0.01, memory_efficient=mode)
    tre.moe_layer_fwd(sh, b, wsf)
    h_fwd = b["h"].clone()
    b["o_saved"] = b["o"].clone()
    b["o"].fill_(float("nan"))
    if mode == 2:
        b["h"].fill_(float("nan"))
    tre.moe_layer_bwd(sh, b, wsb)
    torch.cuda.synchronize()
    quant_rows, dequant_rows, fc1, fc2, fc2_dgrad, fc1_dgrad, wgrad = fp8_ops(wl.dtype)
    L = inp["logits"].cpu().numpy()
    idx, p = oracle.route(L, wl.k)
    counts, off, row_of, token_of = oracle.permute_map(idx, wl.E)
    assert np.array_equal(b["row_of"].cpu().numpy(), row_of)
    pr = p.reshape(-1)[np.argsort(row_of.reshape(-1))]
    Wf, Wb = fp8_weights(wl.dtype, inp)
    f = wl.f
    xpq = b["xpq"].cpu().numpy()
    xps = b["xps"].cpu().numpy()
    a_r, b_r = fc1(xpq, xps, off, Wf["W1"], Wf["W3"])
    ab = to_f64(b["ab"]); a_g, b_g = ab[:, :f], ab[:, f:]
    assert_close("a", a_g, a_r, TOL8)
    h_g = to_f64(h_fwd)
    assert_close("p h", h_g, pr[:, None] * oracle.silu(a_r) * b_r, TOL8)
    o_g = to_f64(b["o_saved"])
    assert_close("o", o_g, fc2(h_g, off, Wf["W2"]), TOL8)
    assert_close("y", to_f64(b["y"]), oracle.combine(o_g, row_of), TOL8)
    assert torch.equal(b["dO"], inp["dY"][torch.from_numpy(token_of).cuda()])
    dO_g = to_f64(b["dO"])
    da_r, db_r = fc2_dgrad(dO_g, a_g, b_g, off, Wb["W2"])
    dab_g = to_f64(b["dab"])
    assert_close("da", dab_g[:, :f], pr[:, None] * da_r, TOL8)
    assert_close("db", dab_g[:, f:], pr[:, None] * db_r, TOL8)
    assert_close("dXp", to_f64(b["dXp"]), fc1_dgrad(dab_g, off, Wb["W1"], Wb["W3"]), TOL8)
    assert_close("dX", to_f64(b["dX"]), oracle.combine(to_f64(b["dXp"]), row_of), TOL8)
    h_w = to_f64(b["h"]) if mode == 2 else h_g            # the h the fc2 weight gradient read
    if mode == 2:
        assert_close("recomputed p h", h_w, pr[:, None] * oracle.silu(a_g) * b_g, TOL8)
    assert_close("dW2", to_f64(b["dW2"]), wgrad(h_w, dO_g, off), TOL8)
    dW13 = wgrad(to_f64(inp["x"])[token_of], dab_g, off)
    assert_close("dW1", to_f64(b["dW1"]), dW13[:, :, :f], TOL8)
    assert_close("dW3", to_f64(b["dW3"]), dW13[:, :, f:], TOL8)
    # dprob = <silu(a) b, Q(dO) W2^T> from the stored a, b
    G = dequant_rows(*quant_rows(dO_g))
    dH = np.zeros((wl.P, f))
    for e in range(wl.E):
        R = slice(int(off[e]), int(off[e + 1]))
        dH[R] = G[R] @ Wb["W2"][e].T
    hh = oracle.silu(a_g) * b_g
    dp_rows = (hh * dH).sum(1)
    mag = np.abs(hh * dH).sum(1)
    dp = b["dprob"].cpu().numpy().astype(np.float64)
    err = np.abs(dp - dp_rows[row_of])
    assert (err <= 1e-4 * mag[row_of] + 1e-30).all(), f"dprob worst {(err / mag[row_of]).max():.3e}"
    ref = oracle.router_bwd(dp, p, idx, wl.E) + oracle.aux_loss(L, counts, wl.k, 0.01)[1]
    assert_close("dlogits", b["dlogits"].cpu().numpy().astype(np.float64), ref, 1e-4)
