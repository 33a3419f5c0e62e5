"""The permutation fused into the expert GEMMs (fc1 forward and the fc1
weight gradient read row token_of[r] of x; no permuted copy xp), through the
C ABI: results bit-identical to the same products on xp = x[token_of], and
within the bf16 / fp32 tolerance of the oracle.

The pages' dispatchers eliminate permutation steps (German technical summary,
section 2 C; the hyper.ai article on Hybrid-EP); on one GPU that is the
gather moved into the operand loads.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_workloads import WORKLOADS, Workload, make_inputs, to_f64

from gpu_common import (TOL, announce, assert_close, bits, check_routing_and_map, host_inputs,
                        need_gpu, oracle_layer, run_layer)
from test_gpu_parity import full_size_sampled

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu(request):
    need_gpu()
    announce(request.node.nodeid)
    yield
    torch.cuda.synchronize()


GG = [
    Workload("gg_bf16", T=600, d=384, E=6, k=2, f=384),
    Workload("gg_f32", T=300, d=96, E=5, k=3, f=80, dtype="f32"),
    # empty experts, a few hot ones, tiles of one to many K stages
    Workload("gg_skew_bf16", T=2048, d=512, E=32, k=4, f=256, skew=True),
    # about 16 rows an expert: weight-gradient tiles of one K stage
    Workload("gg_short_k_bf16", T=512, d=256, E=64, k=2, f=256),
    # one expert: the weight gradient runs K = T over many stages
    Workload("gg_dense_bf16", T=900, d=256, E=1, k=1, f=384),
]


@pytest.mark.parametrize("wl", GG, ids=lambda w: w.name)
def test_gather_entry_points_equal_the_xp_products(wl):
    import token_routed_expert_amd as tre
    from token_routed_expert_amd import _native as N
    inp = make_inputs(wl, seed=4, device="cuda")
    T, d, f, P, E, k = wl.T, wl.d, wl.f, wl.P, wl.E, wl.k
    dt = inp["x"].dtype
    sh = tre.make_shape(T, d, E, k, f, 0, wl.dtype)
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    prob = torch.empty(T, k, dtype=torch.float32, device="cuda")
    tre.moe_route(inp["logits"], k, idx, prob)
    c = torch.empty(E, dtype=torch.int32, device="cuda")
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    r = torch.empty(T, k, dtype=torch.int32, device="cuda")
    tk = torch.empty(P, dtype=torch.int32, device="cuda")
    ws = torch.empty(tre.moe_workspace_bytes(sh, N.MOE_WS_PERMUTE), dtype=torch.uint8, device="cuda")
    tre.moe_permute(sh, None, idx, None, 1, c, off, r, tk, None, ws)      # the map alone
    xp = inp["x"][tk.long()].contiguous()
    dO = torch.randn(P, d, generator=torch.Generator(device="cuda").manual_seed(9),
                     device="cuda").to(dt)

    def outs():
        return dict(ab=torch.empty(P, 2 * f, dtype=dt, device="cuda"),
                    h=torch.empty(P, f, dtype=dt, device="cuda"),
                    o=torch.empty(P, d, dtype=dt, device="cuda"),
                    dab=torch.empty(P, 2 * f, dtype=dt, device="cuda"),
                    dXp=torch.empty(P, d, dtype=dt, device="cuda"),
                    dW1=torch.full_like(inp["W1"], 3.0), dW3=torch.full_like(inp["W3"], 3.0),
                    dW2=torch.full_like(inp["W2"], 3.0))

    W1, W3, W2 = inp["W1"], inp["W3"], inp["W2"]
    a, g = outs(), outs()
    tre.moe_grouped_gemm_fwd(sh, off, xp, W1, W3, W2, a["ab"], a["h"], a["o"])
    tre.moe_grouped_gemm_bwd(sh, off, xp, a["ab"], a["h"], dO, W1, W3, W2, a["dab"], a["dXp"],
                             a["dW1"], a["dW3"], a["dW2"])
    tre.moe_grouped_gemm_fwd_gather(sh, off, tk, inp["x"], W1, W3, W2, g["ab"], g["h"], g["o"])
    tre.moe_grouped_gemm_bwd_gather(sh, off, tk, inp["x"], g["ab"], g["h"], dO, W1, W3, W2,
                                    g["dab"], g["dXp"], g["dW1"], g["dW3"], g["dW2"])
    torch.cuda.synchronize()
    for n in a:
        assert np.array_equal(bits(g[n]), bits(a[n])), n
    # and the oracle, on the same inputs
    h = host_inputs(inp)
    ridx, _ = oracle.route(h["logits"], k)
    counts, offsets, row_of, token_of = oracle.permute_map(ridx, E)
    assert np.array_equal(tk.cpu().numpy(), token_of)
    xp_h = oracle.permute_rows(h["x"], token_of)
    ra, rb, rh, ro = oracle.experts_fwd(xp_h, offsets, h["W1"], h["W3"], h["W2"])
    tol = TOL[wl.dtype]
    assert_close("ab", to_f64(g["ab"]), np.concatenate([ra, rb], 1), tol)
    assert_close("o", to_f64(g["o"]), ro, tol)
    # weight gradients from the device's own dab (the fc1 wgrad's gathered operand is x)
    dab_h = to_f64(g["dab"])
    for e in range(E):
        R = slice(int(offsets[e]), int(offsets[e + 1]))
        ref1 = xp_h[R].T @ dab_h[R, :f]
        if R.stop > R.start:
            assert_close(f"dW1[{e}]", to_f64(g["dW1"][e]), ref1, tol)
        else:
            assert not g["dW1"][e].any() and not g["dW3"][e].any()


FUSED_SMALL = [
    WORKLOADS["tiny_f32"],
    Workload("tiny_bf16", T=256, d=128, E=8, k=2, f=128),
    Workload("multitile_bf16", T=1100, d=512, E=4, k=2, f=640),
    Workload("persistent_skew_bf16", T=2048, d=1024, E=32, k=4, f=768, skew=True),
    Workload("persistent_short_k_bf16", T=1024, d=1024, E=64, k=2, f=512),
    Workload("shared_bf16", T=300, d=256, E=8, k=2, f=128, f_shared=256),
    Workload("wide_e_bf16", T=512, d=128, E=256, k=8, f=128),
    Workload("dense_bf16", T=200, d=256, E=1, k=1, f=384),
    Workload("k_eq_E_bf16", T=64, d=128, E=4, k=4, f=128),
    Workload("one_token_bf16", T=1, d=128, E=8, k=2, f=128),
    Workload("ragged_skew_f32", T=333, d=96, E=16, k=3, f=80, dtype="f32", skew=True),
]

OUTS = ("topk_idx", "row_of", "token_of", "ab", "h", "o", "y", "dO", "dab", "dXp", "dX", "dW1",
        "dW3", "dW2")


@pytest.mark.parametrize("wl", FUSED_SMALL, ids=lambda w: w.name)
def test_layer_fused_permute_small(wl):
    """The layer with fused_permute: every output against the oracle, and
    bit-identical to the layer that writes xp."""
    inp = make_inputs(wl, seed=0, device="cuda")
    b = run_layer(wl, inp, fused_permute=True)
    assert "xp" not in b
    ref = run_layer(wl, inp)
    for n in OUTS + (("dWs1", "dWs3", "dWs2") if wl.f_shared else ()):
        assert np.array_equal(bits(b[n]), bits(ref[n])), n
    st, g = oracle_layer(wl, host_inputs(inp))
    check_routing_and_map(wl, b, inp, st)
    tol = TOL[wl.dtype]
    assert_close("y", to_f64(b["y"]), st["y"], tol)
    assert_close("dX", to_f64(b["dX"]), g["dX"], tol)
    for n in ("dW1", "dW3", "dW2"):
        assert_close(n, to_f64(b[n]), g[n], tol)


@pytest.mark.parametrize("me", [1, 2])
def test_layer_fused_permute_memory_efficient(me):
    """Fused permutation with the probabilities applied before W2 (and the
    SwiGLU recompute): bit-identical to the same layer with xp."""
    wl = Workload("fused_me_bf16", T=900, d=512, E=16, k=4, f=384, skew=True)
    inp = make_inputs(wl, seed=1, device="cuda")
    kw = dict(memory_efficient=me, router_grad=True)
    b = run_layer(wl, inp, fused_permute=True, **kw)
    ref = run_layer(wl, inp, **kw)
    for n in ("y", "dX", "dW1", "dW3", "dW2", "dprob", "dlogits", "aux_loss"):
        assert np.array_equal(bits(b[n]), bits(ref[n])), n


@pytest.mark.parametrize("wl", [WORKLOADS["qwen3_bf16"], WORKLOADS["deepseek_v3_bf16"]],
                         ids=lambda w: w.name)
def test_layer_fused_permute_full_size_sampled(wl):
    """The benchmark's shapes with the fused permutation: routing and map in
    full, y and dX on sampled tokens, dW on sampled experts, against the
    oracle."""
    full_size_sampled(wl, fused_permute=True)


def test_fused_permute_full_size_equals_xp_path():
    """Qwen3 shape: the fused layer's outputs equal the xp layer's bit for bit."""
    wl = WORKLOADS["qwen3_bf16"]
    inp = make_inputs(wl, seed=0, device="cuda")
    b = run_layer(wl, inp, fused_permute=True)
    outs = {n: b[n] for n in ("y", "dX", "dW1", "dW3", "dW2")}
    del b
    ref = run_layer(wl, inp)
    for n, t in outs.items():
        assert torch.equal(t.view(torch.int16), ref[n].view(torch.int16)), n
