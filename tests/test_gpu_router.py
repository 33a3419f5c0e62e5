"""Router gradient and load-balancing loss on the GPU vs the oracle, through the C ABI.

Tolerances follow from the fp32 arithmetic of the kernels:
* dprob is an fp32 dot product of d terms accumulated in at most 72 sequential
  roundings (per-thread chain, then the wavefront and block trees), so
  |gpu - exact| <= 72 * 2**-24 * sum_i |dY_i o_i| < 1e-5 * sum_i |dY_i o_i|;
* dlogits and the loss are short fp32 expressions of softmax values (hardware
  exp, a handful of roundings, sums of positive terms over at most a few
  hundred partials): row-relative 1e-4 against the oracle on its own fp64
  probabilities (the Jacobian is ill-conditioned in rounded probabilities
  whose sum is not exactly one), loss relative 5e-5;
* dO equals moe_permute's scaled rows bit for bit (same product, same rounding).
"""
import numpy as np
import pytest
import torch

import oracle
from moe_workloads import WORKLOADS, Workload, make_inputs, skew_bias, to_f64

from gpu_common import TOL, announce, assert_close, bits, need_gpu, run_layer

pytestmark = pytest.mark.gpu

DOT_TOL = 1e-5
ROW_TOL = 1e-4
LOSS_TOL = 5e-5


@pytest.fixture(autouse=True)
def _gpu(request):
    need_gpu()
    announce(request.node.nodeid)
    yield
    torch.cuda.synchronize()


def routed(T, E, k, seed, skew=False):
    """Seeded fp32 logits, their GPU routing (idx, prob), the oracle's counts
    and row map, and the oracle's fp64 probabilities."""
    import token_routed_expert_amd as tre
    g = torch.Generator().manual_seed(seed)
    L = torch.randn(T, E, generator=g)
    if skew:
        L += skew_bias(Workload("skew", T=T, d=128, E=E, k=k, f=128), seed)[None, :]
    Lg = L.cuda()
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    prob = torch.empty(T, k, dtype=torch.float32, device="cuda")
    tre.moe_route(Lg, k, idx, prob)
    ridx, rp = oracle.route(L.numpy(), k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    counts, offsets, row_of, token_of = oracle.permute_map(ridx, E)
    return L, Lg, idx, prob, counts, row_of.astype(np.int32), rp


def check_dot(name, got, dY, o, row_of):
    """|got - exact| <= DOT_TOL * sum |dY_i o_i| elementwise (fp32 dot bound)."""
    ref = oracle.combine_dprob(dY, o, row_of)
    mag = oracle.combine_dprob(np.abs(dY), np.abs(o), row_of)
    err = np.abs(got - ref)
    assert (err <= DOT_TOL * mag + 1e-30).all(), \
        f"{name}: worst |err|/sum|terms| = {(err / np.maximum(mag, 1e-30)).max():.3e}"


# ---------------------------------------------------------------- combine backward
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T,E,k,d", [(1, 4, 2, 64), (257, 8, 2, 128), (1000, 128, 8, 256),
                                     (300, 16, 16, 32), (64, 8, 1, 7168), (33, 8, 3, 8192),
                                     (17, 4, 2, 16384)])
def test_combine_bwd(dtype, T, E, k, d):
    import token_routed_expert_amd as tre
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    _, _, idx, prob, counts, row_of, _ = routed(T, E, k, seed=T + d)
    P = T * k
    g = torch.Generator().manual_seed(d)
    dY = torch.randn(T, d, generator=g).to(dt)
    o = torch.randn(P, d, generator=g).to(dt)
    sh = tre.make_shape(T, d, E, k, 128, 0, dtype)
    ro = torch.from_numpy(row_of).cuda()
    dO = torch.full((P, d), float("nan"), dtype=dt, device="cuda")
    dprob = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
    if dtype == "f32" and d == 16384:
        # fp32 rows of 16384 values (64 KiB) exceed what one block keeps of
        # dY[t]: the call is refused before anything is launched
        with pytest.raises(tre.MoeError, match="MOE_ERR_UNSUPPORTED"):
            tre.moe_combine_bwd(sh, dY.cuda(), o.cuda(), ro, prob, dO, dprob)
        return
    tre.moe_combine_bwd(sh, dY.cuda(), o.cuda(), ro, prob, dO, dprob)
    # dO: exactly the scaled permutation
    dO_ref = torch.empty_like(dO)
    tre.moe_permute(sh, dY.cuda(), None, prob, 0, None, None, ro, None, dO_ref, None)
    assert np.array_equal(bits(dO), bits(dO_ref))
    check_dot("dprob", dprob.cpu().numpy().astype(np.float64), to_f64(dY), to_f64(o), row_of)


def test_combine_bwd_deterministic():
    import token_routed_expert_amd as tre
    T, E, k, d = 700, 64, 8, 4096
    _, _, idx, prob, counts, row_of, _ = routed(T, E, k, seed=5)
    g = torch.Generator().manual_seed(6)
    dY = torch.randn(T, d, generator=g).to(torch.bfloat16).cuda()
    o = torch.randn(T * k, d, generator=g).to(torch.bfloat16).cuda()
    sh = tre.make_shape(T, d, E, k, 128, 0, "bf16")
    ro = torch.from_numpy(row_of).cuda()
    out = []
    for _ in range(2):
        dO = torch.empty(T * k, d, dtype=torch.bfloat16, device="cuda")
        dp = torch.empty(T, k, dtype=torch.float32, device="cuda")
        tre.moe_combine_bwd(sh, dY, o, ro, prob, dO, dp)
        out.append((dO, dp))
    assert torch.equal(out[0][0], out[1][0]) and torch.equal(out[0][1], out[1][1])


# ---------------------------------------------------------------- router backward
def route_bwd(Lg, k, idx, prob, dprob, counts, alpha, aux_scale):
    import token_routed_expert_amd as tre
    T, E = Lg.shape
    dl = torch.full((T, E), float("nan"), dtype=torch.float32, device="cuda")
    cg = None if counts is None else torch.from_numpy(counts.astype(np.int32)).cuda()
    tre.moe_route_bwd(Lg, k, idx, prob, dprob, cg, alpha, aux_scale, dl)
    return dl.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (5, 2, 1), (999, 8, 2), (1000, 64, 6), (513, 128, 8),
                                   (257, 256, 8), (100, 33, 33), (64, 200, 1)])
def test_route_bwd_jacobian(T, E, k):
    """Top-k softmax Jacobian alone: zeros off the selected experts, bit-exact."""
    L, Lg, idx, prob, counts, _, rp = routed(T, E, k, seed=E * 7 + k)
    dp = torch.randn(T, k, generator=torch.Generator().manual_seed(T)).cuda()
    got = route_bwd(Lg, k, idx, prob, dp, None, 0.0, 1.0)
    ref = oracle.router_bwd(dp.cpu().numpy(), rp, idx.cpu().numpy(), E)
    sel = np.zeros((T, E), bool)
    sel[np.arange(T)[:, None], idx.cpu().numpy()] = True
    assert (got[~sel] == 0).all()
    if E == 1 or k == 1:
        assert (got == 0).all()          # a softmax over one logit is constant
    else:
        assert_close("dlogits", got, ref, ROW_TOL)
    # counts given but alpha == 0: the same values
    got0 = route_bwd(Lg, k, idx, prob, dp, counts, 0.0, 1.0)
    assert np.array_equal(got0, got)


@pytest.mark.parametrize("skew", [False, True])
@pytest.mark.parametrize("T,E,k", [(1, 40, 2), (999, 16, 2), (1000, 128, 8), (130, 256, 8)])
def test_route_bwd_aux(T, E, k, skew):
    """Load-balancing term alone (dprob = 0), then both terms with aux_scale."""
    L, Lg, idx, prob, counts, _, rp = routed(T, E, k, seed=E + k, skew=skew and E > 10 + k)
    alpha = 0.01
    zero = torch.zeros(T, k, device="cuda")
    got = route_bwd(Lg, k, idx, prob, zero, counts, alpha, 1.0)
    _, ref_aux = oracle.aux_loss(L.numpy(), counts, k, alpha)
    assert_close("aux dlogits", got, ref_aux, ROW_TOL)
    dp = torch.randn(T, k, generator=torch.Generator().manual_seed(1)).cuda()
    got = route_bwd(Lg, k, idx, prob, dp, counts, alpha, 3.0)
    ref = oracle.router_bwd(dp.cpu().numpy(), rp, idx.cpu().numpy(), E) + 3.0 * ref_aux
    assert_close("dlogits", got, ref, ROW_TOL)


# ---------------------------------------------------------------- auxiliary loss
def aux_loss_gpu(Lg, k, counts, alpha):
    import token_routed_expert_amd as tre
    from token_routed_expert_amd import _native as N
    T, E = Lg.shape
    sh = tre.make_shape(T, 128, E, k, 128, 0, "bf16")
    ws = torch.empty(max(256, tre.moe_workspace_bytes(sh, N.MOE_WS_AUX_LOSS)), dtype=torch.uint8,
                     device="cuda")
    loss = torch.full((1,), float("nan"), device="cuda")
    tre.moe_aux_loss(Lg, k, torch.from_numpy(counts.astype(np.int32)).cuda(), alpha, loss, ws)
    return float(loss.item())


@pytest.mark.parametrize("skew", [False, True])
@pytest.mark.parametrize("T,E,k", [(1, 12, 1), (63, 8, 2), (64, 8, 2), (65, 8, 2), (8200, 128, 8),
                                   (4097, 256, 8), (300, 1, 1)])
def test_aux_loss(T, E, k, skew):
    L, Lg, idx, prob, counts, _, rp = routed(T, E, k, seed=T ^ E, skew=skew and E > 10 + k)
    got = aux_loss_gpu(Lg, k, counts, 0.01)
    ref, _ = oracle.aux_loss(L.numpy(), counts, k, 0.01)
    assert abs(got - ref) <= LOSS_TOL * abs(ref), (got, ref)
    if E == 1:
        assert abs(got - 0.01) <= 1e-8        # one expert: f = P = 1, L = alpha


@pytest.mark.parametrize("T,E,k,skew", [(1, 12, 1, False), (63, 8, 2, False), (65, 8, 2, True),
                                        (8200, 128, 8, True), (4097, 256, 8, False),
                                        (300, 1, 1, False), (1000, 200, 6, False),
                                        (777, 33, 7, True), (129, 64, 64, False)])
def test_route_aux_fused(T, E, k, skew):
    """moe_route_aux: indices and probabilities bit-identical to moe_route;
    moe_aux_loss_final after it bit-identical to moe_aux_loss, and within
    the loss tolerance of the oracle."""
    import token_routed_expert_amd as tre
    from token_routed_expert_amd import _native as N
    L, Lg, idx, prob, counts, _, _ = routed(T, E, k, seed=T + 3 * E, skew=skew and E > 10 + k)
    if T > 100:
        Lg[5, :] = float("nan")                     # a NaN row routes as moe_route does
        Lg[7, ::3] = float("nan")
        tre.moe_route(Lg, k, idx, prob)
    sh = tre.make_shape(T, 128, E, k, 128, 0, "bf16")
    wsb = max(256, tre.moe_workspace_bytes(sh, N.MOE_WS_AUX_LOSS))
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    idx2 = torch.full_like(idx, -9)
    prob2 = torch.full_like(prob, 5.0)
    tre.moe_route_aux(Lg, k, idx2, prob2, ws)
    assert torch.equal(idx2, idx)
    assert torch.equal(prob2.view(torch.int32), prob.view(torch.int32))
    if T > 100:
        Lg = L.cuda()                               # the loss on finite logits
        tre.moe_route_aux(Lg, k, idx2, prob2, ws)
    c = torch.from_numpy(counts.astype(np.int32)).cuda()
    loss = torch.full((1,), float("nan"), device="cuda")
    tre.moe_aux_loss_final(ws, T, E, k, c, 0.01, loss)
    ws2 = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    loss2 = torch.full((1,), float("nan"), device="cuda")
    tre.moe_aux_loss(Lg, k, c, 0.01, loss2, ws2)
    assert torch.equal(loss.view(torch.int32), loss2.view(torch.int32)), (float(loss), float(loss2))
    ref, _ = oracle.aux_loss(L.numpy(), counts, k, 0.01)
    assert abs(float(loss) - ref) <= LOSS_TOL * abs(ref), (float(loss), ref)


def test_aux_loss_uniform_router():
    """Equal logits: P_e = 1/E and sum_e f_e = 1, so L = alpha exactly."""
    T, E, k = 1000, 64, 4
    Lg = torch.full((T, E), 0.5, device="cuda")
    counts = np.zeros(E, np.int64)
    counts[:k] = T                          # lowest-index ties
    got = aux_loss_gpu(Lg, k, counts, 0.02)
    assert abs(got - 0.02) <= 1e-6 * 0.02


def test_workspace_and_row_limits():
    import token_routed_expert_amd as tre
    from token_routed_expert_amd import MoeError
    T, E, k = 100, 8, 2
    Lg = torch.randn(T, E, device="cuda")
    c = torch.zeros(E, dtype=torch.int32, device="cuda")
    loss = torch.empty(1, device="cuda")
    with pytest.raises(MoeError):
        tre.moe_aux_loss(Lg, k, c, 0.01, loss, torch.empty(8, dtype=torch.uint8, device="cuda"))


# ---------------------------------------------------------------- layer level
LAYERS = [WORKLOADS["tiny_f32"],
          Workload("rg_bf16", T=777, d=256, E=16, k=4, f=256),
          Workload("rg_shared_bf16", T=300, d=128, E=8, k=2, f=128, f_shared=128),
          Workload("rg_e4m3", T=520, d=256, E=16, k=4, f=256, dtype="e4m3")]


@pytest.mark.parametrize("wl", LAYERS, ids=lambda w: w.name)
def test_layer_router_grad(wl):
    """moe_layer_fwd/bwd with the router gradient: every other output is
    bit-identical to the plain layer; loss, dprob and dlogits match the oracle
    on the layer's own expert outputs o."""
    inp = make_inputs(wl, seed=3, device="cuda")
    plain = run_layer(wl, inp)
    b = run_layer(wl, inp, router_grad=True, aux_alpha=0.01)
    for n in ("y", "o", "dO", "dX", "dXp", "dW1", "dW3", "dW2", "topk_idx", "row_of"):
        assert torch.equal(plain[n], b[n]), n
    L = inp["logits"].cpu().numpy()
    idx = b["topk_idx"].cpu().numpy()
    p = oracle.route(L, wl.k)[1]
    counts = b["counts"].cpu().numpy()
    row_of = b["row_of"].cpu().numpy()
    ref_loss, ref_aux = oracle.aux_loss(L, counts, wl.k, 0.01)
    got_loss = float(b["aux_loss"].item())
    assert abs(got_loss - ref_loss) <= LOSS_TOL * abs(ref_loss)
    dY, o = to_f64(inp["dY"]), to_f64(b["o"])
    dp = b["dprob"].cpu().numpy().astype(np.float64)
    check_dot("dprob", dp, dY, o, row_of)
    ref = oracle.router_bwd(dp, p, idx, wl.E) + ref_aux
    assert_close("dlogits", b["dlogits"].cpu().numpy().astype(np.float64), ref, ROW_TOL)
    if wl.dtype != "e4m3":
        # against the oracle's own forward: dprob inherits the error of o, which
        # the layer tests bound by TOL * max|o row|, so
        # |dprob - ref| <= TOL * ||dY[t]||_1 * max|o[row]| (+ the fp32 dot bound)
        st = oracle.layer_fwd(L, to_f64(inp["x"]), to_f64(inp["W1"]), to_f64(inp["W3"]),
                              to_f64(inp["W2"]), wl.k)
        dp_ref = oracle.combine_dprob(dY, st["o"], st["row_of"])
        omax = np.abs(st["o"]).max(axis=1)[st["row_of"]]
        bound = TOL[wl.dtype] * np.abs(dY).sum(axis=1)[:, None] * omax
        assert (np.abs(dp - dp_ref) <= bound).all()


@pytest.mark.parametrize("wl", [WORKLOADS["qwen3_bf16"], WORKLOADS["skewed_fp8"]],
                         ids=lambda w: w.name)
def test_layer_router_grad_full_size(wl):
    """Full-size layer with the router gradient: loss and every dlogits row
    against the oracle on the device's dprob; dprob on sampled tokens."""
    announce(f"{wl.name}: inputs")
    inp = make_inputs(wl, seed=0, device="cuda")
    announce(f"{wl.name}: layer fwd+bwd with the router gradient")
    b = run_layer(wl, inp, router_grad=True, aux_alpha=0.001)
    L = inp["logits"].cpu().numpy()
    idx = b["topk_idx"].cpu().numpy()
    ridx, p = oracle.route(L, wl.k)
    assert np.array_equal(idx, ridx)
    counts = b["counts"].cpu().numpy()
    row_of = b["row_of"].cpu().numpy()
    announce(f"{wl.name}: oracle loss and dlogits")
    ref_loss, ref_aux = oracle.aux_loss(L, counts, wl.k, 0.001)
    assert abs(float(b["aux_loss"].item()) - ref_loss) <= LOSS_TOL * abs(ref_loss)
    dp = b["dprob"].cpu().numpy().astype(np.float64)
    ref = oracle.router_bwd(dp, p, idx, wl.E) + ref_aux
    assert_close("dlogits", b["dlogits"].cpu().numpy().astype(np.float64), ref, ROW_TOL)
    rng = np.random.default_rng(1)
    toks = np.array([0, wl.T - 1] + list(rng.choice(wl.T, 30, replace=False)))
    dY = to_f64(inp["dY"][torch.from_numpy(toks).cuda()])
    rows = row_of[toks]
    o = to_f64(b["o"][torch.from_numpy(rows.reshape(-1)).cuda()])
    check_dot("dprob", dp[toks], dY, o, np.arange(rows.size).reshape(rows.shape))
