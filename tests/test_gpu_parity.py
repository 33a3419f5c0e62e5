"""GPU path vs the oracle, through the C ABI, on seeded synthetic inputs.

Small workloads are compared element by element on every output; the
full-size workloads (the launch configuration the benchmark times) compare
routing and permutation in full and the floating-point outputs on sampled
tokens and experts, which the oracle computes one by one.
Tolerances (max over rows of max|gpu-ref| / max|ref|): fp32 1e-4, bf16 2e-2;
routing indices, counts, offsets, row maps and permuted rows bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_workloads import WORKLOADS, Workload, make_inputs, skew_bias, tied_logits, to_f64

from gpu_common import (PROB_TOL, TOL, announce, assert_close, bits, check_routing_and_map,
                        host_inputs, need_gpu, oracle_layer, run_layer)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu(request):
    need_gpu()
    announce(request.node.nodeid)
    yield
    torch.cuda.synchronize()


# ---------------------------------------------------------------- routing
@pytest.mark.parametrize("E,k", [(1, 1), (2, 1), (3, 2), (5, 5), (8, 2), (16, 4), (33, 7), (64, 8),
                                 (100, 8), (128, 8), (200, 6), (256, 8), (256, 1)])
@pytest.mark.parametrize("tied", [False, True])
def test_route_bit_exact(E, k, tied):
    import token_routed_expert_amd as tre
    T = 1000
    L = tied_logits(T, E, levels=3, seed=E) if tied else torch.randn(
        T, E, generator=torch.Generator().manual_seed(E))
    if tied:
        L[::7] = 0.0
        L[3::7, :] = -0.0       # +0 / -0 ties
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    prob = torch.empty(T, k, dtype=torch.float32, device="cuda")
    tre.moe_route(L.cuda(), k, idx, prob)
    ridx, rp = oracle.route(L.numpy(), k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.abs(prob.cpu().numpy() - rp).max() <= PROB_TOL


@pytest.mark.parametrize("E,k", [(8, 2), (8, 8), (128, 8), (256, 4)])
def test_route_nan_logits_give_valid_experts(E, k):
    """NaN logits rank below every number: indices bit-exact against the
    oracle, always k distinct experts in [0, E); the map built from them is
    the oracle's."""
    import token_routed_expert_amd as tre
    from token_routed_expert_amd import _native as N
    T = 700
    g = torch.Generator().manual_seed(E + k)
    L = torch.randn(T, E, generator=g)
    L[0] = float("nan")                                    # all NaN
    L[1, ::2] = float("nan")                               # half NaN
    L[2, :] = float("-inf")
    L[2, 1::3] = float("nan")                              # -inf and NaN mixed
    L[5::11, 0] = float("nan")
    L[7::13, E - 1] = float("nan")
    L[9::17, : max(1, E - k + 1)] = float("nan")           # at most k - 1 numbers left
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    prob = torch.empty(T, k, dtype=torch.float32, device="cuda")
    tre.moe_route(L.cuda(), k, idx, prob)
    ridx, rp = oracle.route(L.numpy(), k)
    gi = idx.cpu().numpy()
    assert np.array_equal(gi, ridx)
    assert (gi >= 0).all() and (gi < E).all()
    assert all(len(set(r)) == k for r in gi)
    gp = prob.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isnan(gp), np.isnan(rp))
    fin = ~np.isnan(rp)
    assert np.abs(gp[fin] - rp[fin]).max() <= PROB_TOL
    sh = tre.make_shape(T, 64, E, k, 128, 0, "bf16")
    counts, offsets, row_of, token_of = oracle.permute_map(ridx, E)
    c = torch.empty(E, dtype=torch.int32, device="cuda")
    o = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    r = torch.empty(T, k, dtype=torch.int32, device="cuda")
    tk = torch.empty(T * k, dtype=torch.int32, device="cuda")
    x = torch.randn(T, 64, generator=g).to(torch.bfloat16).cuda()
    xp = torch.empty(T * k, 64, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(tre.moe_workspace_bytes(sh, N.MOE_WS_PERMUTE), dtype=torch.uint8, device="cuda")
    tre.moe_permute(sh, x, idx, None, 1, c, o, r, tk, xp, ws)
    assert np.array_equal(c.cpu().numpy(), counts) and np.array_equal(r.cpu().numpy(), row_of)
    assert np.array_equal(tk.cpu().numpy(), token_of)


def test_permute_skips_indices_outside_the_experts():
    """An index outside [0, E) gets row_of = -1 and no row; counts and rows
    are those of the valid assignments in the canonical order; the row moves
    and the combine skip the assignment (rows from offsets[E] on stay as they
    were)."""
    import token_routed_expert_amd as tre
    from token_routed_expert_amd import _native as N
    T, E, k, d = 300, 16, 4, 128
    rng = np.random.default_rng(4)
    idx_np = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    bad = rng.random((T, k)) < 0.1
    idx_np[bad] = rng.choice(np.array([-1, E, E + 7, 1 << 30, -(1 << 30)], dtype=np.int32), bad.sum())
    valid = (idx_np >= 0) & (idx_np < E)
    flat, vflat = idx_np.reshape(-1), valid.reshape(-1)
    pos = np.nonzero(vflat)[0]
    order = pos[np.argsort(flat[pos], kind="stable")]       # token-major, then by expert
    nv = len(pos)
    ref_row = np.full(T * k, -1, np.int64)
    ref_row[order] = np.arange(nv)
    ref_counts = np.bincount(flat[pos], minlength=E)
    ref_tok = order // k
    sh = tre.make_shape(T, d, E, k, 128, 0, "bf16")
    x = torch.randn(T, d, generator=torch.Generator().manual_seed(2)).to(torch.bfloat16)
    c = torch.empty(E, dtype=torch.int32, device="cuda")
    o = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    r = torch.empty(T, k, dtype=torch.int32, device="cuda")
    tk = torch.full((T * k,), -7, dtype=torch.int32, device="cuda")
    xp = torch.full((T * k, d), 3.0, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(tre.moe_workspace_bytes(sh, N.MOE_WS_PERMUTE), dtype=torch.uint8, device="cuda")
    tre.moe_permute(sh, x.cuda(), torch.from_numpy(idx_np).cuda(), None, 1, c, o, r, tk, xp, ws)
    assert np.array_equal(c.cpu().numpy(), ref_counts)
    assert int(o.cpu()[E]) == nv
    assert np.array_equal(r.cpu().numpy().reshape(-1), ref_row)
    assert np.array_equal(tk.cpu().numpy()[:nv], ref_tok) and (tk.cpu().numpy()[nv:] == -7).all()
    xpn = xp.cpu()
    assert torch.equal(xpn[:nv], x[torch.from_numpy(ref_tok)]) and (xpn[nv:] == 3.0).all()
    p = torch.rand(T, k, generator=torch.Generator().manual_seed(3))
    dO = torch.full((T * k, d), 5.0, dtype=torch.bfloat16, device="cuda")
    tre.moe_permute(sh, x.cuda(), None, p.cuda(), 0, None, None, r, None, dO, None)
    assert (dO.cpu()[nv:] == 5.0).all()
    y = torch.empty(T, d, dtype=torch.bfloat16, device="cuda")
    tre.moe_unpermute(sh, xp, r, p.cuda(), None, y)
    xf = to_f64(x)
    ref = np.zeros((T, d))
    for t in range(T):
        for j in range(k):
            if valid[t, j]:
                ref[t] += float(p[t, j]) * xf[t]
    assert_close("combine", to_f64(y), ref, TOL["bf16"] / 4)


# ---------------------------------------------------------------- permute / combine
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T,E,k,d", [(1, 4, 2, 64), (257, 8, 2, 128), (1000, 128, 8, 256),
                                     (513, 256, 8, 64), (300, 16, 16, 32)])
def test_permute_unpermute(dtype, T, E, k, d):
    import token_routed_expert_amd as tre
    from token_routed_expert_amd import _native as N
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    sh = tre.make_shape(T, d, E, k, 128, 0, dtype)
    g = torch.Generator().manual_seed(T + E)
    L = torch.randn(T, E, generator=g)
    # expert 0 gets no rows when k < E; with k == E every expert is picked, so keep its
    # weight a normal fp32 number (exp(-100) would be subnormal and lose precision)
    L[:, 0] -= 100.0 if k < E else 5.0
    x = torch.randn(T, d, generator=g).to(dt)
    dY = torch.randn(T, d, generator=g).to(dt)
    ridx, rp = oracle.route(L.numpy(), k)
    counts, offsets, row_of, token_of = oracle.permute_map(ridx, E)
    idx = torch.from_numpy(ridx).cuda()
    P = T * k
    c = torch.empty(E, dtype=torch.int32, device="cuda")
    o = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    r = torch.empty(T, k, dtype=torch.int32, device="cuda")
    tk = torch.empty(P, dtype=torch.int32, device="cuda")
    xp = torch.empty(P, d, dtype=dt, device="cuda")
    ws = torch.empty(tre.moe_workspace_bytes(sh, N.MOE_WS_PERMUTE), dtype=torch.uint8, device="cuda")
    tre.moe_permute(sh, x.cuda(), idx, None, 1, c, o, r, tk, xp, ws)
    assert np.array_equal(c.cpu().numpy(), counts) and np.array_equal(o.cpu().numpy(), offsets)
    assert np.array_equal(r.cpu().numpy(), row_of) and np.array_equal(tk.cpu().numpy(), token_of)
    assert np.array_equal(bits(xp), oracle.permute_rows(bits(x), token_of))
    # scaled permute (backward of the weighted combine), reusing the map
    p = torch.from_numpy(rp.astype(np.float32)).cuda()
    dO = torch.empty(P, d, dtype=dt, device="cuda")
    tre.moe_permute(sh, dY.cuda(), None, p, 0, None, None, r, None, dO, None)
    ref = oracle.permute_scaled(to_f64(dY), row_of, p.cpu().numpy().astype(np.float64))
    assert_close("dO", to_f64(dO), ref, TOL[dtype] / 4)
    # weighted combine of the permuted rows is the identity (probabilities sum to 1)
    y = torch.empty(T, d, dtype=dt, device="cuda")
    tre.moe_unpermute(sh, xp, r, p, None, y)
    assert_close("identity combine", to_f64(y), to_f64(x), 1e-6)
    if dtype == "bf16":
        assert torch.equal(y.cpu(), x)                       # bit-exact in bf16
    # unit-weight combine with an added tensor
    src = torch.randn(P, d, generator=g).to(dt)
    add = torch.randn(T, d, generator=g).to(dt)
    tre.moe_unpermute(sh, src.cuda(), r, None, add.cuda(), y)
    ref = oracle.combine(to_f64(src), row_of, None, to_f64(add))
    assert_close("unit combine", to_f64(y), ref, TOL[dtype] / 4)
    tre.moe_unpermute(sh, src.cuda(), r, p, None, y)
    ref = oracle.combine(to_f64(src), row_of, p.cpu().numpy().astype(np.float64))
    assert_close("weighted combine", to_f64(y), ref, TOL[dtype] / 4)


# ---------------------------------------------------------------- grouped GEMM entry points
@pytest.mark.parametrize("wl", [
    Workload("gg_bf16", T=600, d=384, E=6, k=2, f=384),
    Workload("gg_f32", T=300, d=96, E=5, k=3, f=80, dtype="f32"),
], ids=lambda w: w.name)
def test_grouped_gemm_entry_points(wl):
    import token_routed_expert_amd as tre
    inp = make_inputs(wl, seed=3)
    h = host_inputs(inp)
    ridx, rp = oracle.route(h["logits"], wl.k)
    counts, offsets, row_of, token_of = oracle.permute_map(ridx, wl.E)
    xp = oracle.permute_rows(h["x"], token_of)
    a, b, hh, o = oracle.experts_fwd(xp, offsets, h["W1"], h["W3"], h["W2"])
    dO = oracle.permute_scaled(h["dY"], row_of, rp)
    dXp, dW1, dW3, dW2, da, db = oracle.experts_bwd(dO, xp, a, b, hh, offsets, h["W1"], h["W3"], h["W2"])
    dt = inp["x"].dtype
    dev = {k: v.cuda() for k, v in inp.items()}
    P, f, d = wl.P, wl.f, wl.d
    sh = tre.make_shape(wl.T, d, wl.E, wl.k, f, 0, wl.dtype)
    off = torch.from_numpy(offsets.astype(np.int32)).cuda()
    xp_d = torch.from_numpy(xp).to(dt).cuda()
    ab_d = torch.empty(P, 2 * f, dtype=dt, device="cuda")
    h_d = torch.empty(P, f, dtype=dt, device="cuda")
    o_d = torch.empty(P, d, dtype=dt, device="cuda")
    tre.moe_grouped_gemm_fwd(sh, off, xp_d, dev["W1"], dev["W3"], dev["W2"], ab_d, h_d, o_d)
    tol = TOL[wl.dtype]
    assert_close("ab", to_f64(ab_d), np.concatenate([a, b], 1), tol)
    assert_close("h", to_f64(h_d), hh, tol)
    assert_close("o", to_f64(o_d), o, tol)
    dO_d = torch.from_numpy(dO).to(dt).cuda()
    dab_d = torch.empty(P, 2 * f, dtype=dt, device="cuda")
    dXp_d = torch.empty(P, d, dtype=dt, device="cuda")
    dW1_d, dW3_d = torch.empty_like(dev["W1"]), torch.empty_like(dev["W3"])
    dW2_d = torch.empty_like(dev["W2"])
    tre.moe_grouped_gemm_bwd(sh, off, xp_d, ab_d, h_d, dO_d, dev["W1"], dev["W3"], dev["W2"], dab_d,
                             dXp_d, dW1_d, dW3_d, dW2_d)
    assert_close("dab", to_f64(dab_d), np.concatenate([da, db], 1), tol)
    assert_close("dXp", to_f64(dXp_d), dXp, tol)
    assert_close("dW1", to_f64(dW1_d), dW1, tol)
    assert_close("dW3", to_f64(dW3_d), dW3, tol)
    assert_close("dW2", to_f64(dW2_d), dW2, tol)


# ---------------------------------------------------------------- whole layer, small
SMALL = [
    WORKLOADS["tiny_f32"],
    Workload("tiny_bf16", T=256, d=128, E=8, k=2, f=128),
    Workload("small_bf16", T=512, d=256, E=8, k=2, f=256),
    Workload("multitile_bf16", T=1100, d=512, E=4, k=2, f=640),
    Workload("ragged_skew_bf16", T=700, d=384, E=16, k=4, f=384, skew=True),
    # more tiles than compute units: every persistent block runs several
    # tiles, across experts with hundreds of rows, a few rows and none
    Workload("persistent_skew_bf16", T=2048, d=1024, E=32, k=4, f=768, skew=True),
    # ... and weight-gradient tiles of 1 to 3 K stages (about 32 rows an expert)
    Workload("persistent_short_k_bf16", T=1024, d=1024, E=64, k=2, f=512),
    Workload("shared_bf16", T=300, d=256, E=8, k=2, f=128, f_shared=256),
    Workload("wide_e_bf16", T=512, d=128, E=256, k=8, f=128),
    Workload("dense_bf16", T=200, d=256, E=1, k=1, f=384),
    Workload("k_eq_E_bf16", T=64, d=128, E=4, k=4, f=128),
    Workload("one_token_bf16", T=1, d=128, E=8, k=2, f=128),
    Workload("ragged_skew_f32", T=333, d=96, E=16, k=3, f=80, dtype="f32", skew=True),
    Workload("shared_f32", T=100, d=32, E=4, k=2, f=48, f_shared=24, dtype="f32"),
]


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_layer_small(wl):
    inp = make_inputs(wl, seed=0, device="cuda")
    b = run_layer(wl, inp)
    h = host_inputs(inp)
    st, g = oracle_layer(wl, h)
    check_routing_and_map(wl, b, inp, st)
    tol = TOL[wl.dtype]
    assert_close("ab", to_f64(b["ab"]), np.concatenate([st["a"], st["b"]], 1), tol)
    assert_close("h", to_f64(b["h"]), st["h"], tol)
    assert_close("o", to_f64(b["o"]), st["o"], tol)
    assert_close("y", to_f64(b["y"]), st["y"], tol)
    assert_close("dXp", to_f64(b["dXp"]), g["dXp"], tol)
    assert_close("dX", to_f64(b["dX"]), g["dX"], tol)
    for n in ("dW1", "dW3", "dW2") + (("dWs1", "dWs3", "dWs2") if wl.f_shared else ()):
        assert_close(n, to_f64(b[n]), g[n], tol)
    for e in np.nonzero(st["counts"] == 0)[0]:                  # empty experts: exact zeros
        assert not b["dW1"][e].any() and not b["dW3"][e].any() and not b["dW2"][e].any()


def test_one_expert_takes_all_tokens():
    wl = Workload("all_to_one_bf16", T=700, d=256, E=8, k=1, f=256)
    inp = make_inputs(wl, seed=1, device="cuda")
    inp["logits"][:, 5] += 50.0
    b = run_layer(wl, inp)
    st, g = oracle_layer(wl, host_inputs(inp))
    assert st["counts"][5] == 700
    check_routing_and_map(wl, b, inp, st)
    assert_close("y", to_f64(b["y"]), st["y"], TOL["bf16"])
    assert_close("dX", to_f64(b["dX"]), g["dX"], TOL["bf16"])
    for n in ("dW1", "dW3", "dW2"):
        assert_close(n, to_f64(b[n]), g[n], TOL["bf16"])


def test_layer_is_deterministic():
    wl = Workload("det_bf16", T=900, d=256, E=16, k=4, f=256)
    inp = make_inputs(wl, seed=2, device="cuda")
    b1 = run_layer(wl, inp)
    b2 = run_layer(wl, inp)
    for n in ("y", "dX", "dW1", "dW3", "dW2", "xp", "ab", "h", "row_of", "token_of"):
        assert torch.equal(b1[n], b2[n]), n


# ---------------------------------------------------------------- full size, sampled
FULL = [WORKLOADS["mixtral_bf16"], WORKLOADS["qwen3_bf16"], WORKLOADS["deepseek_v3_bf16"],
        WORKLOADS["skewed_fp8"].with_(name="skewed_bf16", dtype="bf16")]


@pytest.mark.parametrize("wl", FULL, ids=lambda w: w.name)
def test_layer_full_size_sampled(wl):
    full_size_sampled(wl)


def full_size_sampled(wl, n_tokens=32, **kw):
    """The layer at full size (kw: layer_buffers options) against the oracle:
    routing and permutation in full; for five experts (the first non-empty,
    the median, the hottest, the smallest non-empty and the highest-index one
    with rows) every product on sampled rows of theirs (first, last and six
    more: ab, h, o, dab, dXp from each row's own oracle chain) and their
    weight gradients; y and dX on n_tokens tokens (the first, the last, tokens
    of the hottest and of the highest-index expert, the rest random)."""
    announce(f"{wl.name}: inputs")
    inp = make_inputs(wl, seed=0, device="cuda")
    announce(f"{wl.name}: layer fwd+bwd {kw}")
    b = run_layer(wl, inp, **kw)
    announce(f"{wl.name}: oracle routing/permutation")
    L = inp["logits"].cpu().numpy()
    idx, p = oracle.route(L, wl.k)
    counts, offsets, row_of, token_of = oracle.permute_map(idx, wl.E)
    st = dict(idx=idx, p=p, counts=counts, offsets=offsets, row_of=row_of, token_of=token_of)
    check_routing_and_map(wl, b, inp, st)
    if wl.skew:
        assert (counts == 0).sum() >= 10
    tol = TOL[wl.dtype]
    me = kw.get("memory_efficient", 0)          # h and o then hold p-scaled rows
    W = {n: inp[n] for n in ("W1", "W3", "W2")}
    shared = None
    if wl.f_shared:
        shared = tuple(to_f64(inp[n]) for n in ("Ws1", "Ws3", "Ws2"))
    cache = {}

    def expert(e):
        if e not in cache:
            if len(cache) >= 16:
                cache.pop(next(iter(cache)))
            cache[e] = tuple(to_f64(W[n][e]) for n in ("W1", "W3", "W2"))
        return cache[e]

    x_h, dY_h = inp["x"], inp["dY"]
    p_rows = p.reshape(-1)[np.argsort(row_of.reshape(-1))]          # probability of each row
    nonempty = np.nonzero(counts)[0]
    hot, last = int(np.argmax(counts)), int(nonempty[-1])
    small = int(nonempty[np.argmin(counts[nonempty])])
    if counts[wl.E - 1] > 0:
        assert last == wl.E - 1
    experts = list(dict.fromkeys([int(nonempty[0]), int(nonempty[len(nonempty) // 2]), hot, small,
                                  last]))
    rng = np.random.default_rng(0)
    f = wl.f
    for e in experts:
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        announce(f"{wl.name}: expert {e} ({r1 - r0} rows): sampled rows and weight gradients")
        rows = np.array(sorted({r0, r1 - 1} | set(rng.choice(np.arange(r0, r1), min(6, r1 - r0),
                                                              replace=False).tolist())))
        sel = torch.from_numpy(rows).cuda()
        toks = torch.from_numpy(token_of[rows]).cuda()
        X = to_f64(x_h[toks])
        dO = p_rows[rows, None] * to_f64(dY_h[toks])
        W1, W3, W2 = expert(e)
        a, bb, h, o = oracle.swiglu_fwd(X, W1, W3, W2)
        dXr, _, _, _, da, db = oracle.swiglu_bwd(X, a, bb, h, dO, W1, W3, W2)
        pr = p_rows[rows, None] if me else 1.0
        assert_close(f"ab[{e}]", to_f64(b["ab"][sel]), np.concatenate([a, bb], 1), tol)
        assert_close(f"h[{e}]", to_f64(b["h"][sel]), pr * h, tol)
        assert_close(f"o[{e}]", to_f64(b["o"][sel]), pr * o, tol)
        assert_close(f"dab[{e}]", to_f64(b["dab"][sel]), np.concatenate([da, db], 1), tol)
        assert_close(f"dXp[{e}]", to_f64(b["dXp"][sel]), dXr, tol)
        allr = torch.from_numpy(token_of[r0:r1]).cuda()
        dO_e = p_rows[r0:r1, None] * to_f64(dY_h[allr])
        dW1, dW3, dW2 = oracle.expert_wgrad(to_f64(x_h[allr]), dO_e, W1, W3, W2)
        assert_close(f"dW1[{e}]", to_f64(b["dW1"][e]), dW1, tol)
        assert_close(f"dW3[{e}]", to_f64(b["dW3"][e]), dW3, tol)
        assert_close(f"dW2[{e}]", to_f64(b["dW2"][e]), dW2, tol)
    for e in np.nonzero(counts == 0)[0][:4]:
        assert not b["dW1"][int(e)].any() and not b["dW2"][int(e)].any()
    # tokens: first, last, some of the hottest and of the highest-index expert, random
    picks = [0, wl.T - 1]
    for e in (hot, last):
        seg = token_of[int(offsets[e]):int(offsets[e + 1])]
        picks += [int(t) for t in rng.choice(seg, min(4, len(seg)), replace=False)]
    picks += [int(t) for t in rng.choice(wl.T, n_tokens, replace=False)]
    tokens = list(dict.fromkeys(picks))[:max(n_tokens, 10)]
    announce(f"{wl.name}: oracle y and dX on {len(tokens)} tokens")
    for t in tokens:
        Ws = {int(e): expert(int(e)) for e in idx[t]}
        y_t, dX_t = oracle.token_fwd_bwd(to_f64(x_h[t]), to_f64(dY_h[t]), idx[t], p[t],
                                         {e: w[0] for e, w in Ws.items()},
                                         {e: w[1] for e, w in Ws.items()},
                                         {e: w[2] for e, w in Ws.items()}, shared)
        assert_close(f"y[{t}]", to_f64(b["y"][t])[None], y_t[None], tol)
        assert_close(f"dX[{t}]", to_f64(b["dX"][t])[None], dX_t[None], tol)


# ---------------------------------------------------------------- matrix-core probe
@pytest.mark.parametrize("dtype", ["bf16", "e4m3"])
def test_mfma_probe(dtype):
    """The probe runs, reports the launch's flop count and a plausible clock
    (ticks of a wavefront's loop against the wall clock)."""
    import token_routed_expert_amd as tre
    ticks = torch.zeros(2, dtype=torch.int64, device="cuda")
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    flops, khz = tre.moe_probe_mfma(dtype, 64, ticks, sink)
    torch.cuda.synchronize()
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    per = 16 * 16 * (32 if dtype == "bf16" else 128) * 2
    assert flops == n_cu * 8 * 4 * 64 * 8 * per
    cyc, wall = (int(v) for v in ticks.cpu())
    assert cyc > 0 and wall > 0 and khz > 0
    ghz = cyc / (wall / (khz * 1e3)) / 1e9
    assert 0.3 < ghz < 3.5, ghz
    with pytest.raises(tre.MoeError):
        tre.moe_probe_mfma(dtype, 0, ticks, sink)


# ---------------------------------------------------------------- hand-derived fixture
def test_route_permute_golden():
    """moe_route and moe_permute on the hand-built case of
    tests/golden/route_permute_tiny.json (ties, an empty expert): indices,
    counts, offsets and the map bit-exact, probabilities to float32 rounding,
    and the permuted rows equal to their source rows."""
    import token_routed_expert_amd as tre
    from token_routed_expert_amd import _native as N
    from golden_fixtures import fraction, load, logits_f32
    fx = load("route_permute_tiny.json")
    T, E, k, d = fx["T"], fx["E"], fx["k"], 64
    L = torch.from_numpy(logits_f32(fx)).cuda()
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    p = torch.empty(T, k, dtype=torch.float32, device="cuda")
    tre.moe_route(L, k, idx, p)
    assert np.array_equal(idx.cpu().numpy(), np.array(fx["topk_idx"]))
    want = np.array([[fraction(v) for v in row] for row in fx["topk_prob"]])
    assert np.allclose(p.cpu().numpy(), want, rtol=0, atol=1e-6)
    sh = tre.make_shape(T, d, E, k, 128, 0, "f32")
    x = (torch.arange(T, dtype=torch.float32)[:, None] * 1000 + torch.arange(d)[None, :]).cuda()
    P = T * k
    c = torch.empty(E, dtype=torch.int32, device="cuda")
    o = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    r = torch.empty(T, k, dtype=torch.int32, device="cuda")
    tk = torch.empty(P, dtype=torch.int32, device="cuda")
    xp = torch.empty(P, d, dtype=torch.float32, device="cuda")
    ws = torch.empty(tre.moe_workspace_bytes(sh, N.MOE_WS_PERMUTE), dtype=torch.uint8, device="cuda")
    tre.moe_permute(sh, x, idx, None, 1, c, o, r, tk, xp, ws)
    assert np.array_equal(c.cpu().numpy(), fx["counts"])
    assert np.array_equal(o.cpu().numpy(), fx["offsets"])
    assert np.array_equal(r.cpu().numpy(), np.array(fx["row_of"]))
    assert np.array_equal(tk.cpu().numpy(), fx["token_of"])
    assert torch.equal(xp.cpu(), x.cpu()[torch.tensor(fx["token_of"])])
