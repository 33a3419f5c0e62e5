"""MXFP8 path vs the oracle, through the C ABI, on seeded synthetic inputs.

* Quantisers (1 x 32 rows, both orientations of the expert weights, 32-row
  token blocks) and the MXFP8 permutation: codes and E8M0 scale bytes
  bit-exact.
* Expert GEMM products: within 6e-2 (max over rows of max|gpu-ref| /
  max|ref|) of the oracle run on the same quantised inputs, as for e4m3.
* The whole layer is also compared with the oracle's own MXFP8 chain.
"""
import numpy as np
import pytest
import torch

import device_layout
import oracle
from moe_workloads import VARIANTS, Workload, make_inputs, to_f64

from gpu_common import PROB_TOL, announce, assert_close, need_gpu, run_layer
from test_gpu_e4m3 import TOL8, edge_blocks, u8

pytestmark = pytest.mark.gpu

# End-to-end against the oracle's own MXFP8 chain (every intermediate fp64):
# the device stores a, b, h, o, dO, [da|db], dXp in bf16 between products,
# and a value moving across a code boundary changes its block's rounding.
# The oracle alone, with bf16 storage inserted at the device's points, differs
# from its pure chain by up to 6.9 % (y, dX) and 16.9 % (dW) row max on these
# workloads, so the chain comparison uses 0.1 and 0.25; every product on the
# same quantised inputs is held to 6e-2 (measured: about 4e-3).
CHAIN_TOL = 0.1
CHAIN_DW_TOL = 0.25


@pytest.fixture(autouse=True)
def _gpu(request):
    need_gpu()
    announce(request.node.nodeid)
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,cols", [(1, 128), (37, 384), (1000, 4096)])
def test_quantize_rows_mx_bit_exact(dtype, rows, cols):
    import token_routed_expert_amd as tre
    rng = np.random.default_rng(rows * 5 + cols)
    X = edge_blocks(rows, cols, rng)
    X[0, :32] = 448.0 * 2.0 ** 3 * (1 + 2.0 ** -23)      # just above a power-of-two boundary
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    src = torch.from_numpy(X.astype(np.float32)).to(dt)
    codes = torch.empty(rows, cols, dtype=torch.uint8, device="cuda")
    sb = torch.empty(rows, cols // 32, dtype=torch.uint8, device="cuda")
    tre.moe_quantize_rows_mx(src.cuda(), codes, sb)
    rq, rs = oracle.quant_mx_rows(src.float().numpy())
    assert np.array_equal(u8(codes), rq)
    assert np.array_equal(u8(sb), rs)


def test_quantize_weights_mx_bit_exact():
    import token_routed_expert_amd as tre
    E, R, C = 3, 256, 384
    rng = np.random.default_rng(6)
    W = (rng.standard_normal((E, R, C)) / 64 * 2.0 ** rng.integers(-8, 8, (E, R, 1))).astype(
        np.float32)
    W[1, :128, :128] = 0.0
    W[1, 128:, :128] = -0.0
    W[2, :128, 128:256] = edge_blocks(128, 128, rng).astype(np.float32)
    Wt = torch.from_numpy(W).cuda()
    t = {n: torch.empty(*shape, dtype=torch.uint8, device="cuda") for n, shape in
         (("q", (E, R, C)), ("s", (E, R, C // 32)), ("qt", (E, C, R)), ("st", (E, C, R // 32)))}
    tre.moe_quantize_weights_mx(Wt, t["q"], t["s"], t["qt"], t["st"])
    rq, rs, rqt, rst = oracle.quant_mx_weights(W)
    assert np.array_equal(u8(t["q"]), rq)
    assert np.array_equal(u8(t["s"]), rs)
    assert np.array_equal(u8(t["qt"]), rqt)
    assert np.array_equal(u8(t["st"]), rst)


@pytest.mark.parametrize("gather", [False, True])
def test_quantize_token_blocks_mx_bit_exact(gather):
    import token_routed_expert_amd as tre
    rng = np.random.default_rng(21 + gather)
    m = np.array([300, 0, 128, 77, 1, 256, 0, 129, 33])
    off = np.concatenate([[0], np.cumsum(m)]).astype(np.int32)
    E, P, C = len(m), int(off[-1]), 384
    if gather:
        T = 500
        src_np = edge_blocks(T, C, rng)
        src_row = rng.integers(0, T, P).astype(np.int32)
    else:
        src_np = edge_blocks(P, C, rng)
        src_row = None
    src = torch.from_numpy(src_np.astype(np.float32)).to(torch.bfloat16)
    cap = tre.moe_token_block_capacity(P, E)
    blk = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    codes = torch.full((P, C), 0xAB, dtype=torch.uint8, device="cuda")
    sbt = torch.full((cap, C, 4), 0xCD, dtype=torch.uint8, device="cuda")
    tre.moe_quantize_token_blocks_mx(torch.from_numpy(off).cuda(), E, P, src.cuda(),
                                     None if src_row is None else torch.from_numpy(src_row).cuda(),
                                     blk, codes, sbt)
    vals = src.float().numpy()[src_row] if gather else src.float().numpy()
    rq, rs = oracle.quant_mx_token_blocks(vals, off)
    NB = int(oracle.token_block_offsets(off)[-1])
    assert np.array_equal(blk.cpu().numpy(), oracle.token_block_offsets(off))
    # codes in the matrix's own row-major layout; the scale words taken apart
    # (indexing only)
    assert np.array_equal(u8(codes), rq)
    assert np.array_equal(device_layout.mx_token_block_scales(u8(sbt)[:NB], off), rs)
    # the same pass with the 1 x 32 row blocks: rows as moe_quantize_rows_mx
    codes2 = torch.full((P, C), 0xAB, dtype=torch.uint8, device="cuda")
    sbt2 = torch.full((cap, C, 4), 0xCD, dtype=torch.uint8, device="cuda")
    rcodes = torch.full((P, C), 0xEF, dtype=torch.uint8, device="cuda")
    rsb = torch.full((P, C // 32), 0x11, dtype=torch.uint8, device="cuda")
    tre.moe_quantize_token_blocks_with_rows_mx(
        torch.from_numpy(off).cuda(), E, P, src.cuda(),
        None if src_row is None else torch.from_numpy(src_row).cuda(), blk, codes2, sbt2, rcodes, rsb)
    assert torch.equal(codes2, codes) and torch.equal(sbt2[:NB], sbt[:NB])
    rowq, rows_b = oracle.quant_mx_rows(vals)
    assert np.array_equal(u8(rcodes), rowq)
    assert np.array_equal(u8(rsb), rows_b)


def test_permute_mx_bit_exact():
    import token_routed_expert_amd as tre
    T, E, k, d = 777, 64, 6, 512
    g = torch.Generator().manual_seed(9)
    L = torch.randn(T, E, generator=g)
    codes = torch.randint(0, 256, (T, d), generator=g, dtype=torch.uint8)
    sb = torch.randint(0, 256, (T, d // 32), generator=g, dtype=torch.uint8)
    sh = tre.make_shape(T, d, E, k, 128, 0, "mxfp8")
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    prob = torch.empty(T, k, dtype=torch.float32, device="cuda")
    tre.moe_route(L.cuda(), k, idx, prob)
    P = T * k
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    row_of = torch.empty(T, k, dtype=torch.int32, device="cuda")
    token_of = torch.empty(P, dtype=torch.int32, device="cuda")
    dq = torch.empty(P, d, dtype=torch.uint8, device="cuda")
    ds = torch.empty(P, d // 32, dtype=torch.uint8, device="cuda")
    ws = torch.empty(max(256, tre.moe_workspace_bytes(sh, 0)), dtype=torch.uint8, device="cuda")
    tre.moe_permute_mx(sh, codes.cuda(), sb.cuda(), idx, 1, counts, offsets, row_of, token_of,
                       dq, ds, ws)
    ridx, _ = oracle.route(L.numpy(), k)
    _, roff, rrow, rtok = oracle.permute_map(ridx, E)
    assert np.array_equal(row_of.cpu().numpy(), rrow)
    assert np.array_equal(u8(dq), codes.numpy()[rtok])
    assert np.array_equal(u8(ds), sb.numpy()[rtok])


def weights_dequant(wmx, inp, experts=None):
    """Bit-exact check of the device's MX weights against the oracle, and the
    oracle's dequantised row-blocked / column-blocked weights."""
    rowd, cold = {}, {}
    for n in ("W1", "W3", "W2"):
        W = inp[n].cpu().numpy() if experts is None else inp[n][experts].cpu().numpy()
        sel = (lambda t: t) if experts is None else (lambda t: t[experts])
        rq, rs, rqt, rst = oracle.quant_mx_weights(W)
        assert np.array_equal(u8(sel(wmx[n])), rq), n
        assert np.array_equal(u8(sel(wmx[n + "s"])), rs), n + "s"
        assert np.array_equal(u8(sel(wmx[n + "t"])), rqt), n + "t"
        assert np.array_equal(u8(sel(wmx[n + "ts"])), rst), n + "ts"
        rowd[n] = oracle.dequant_mx_weights(rq, rs)
        cold[n] = oracle.dequant_mx_weights(rqt, rst)
    return rowd, cold


def check_layer_mx(wl, inp, b, tol=TOL8):
    """Every stage of the MXFP8 layer against the oracle on the device's own
    quantised inputs; returns the errors."""
    errs = {}
    L = inp["logits"].cpu().numpy()
    idx, p = oracle.route(L, wl.k)
    counts, off, row_of, token_of = oracle.permute_map(idx, wl.E)
    assert np.array_equal(b["topk_idx"].cpu().numpy(), idx)
    assert np.abs(b["topk_prob"].cpu().numpy() - p).max() <= PROB_TOL
    assert np.array_equal(b["offsets"].cpu().numpy(), off)
    assert np.array_equal(b["row_of"].cpu().numpy(), row_of)
    assert np.array_equal(b["token_of"].cpu().numpy(), token_of)
    xq, xs = oracle.quant_mx_rows(inp["x"].float().cpu().numpy())
    assert np.array_equal(u8(b["xq"]), xq)
    assert np.array_equal(u8(b["xs"]), xs)
    assert np.array_equal(u8(b["xpq"]), xq[token_of])
    assert np.array_equal(u8(b["xps"]), xs[token_of])
    rowd, cold = weights_dequant(b["wmx"], inp)
    f = wl.f
    ab = to_f64(b["ab"]); a_g, b_g = ab[:, :f], ab[:, f:]
    a_r, b_r = oracle.fc1_fwd_mx(u8(b["xpq"]), u8(b["xps"]), off, cold["W1"], cold["W3"])
    errs["a"] = assert_close("a", a_g, a_r, tol)
    errs["b"] = assert_close("b", b_g, b_r, tol)
    errs["h"] = assert_close("h", to_f64(b["h"]), oracle.silu(a_r) * b_r, tol)
    h_g = to_f64(b["h"])
    errs["o"] = assert_close("o", to_f64(b["o"]), oracle.fc2_fwd_mx(h_g, off, cold["W2"]), tol)
    errs["y"] = assert_close("y", to_f64(b["y"]), oracle.combine(to_f64(b["o"]), row_of, p), tol)
    dO_g = to_f64(b["dO"])
    da_r, db_r = oracle.fc2_dgrad_mx(dO_g, a_g, b_g, off, rowd["W2"])
    dab_g = to_f64(b["dab"])
    errs["da"] = assert_close("da", dab_g[:, :f], da_r, tol)
    errs["db"] = assert_close("db", dab_g[:, f:], db_r, tol)
    errs["dXp"] = assert_close("dXp", to_f64(b["dXp"]),
                               oracle.fc1_dgrad_mx(dab_g, off, rowd["W1"], rowd["W3"]), tol)
    errs["dX"] = assert_close("dX", to_f64(b["dX"]), oracle.combine(to_f64(b["dXp"]), row_of), tol)
    errs["dW2"] = assert_close("dW2", to_f64(b["dW2"]), oracle.wgrad_mx(h_g, dO_g, off), tol)
    dW13 = oracle.wgrad_mx(to_f64(inp["x"])[token_of], dab_g, off)
    errs["dW1"] = assert_close("dW1", to_f64(b["dW1"]), dW13[:, :, :f], tol)
    errs["dW3"] = assert_close("dW3", to_f64(b["dW3"]), dW13[:, :, f:], tol)
    for e in np.nonzero(counts == 0)[0]:
        assert not b["dW1"][int(e)].any() and not b["dW3"][int(e)].any()
        assert not b["dW2"][int(e)].any()
    return errs


SMALLMX = [
    Workload("mx_tiny", T=64, d=128, E=4, k=2, f=128, dtype="mxfp8"),
    Workload("mx_ragged", T=300, d=256, E=8, k=2, f=384, dtype="mxfp8"),
    Workload("mx_skew", T=700, d=384, E=16, k=4, f=256, dtype="mxfp8", skew=True),
    Workload("mx_k_eq_E", T=129, d=256, E=4, k=4, f=128, dtype="mxfp8"),
    Workload("mx_one_token", T=1, d=128, E=8, k=3, f=256, dtype="mxfp8"),
]


@pytest.mark.parametrize("wl", SMALLMX, ids=lambda w: w.name)
def test_layer_mx_small(wl):
    inp = make_inputs(wl, seed=1, device="cuda")
    if wl.k == wl.E:
        inp["logits"] = inp["logits"] * 0.1
    b = run_layer(wl, inp)
    errs = check_layer_mx(wl, inp, b)
    announce(f"{wl.name}: max errors " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    h = {n: inp[n].cpu().numpy() for n in ("W1", "W3", "W2")}
    x = inp["x"].float().cpu().numpy()
    st = oracle.layer_fwd_mx(inp["logits"].cpu().numpy(), x, h["W1"], h["W3"], h["W2"], wl.k)
    g = oracle.layer_bwd_mx(st, x, inp["dY"].float().cpu().numpy())
    for n, ref, tol in (("y", st["y"], CHAIN_TOL), ("dX", g["dX"], CHAIN_TOL),
                        ("dW1", g["dW1"], CHAIN_DW_TOL),
                        ("dW3", g["dW3"], CHAIN_DW_TOL), ("dW2", g["dW2"], CHAIN_DW_TOL)):
        assert_close(f"chain {n}", to_f64(b[n]), ref, tol)


def test_layer_mx_one_expert_takes_all():
    wl = Workload("mx_all_to_one", T=333, d=256, E=8, k=1, f=256, dtype="mxfp8")
    inp = make_inputs(wl, seed=4, device="cuda")
    inp["logits"][:, 5] += 100.0
    b = run_layer(wl, inp)
    check_layer_mx(wl, inp, b)
    assert int(b["counts"][5]) == wl.T


def test_layer_mx_deterministic():
    wl = SMALLMX[2]
    inp = make_inputs(wl, seed=2, device="cuda")
    b1 = run_layer(wl, inp)
    b2 = run_layer(wl, inp)
    for n in ("y", "dX", "dW1", "dW3", "dW2", "ab", "h", "xpq", "dab"):
        assert torch.equal(b1[n], b2[n]), n


def test_layer_mx_with_router_grad():
    """The router gradient and the loss on an MXFP8 layer (dprob against the
    layer's own expert outputs, as for the other dtypes)."""
    wl = SMALLMX[2]
    inp = make_inputs(wl, seed=5, device="cuda")
    b = run_layer(wl, inp, router_grad=True, aux_alpha=0.01)
    plain = run_layer(wl, inp)
    for n in ("y", "dX", "dW1", "dW3", "dW2"):
        assert torch.equal(plain[n], b[n]), n
    L = inp["logits"].cpu().numpy()
    ridx, rp = oracle.route(L, wl.k)
    counts = b["counts"].cpu().numpy()
    ref_loss, ref_aux = oracle.aux_loss(L, counts, wl.k, 0.01)
    assert abs(float(b["aux_loss"].item()) - ref_loss) <= 5e-5 * ref_loss
    dp = b["dprob"].cpu().numpy().astype(np.float64)
    dp_ref = oracle.combine_dprob(to_f64(inp["dY"]), to_f64(b["o"]), b["row_of"].cpu().numpy())
    mag = oracle.combine_dprob(np.abs(to_f64(inp["dY"])), np.abs(to_f64(b["o"])),
                               b["row_of"].cpu().numpy())
    assert (np.abs(dp - dp_ref) <= 1e-5 * mag + 1e-30).all()
    ref = oracle.router_bwd(dp, rp, ridx, wl.E) + ref_aux
    assert_close("dlogits", b["dlogits"].cpu().numpy().astype(np.float64), ref, 1e-4)


def test_layer_mx_full_size_sampled():
    """The skewed shape (T=8200, d=4096, E=128, k=8, f=1536) with MXFP8
    operands in the benchmark's launch configuration: routing, map and x
    quantisation in full; weights and every product on sampled experts."""
    wl = VARIANTS["skewed_mxfp8"]
    announce("skewed_mxfp8: inputs")
    inp = make_inputs(wl, seed=0, device="cuda")
    announce("skewed_mxfp8: layer fwd+bwd")
    b = run_layer(wl, inp)
    L = inp["logits"].cpu().numpy()
    idx, p = oracle.route(L, wl.k)
    counts, off, row_of, token_of = oracle.permute_map(idx, wl.E)
    assert (counts == 0).sum() >= 10
    assert np.array_equal(b["topk_idx"].cpu().numpy(), idx)
    assert np.array_equal(b["offsets"].cpu().numpy(), off)
    assert np.array_equal(b["token_of"].cpu().numpy(), token_of)
    announce("skewed_mxfp8: x codes")
    xq, xs = oracle.quant_mx_rows(inp["x"].float().cpu().numpy())
    assert np.array_equal(u8(b["xq"]), xq)
    assert np.array_equal(u8(b["xs"]), xs)
    tok = torch.from_numpy(token_of.astype(np.int64)).cuda()
    assert torch.equal(b["xpq"], b["xq"][tok]) and torch.equal(b["xps"], b["xs"][tok])
    f = wl.f
    nonempty = np.nonzero(counts)[0]
    order = nonempty[np.argsort(counts[nonempty])]
    for e in [int(order[-1]), int(order[len(order) // 2]), int(order[0])]:
        announce(f"skewed_mxfp8: expert {e} ({counts[e]} rows)")
        r0, r1 = int(off[e]), int(off[e + 1])
        R = slice(r0, r1)
        o1 = np.array([0, r1 - r0])
        rowd, cold = weights_dequant(b["wmx"], inp, experts=[e])
        ab = to_f64(b["ab"][r0:r1]); a_g, b_g = ab[:, :f], ab[:, f:]
        a_r, b_r = oracle.fc1_fwd_mx(u8(b["xpq"][r0:r1]), u8(b["xps"][r0:r1]), o1, cold["W1"],
                                     cold["W3"])
        assert_close(f"a[{e}]", a_g, a_r, TOL8)
        assert_close(f"b[{e}]", b_g, b_r, TOL8)
        h_g = to_f64(b["h"][r0:r1])
        assert_close(f"o[{e}]", to_f64(b["o"][r0:r1]), oracle.fc2_fwd_mx(h_g, o1, cold["W2"]), TOL8)
        dO_g = to_f64(b["dO"][r0:r1])
        da_r, db_r = oracle.fc2_dgrad_mx(dO_g, a_g, b_g, o1, rowd["W2"])
        dab_g = to_f64(b["dab"][r0:r1])
        assert_close(f"da[{e}]", dab_g[:, :f], da_r, TOL8)
        assert_close(f"db[{e}]", dab_g[:, f:], db_r, TOL8)
        assert_close(f"dXp[{e}]", to_f64(b["dXp"][r0:r1]),
                     oracle.fc1_dgrad_mx(dab_g, o1, rowd["W1"], rowd["W3"]), TOL8)
        assert_close(f"dW2[{e}]", to_f64(b["dW2"][e]), oracle.wgrad_mx(h_g, dO_g, o1)[0], TOL8)
        xe = to_f64(inp["x"][tok[R]])
        dW13 = oracle.wgrad_mx(xe, dab_g, o1)[0]
        assert_close(f"dW1[{e}]", to_f64(b["dW1"][e]), dW13[:, :f], TOL8)
        assert_close(f"dW3[{e}]", to_f64(b["dW3"][e]), dW13[:, f:], TOL8)
    for e in np.nonzero(counts == 0)[0]:
        assert not b["dW1"][int(e)].any() and not b["dW2"][int(e)].any()
    for t in [0, wl.T - 1, 4100]:
        y_t = sum(p[t, j] * to_f64(b["o"][int(row_of[t, j])]) for j in range(wl.k))
        assert_close(f"y[{t}]", to_f64(b["y"][t])[None], y_t[None], TOL8)
