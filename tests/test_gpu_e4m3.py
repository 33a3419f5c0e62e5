"""e4m3 path vs the oracle, through the C ABI, on seeded synthetic inputs.

* Quantisers (1 x 128 rows, 128 x 128 weight tiles, per-expert 128-row token
  blocks) and the e4m3 permutation: codes and scales bit-exact.
* Expert GEMM products: within 6e-2 (max over rows of max|gpu-ref| /
  max|ref|) of the oracle run on the same quantised inputs -- the oracle
  quantises the device's own stored intermediates (xp codes, h, dO, [da|db]),
  and the quantiser tests above prove its codes equal the device's.
* The whole layer is also compared with the oracle's own e4m3 chain.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_workloads import WORKLOADS, Workload, make_inputs, to_f64

from gpu_common import PROB_TOL, announce, assert_close, need_gpu, run_layer

pytestmark = pytest.mark.gpu

TOL8 = 6e-2
# The oracle's own e4m3 chain (every intermediate kept in fp64) and the
# device chain (a, b, h, dO, [da|db] stored bf16 between products) quantise
# slightly different values.  Weight gradients are sums over an expert's rows
# of terms with mixed signs, each operand quantised in 128-row blocks per
# column, so one code flipping between the chains moves a sum by a sizeable
# fraction of itself: on these inputs the oracle's chain with bf16 storage
# inserted at the device's points differs from the pure chain by up to 9.4 %
# (row max) in dW, and either chain differs from the unquantised gradient by
# about 15 %.  The end-to-end dW comparison therefore uses 0.15; each product
# on the same quantised inputs is held to 6e-2 above.
CHAIN_DW_TOL = 0.15


@pytest.fixture(autouse=True)
def _gpu(request):
    need_gpu()
    announce(request.node.nodeid)
    yield
    torch.cuda.synchronize()


def u8(t):
    return t.detach().cpu().numpy().astype(np.uint8)


def f32bits(t):
    return t.detach().cpu().contiguous().view(torch.int32).numpy()


def np32bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.int32)


# ---------------------------------------------------------------- inputs with edge cases
def edge_blocks(rows, cols, rng):
    """fp32 [rows][cols] whose 128-blocks include: all +0, all -0, exact
    rounding ties (block max 448 * 2^s, so scale = 2^s), the subnormal range
    of the codes, values that saturate after the scale division, blocks so
    small that their scale lies below 2^-90 (some of them with subnormal
    values or a subnormal scale), and plain normals over a wide exponent
    range."""
    X = rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-20, 20, (rows, 1)))
    nb = cols // 128
    kinds = rng.integers(0, 7, size=(rows, nb))
    for r in range(rows):
        for b in range(nb):
            blk = X[r, 128 * b:128 * (b + 1)]
            k = kinds[r, b]
            s = float(np.exp2(rng.integers(-12, 12)))
            if k == 0:
                blk[:] = 0.0
            elif k == 1:
                blk[:] = -0.0
            elif k == 2:   # ties between neighbouring codes, normal and subnormal ranges
                m = rng.integers(0, 8, 128)
                e = rng.integers(-6, 8, 128)
                tie = (1.0 + (m + 0.5) / 8.0) * np.exp2(e)
                sub = (rng.integers(0, 8, 128) + 0.5) * 2.0 ** -9
                blk[:] = np.where(rng.random(128) < 0.7, tie, sub) * s
                blk[:] *= np.where(rng.random(128) < 0.5, 1.0, -1.0)
                blk[0] = 448.0 * s
            elif k == 3:   # tiny values next to one large one: codes 0, 0x80, subnormals
                blk[:] = rng.standard_normal(128) * s * 2.0 ** -12
                blk[5] = -448.0 * s
            elif k == 4:   # a single non-zero value
                blk[:] = 0.0
                blk[rng.integers(0, 128)] = rng.standard_normal() * s
            elif k == 5:   # tiny block: scale 2^-104 .. 2^-130, a few subnormal values
                blk[:] = rng.standard_normal(128) * np.exp2(rng.integers(-122, -95))
                blk[rng.integers(0, 128, 8)] *= 2.0 ** -20
    return X


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,cols", [(1, 128), (37, 384), (1000, 4096)])
def test_quantize_rows_bit_exact(dtype, rows, cols):
    import token_routed_expert_amd as tre
    rng = np.random.default_rng(rows * 7 + cols)
    X = edge_blocks(rows, cols, rng)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    src = torch.from_numpy(X.astype(np.float32)).to(dt)
    codes = torch.empty(rows, cols, dtype=torch.uint8, device="cuda")
    scales = torch.empty(rows, cols // 128, dtype=torch.float32, device="cuda")
    tre.moe_quantize_rows(src.cuda(), codes, scales)
    rq, rs = oracle.quant_rows(src.float().numpy())
    assert np.array_equal(u8(codes), rq)
    assert np.array_equal(f32bits(scales), np32bits(rs))


def test_quantize_weights_bit_exact():
    import token_routed_expert_amd as tre
    E, R, C = 3, 256, 384
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((E, R, C)) / 64).astype(np.float32)
    W[1, :128, :128] = 0.0           # zero tile
    W[1, 128:, :128] = -0.0          # negative-zero tile
    W[2, :128, 128:256] = edge_blocks(128, 128, rng).astype(np.float32)
    W[0, 128:, 256:] = rng.standard_normal((128, 128)) * 2.0 ** -110   # scale below 2^-90
    Wt = torch.from_numpy(W).cuda()
    codes = torch.empty(E, R, C, dtype=torch.uint8, device="cuda")
    codes_t = torch.empty(E, C, R, dtype=torch.uint8, device="cuda")
    scales = torch.empty(E, R // 128, C // 128, dtype=torch.float32, device="cuda")
    tre.moe_quantize_weights(Wt, codes, codes_t, scales)
    rq, rs = oracle.quant_expert_weights(W)
    # without the transposed copy (what the layer writes): the same codes
    codes1 = torch.empty_like(codes)
    tre.moe_quantize_weights(Wt, codes1, None, torch.empty_like(scales))
    assert torch.equal(codes1, codes)
    assert np.array_equal(u8(codes), rq)
    assert np.array_equal(u8(codes_t), rq.transpose(0, 2, 1))
    assert np.array_equal(f32bits(scales), np32bits(rs))


@pytest.mark.parametrize("gather", [False, True])
def test_quantize_token_blocks_bit_exact(gather):
    import token_routed_expert_amd as tre
    rng = np.random.default_rng(11 + gather)
    m = np.array([300, 0, 128, 77, 1, 256, 0, 129])
    off = np.concatenate([[0], np.cumsum(m)]).astype(np.int32)
    E, P, C = len(m), int(off[-1]), 384
    # expert 5 reads only rows scaled by 2^-112: its blocks' scales lie below 2^-90
    if gather:
        T = 500
        src_np = edge_blocks(T, C, rng)
        src_np[:50] *= 2.0 ** -112
        src_row = rng.integers(50, T, P).astype(np.int32)
        src_row[off[5]:off[6]] = rng.integers(0, 50, m[5])
    else:
        src_np = edge_blocks(P, C, rng)
        src_np[off[5]:off[6]] *= 2.0 ** -112
        src_row = None
    src = torch.from_numpy(src_np.astype(np.float32)).to(torch.bfloat16)
    cap = tre.moe_token_block_capacity(P, E)
    blk = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    codes = torch.full((P, C), 0xAB, dtype=torch.uint8, device="cuda")
    scales = torch.empty(cap, C, dtype=torch.float32, device="cuda")
    tre.moe_quantize_token_blocks(torch.from_numpy(off).cuda(), E, P, src.cuda(),
                                  None if src_row is None else torch.from_numpy(src_row).cuda(),
                                  blk, codes, scales)
    vals = src.float().numpy()[src_row] if gather else src.float().numpy()
    rq, rs = oracle.quant_token_blocks(vals, off)
    rblk = oracle.token_block_offsets(off)
    assert np.array_equal(blk.cpu().numpy(), rblk)
    NB = int(rblk[-1])
    assert np.array_equal(f32bits(scales)[:NB], np32bits(rs))
    # codes in the matrix's own row-major layout: every row written
    assert np.array_equal(u8(codes), rq)
    # the same pass with the row blocks: token blocks unchanged, rows as moe_quantize_rows
    codes2 = torch.full((P, C), 0xAB, dtype=torch.uint8, device="cuda")
    scales2 = torch.empty(cap, C, dtype=torch.float32, device="cuda")
    rcodes = torch.full((P, C), 0xCD, dtype=torch.uint8, device="cuda")
    rscales = torch.empty(P, C // 128, dtype=torch.float32, device="cuda")
    tre.moe_quantize_token_blocks_with_rows(
        torch.from_numpy(off).cuda(), E, P, src.cuda(),
        None if src_row is None else torch.from_numpy(src_row).cuda(), blk, codes2, scales2,
        rcodes, rscales)
    assert torch.equal(codes2, codes) and torch.equal(scales2[:NB], scales[:NB])
    rowq, rows_s = oracle.quant_rows(vals)
    assert np.array_equal(u8(rcodes), rowq)
    assert np.array_equal(f32bits(rscales), np32bits(rows_s))


def test_permute_e4m3_bit_exact():
    import token_routed_expert_amd as tre
    T, E, k, d = 777, 64, 6, 512
    g = torch.Generator().manual_seed(3)
    L = torch.randn(T, E, generator=g)
    codes = torch.randint(0, 256, (T, d), generator=g, dtype=torch.uint8)
    scales = torch.rand(T, d // 128, generator=g)
    sh = tre.make_shape(T, d, E, k, 128, 0, "e4m3")
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    prob = torch.empty(T, k, dtype=torch.float32, device="cuda")
    tre.moe_route(L.cuda(), k, idx, prob)
    P = T * k
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    row_of = torch.empty(T, k, dtype=torch.int32, device="cuda")
    token_of = torch.empty(P, dtype=torch.int32, device="cuda")
    dq = torch.empty(P, d, dtype=torch.uint8, device="cuda")
    ds = torch.empty(P, d // 128, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(256, tre.moe_workspace_bytes(sh, 0)), dtype=torch.uint8, device="cuda")
    tre.moe_permute_e4m3(sh, codes.cuda(), scales.cuda(), idx, 1, counts, offsets, row_of, token_of,
                         dq, ds, ws)
    ridx, _ = oracle.route(L.numpy(), k)
    _, roff, rrow, rtok = oracle.permute_map(ridx, E)
    assert np.array_equal(offsets.cpu().numpy(), roff)
    assert np.array_equal(row_of.cpu().numpy(), rrow)
    assert np.array_equal(u8(dq), codes.numpy()[rtok])
    assert np.array_equal(f32bits(ds), scales.numpy().view(np.int32)[rtok])


# ---------------------------------------------------------------- layer
def check_layer_e4m3(wl, inp, b, tol=TOL8):
    """Every stage of the e4m3 layer against the oracle on the device's own
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
    # activation quantisation and its permutation, bit-exact
    xq, xs = oracle.quant_rows(inp["x"].float().cpu().numpy())
    assert np.array_equal(u8(b["xq"]), xq)
    assert np.array_equal(f32bits(b["xs"]), np32bits(xs))
    assert np.array_equal(u8(b["xpq"]), xq[token_of])
    assert np.array_equal(f32bits(b["xps"]), np32bits(xs)[token_of])
    # weights, bit-exact
    wq = b["wq"]
    Wd = {}
    for n in ("W1", "W3", "W2"):
        rq, rs = oracle.quant_expert_weights(inp[n].cpu().numpy())
        assert np.array_equal(u8(wq[n]), rq), n
        assert wq[n + "t"] is None            # the products read one orientation
        assert np.array_equal(f32bits(wq[n + "s"]), np32bits(rs)), n + "s"
        Wd[n] = oracle.dequant_expert_weights(rq, rs)
    f = wl.f
    ab = to_f64(b["ab"]); a_g, b_g = ab[:, :f], ab[:, f:]
    a_r, b_r = oracle.fc1_fwd_e4m3(u8(b["xpq"]), b["xps"].cpu().numpy(), off, Wd["W1"], Wd["W3"])
    errs["a"] = assert_close("a", a_g, a_r, tol)
    errs["b"] = assert_close("b", b_g, b_r, tol)
    errs["h"] = assert_close("h", to_f64(b["h"]), oracle.silu(a_r) * b_r, tol)
    h_g = to_f64(b["h"])
    errs["o"] = assert_close("o", to_f64(b["o"]), oracle.fc2_fwd_e4m3(h_g, off, Wd["W2"]), tol)
    errs["y"] = assert_close("y", to_f64(b["y"]), oracle.combine(to_f64(b["o"]), row_of, p), tol)
    dO_g = to_f64(b["dO"])
    errs["dO"] = assert_close("dO", dO_g, oracle.permute_scaled(to_f64(inp["dY"]), row_of, p), tol)
    da_r, db_r = oracle.fc2_dgrad_e4m3(dO_g, a_g, b_g, off, Wd["W2"])
    dab_g = to_f64(b["dab"])
    errs["da"] = assert_close("da", dab_g[:, :f], da_r, tol)
    errs["db"] = assert_close("db", dab_g[:, f:], db_r, tol)
    errs["dXp"] = assert_close("dXp", to_f64(b["dXp"]),
                               oracle.fc1_dgrad_e4m3(dab_g, off, Wd["W1"], Wd["W3"]), tol)
    errs["dX"] = assert_close("dX", to_f64(b["dX"]), oracle.combine(to_f64(b["dXp"]), row_of), tol)
    dW2 = oracle.wgrad_e4m3(h_g, dO_g, off)
    errs["dW2"] = assert_close("dW2", to_f64(b["dW2"]), dW2, tol)
    dW13 = oracle.wgrad_e4m3(to_f64(inp["x"])[token_of], dab_g, off)
    errs["dW1"] = assert_close("dW1", to_f64(b["dW1"]), dW13[:, :, :f], tol)
    errs["dW3"] = assert_close("dW3", to_f64(b["dW3"]), dW13[:, :, f:], tol)
    for e in np.nonzero(counts == 0)[0]:
        assert not b["dW1"][int(e)].any() and not b["dW3"][int(e)].any()
        assert not b["dW2"][int(e)].any()
    return errs


SMALL8 = [
    Workload("e4m3_tiny", T=64, d=128, E=4, k=2, f=128, dtype="e4m3"),
    Workload("e4m3_ragged", T=300, d=256, E=8, k=2, f=384, dtype="e4m3"),
    Workload("e4m3_skew", T=700, d=384, E=16, k=4, f=256, dtype="e4m3", skew=True),
    Workload("e4m3_k_eq_E", T=129, d=256, E=4, k=4, f=128, dtype="e4m3"),
    Workload("e4m3_one_token", T=1, d=128, E=8, k=3, f=256, dtype="e4m3"),
]


@pytest.mark.parametrize("wl", SMALL8, ids=lambda w: w.name)
def test_layer_e4m3_small(wl):
    inp = make_inputs(wl, seed=1, device="cuda")
    if wl.k == wl.E:
        inp["logits"] = inp["logits"] * 0.1
    b = run_layer(wl, inp)
    errs = check_layer_e4m3(wl, inp, b)
    announce(f"{wl.name}: max errors " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    # the oracle's own e4m3 chain end to end
    h = {n: inp[n].cpu().numpy() for n in ("W1", "W3", "W2")}
    x = inp["x"].float().cpu().numpy()
    st = oracle.layer_fwd_e4m3(inp["logits"].cpu().numpy(), x, h["W1"], h["W3"], h["W2"], wl.k)
    g = oracle.layer_bwd_e4m3(st, x, inp["dY"].float().cpu().numpy())
    chain = {}
    for n, ref, tol in (("y", st["y"], TOL8), ("dX", g["dX"], TOL8), ("dW1", g["dW1"], CHAIN_DW_TOL),
                        ("dW3", g["dW3"], CHAIN_DW_TOL), ("dW2", g["dW2"], CHAIN_DW_TOL)):
        chain[n] = assert_close(f"chain {n}", to_f64(b[n]), ref, tol)
    announce(f"{wl.name}: oracle's own chain vs device " +
             ", ".join(f"{k}={v:.2e}" for k, v in chain.items()))


def test_layer_e4m3_one_expert_takes_all():
    wl = Workload("e4m3_all_to_one", T=333, d=256, E=8, k=1, f=256, dtype="e4m3")
    inp = make_inputs(wl, seed=4, device="cuda")
    inp["logits"][:, 5] += 100.0
    b = run_layer(wl, inp)
    check_layer_e4m3(wl, inp, b)
    assert int(b["counts"][5]) == wl.T


def test_layer_e4m3_deterministic():
    wl = SMALL8[2]
    inp = make_inputs(wl, seed=2, device="cuda")
    b1 = run_layer(wl, inp)
    b2 = run_layer(wl, inp)
    for n in ("y", "dX", "dW1", "dW3", "dW2", "ab", "h", "xpq", "dab"):
        assert torch.equal(b1[n], b2[n]), n


def test_layer_e4m3_full_size_sampled():
    """The skewed fp8 workload (T=8200, d=4096, E=128, k=8, f=1536) in the
    benchmark's launch configuration: routing, map and x quantisation in full;
    weights and every product on sampled experts (hottest, median, smallest
    non-empty), whose operands the oracle takes from the device's stored
    intermediates; empty experts get zero weight gradients."""
    wl = WORKLOADS["skewed_fp8"]
    announce("skewed_fp8: inputs")
    inp = make_inputs(wl, seed=0, device="cuda")
    announce("skewed_fp8: layer fwd+bwd")
    b = run_layer(wl, inp)
    announce("skewed_fp8: routing, map, x codes")
    L = inp["logits"].cpu().numpy()
    idx, p = oracle.route(L, wl.k)
    counts, off, row_of, token_of = oracle.permute_map(idx, wl.E)
    assert (counts == 0).sum() >= 10
    assert np.array_equal(b["topk_idx"].cpu().numpy(), idx)
    assert np.array_equal(b["offsets"].cpu().numpy(), off)
    assert np.array_equal(b["row_of"].cpu().numpy(), row_of)
    assert np.array_equal(b["token_of"].cpu().numpy(), token_of)
    xq, xs = oracle.quant_rows(inp["x"].float().cpu().numpy())
    assert np.array_equal(u8(b["xq"]), xq)
    assert np.array_equal(f32bits(b["xs"]), np32bits(xs))
    tok = torch.from_numpy(token_of.astype(np.int64)).cuda()
    assert torch.equal(b["xpq"], b["xq"][tok]) and torch.equal(b["xps"], b["xs"][tok])
    f = wl.f
    nonempty = np.nonzero(counts)[0]
    order = nonempty[np.argsort(counts[nonempty])]
    for e in [int(order[-1]), int(order[len(order) // 2]), int(order[0])]:
        announce(f"skewed_fp8: expert {e} ({counts[e]} rows)")
        r0, r1 = int(off[e]), int(off[e + 1])
        R = slice(r0, r1)
        o1 = np.array([0, r1 - r0])
        wq = b["wq"]
        Wd = {}
        for n in ("W1", "W3", "W2"):
            rq, rs = oracle.quant_tiles(inp[n][e].cpu().numpy())
            assert np.array_equal(u8(wq[n][e]), rq), n
            assert np.array_equal(f32bits(wq[n + "s"][e]), np32bits(rs)), n + "s"
            Wd[n] = oracle.dequant_tiles(rq, rs)[None]
        ab = to_f64(b["ab"][r0:r1]); a_g, b_g = ab[:, :f], ab[:, f:]
        a_r, b_r = oracle.fc1_fwd_e4m3(u8(b["xpq"][r0:r1]), b["xps"][r0:r1].cpu().numpy(), o1,
                                       Wd["W1"], Wd["W3"])
        assert_close(f"a[{e}]", a_g, a_r, TOL8)
        assert_close(f"b[{e}]", b_g, b_r, TOL8)
        h_g = to_f64(b["h"][r0:r1])
        assert_close(f"h[{e}]", h_g, oracle.silu(a_r) * b_r, TOL8)
        assert_close(f"o[{e}]", to_f64(b["o"][r0:r1]), oracle.fc2_fwd_e4m3(h_g, o1, Wd["W2"]), TOL8)
        dO_g = to_f64(b["dO"][r0:r1])
        da_r, db_r = oracle.fc2_dgrad_e4m3(dO_g, a_g, b_g, o1, Wd["W2"])
        dab_g = to_f64(b["dab"][r0:r1])
        assert_close(f"da[{e}]", dab_g[:, :f], da_r, TOL8)
        assert_close(f"db[{e}]", dab_g[:, f:], db_r, TOL8)
        assert_close(f"dXp[{e}]", to_f64(b["dXp"][r0:r1]),
                     oracle.fc1_dgrad_e4m3(dab_g, o1, Wd["W1"], Wd["W3"]), TOL8)
        assert_close(f"dW2[{e}]", to_f64(b["dW2"][e]), oracle.wgrad_e4m3(h_g, dO_g, o1)[0], TOL8)
        xe = to_f64(inp["x"][tok[R]])
        dW13 = oracle.wgrad_e4m3(xe, dab_g, o1)[0]
        assert_close(f"dW1[{e}]", to_f64(b["dW1"][e]), dW13[:, :f], TOL8)
        assert_close(f"dW3[{e}]", to_f64(b["dW3"][e]), dW13[:, f:], TOL8)
    for e in np.nonzero(counts == 0)[0]:
        assert not b["dW1"][int(e)].any() and not b["dW2"][int(e)].any()
    announce("skewed_fp8: combine on sampled tokens")
    for t in [0, wl.T - 1, 4100]:
        y_t = sum(p[t, j] * to_f64(b["o"][int(row_of[t, j])]) for j in range(wl.k))
        assert_close(f"y[{t}]", to_f64(b["y"][t])[None], y_t[None], TOL8)
        dX_t = sum(to_f64(b["dXp"][int(row_of[t, j])]) for j in range(wl.k))
        assert_close(f"dX[{t}]", to_f64(b["dX"][t])[None], dX_t[None], TOL8)
