"""The oracle against hand-derived fixtures (tests/golden/): routing and the
permutation map of a tiny case with ties and an empty expert, and a scalar
SwiGLU expert whose forward and backward have closed forms."""
import numpy as np

import oracle
from golden_fixtures import closed_form, fraction, load, logits_f32, LN3


def test_route_permute_tiny():
    fx = load("route_permute_tiny.json")
    idx, p = oracle.route(logits_f32(fx), fx["k"])
    assert np.array_equal(idx, np.array(fx["topk_idx"]))
    want = np.array([[fraction(v) for v in row] for row in fx["topk_prob"]])
    assert np.allclose(p, want, rtol=0, atol=1e-6)   # the logits are float32 roundings of ln 3
    counts, offsets, row_of, token_of = oracle.permute_map(idx, fx["E"])
    assert np.array_equal(counts, fx["counts"])
    assert np.array_equal(offsets, fx["offsets"])
    assert np.array_equal(row_of, np.array(fx["row_of"]))
    assert np.array_equal(token_of, fx["token_of"])


def test_swiglu_scalar_closed_form():
    fx = load("swiglu_scalar.json")
    x = np.array([[fx["x"]]])
    W1 = np.array([[[LN3]]])
    W3 = np.array([[[fx["W3"]]]])
    W2 = np.array([[[fx["W2"]]]])
    offsets = np.array([0, 1])
    a, b, h, o = oracle.experts_fwd(x, offsets, W1, W3, W2)
    e = {k: closed_form(v) for k, v in fx["expect"].items()}
    for name, got in (("a", a), ("b", b), ("h", h), ("o", o)):
        assert abs(float(got.ravel()[0]) - e[name]) < 1e-12, name
    dO = np.array([[fx["dY"]]])          # p = 1 with E = k = 1
    dXp, dW1, dW3, dW2, da, db = oracle.experts_bwd(dO, x, a, b, h, offsets, W1, W3, W2)
    for name, got in (("dX", dXp), ("dW1", dW1), ("dW3", dW3), ("dW2", dW2), ("da", da), ("db", db)):
        assert abs(float(np.asarray(got).ravel()[0]) - e[name]) < 1e-12, name
