"""Pins of the backward oracle (CPU only): central finite differences of a
float64 forward with the selection held fixed, closed forms, invariants."""
import numpy as np
import pytest

from oracle import omni_backward as OB
from oracle import omni_oracle as O


def _problem(L=3, d=6, Nr=4, Nc=5, K=3, seed=0, bias=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((L, d))
    wr = rng.standard_normal((Nr, d)) / np.sqrt(d)
    wc = rng.standard_normal((Nc, d)) / np.sqrt(d)
    w = rng.standard_normal((Nr * Nc, d)) / np.sqrt(d) * 2.0
    v = rng.standard_normal((Nr * Nc, d)) / np.sqrt(d)
    rb = rng.standard_normal(Nr) * 0.3 if bias else None
    cb = rng.standard_normal(Nc) * 0.3 if bias else None
    idx = np.stack([rng.choice(Nr * Nc, K, replace=False) for _ in range(L)]).astype(np.int32)
    dy = rng.standard_normal((L, d))
    return x, wr, wc, w, v, rb, cb, idx, dy


def _loss(p, idx, dy):
    y, _ = OB.forward_fixed_f64(p["x"], p["wr"], p["wc"], p["w"], p["v"], idx, p["rb"], p["cb"])
    return float((y * dy).sum())


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_backward_matches_finite_differences(seed):
    x, wr, wc, w, v, rb, cb, idx, dy = _problem(seed=seed)
    p = {"x": x, "wr": wr, "wc": wc, "w": w, "v": v, "rb": rb, "cb": cb}
    _, g = OB.forward_fixed_f64(x, wr, wc, w, v, idx, rb, cb)
    gr = OB.backward(x, wr, wc, w, v, idx, g, dy, rb, cb)
    # dense dW / dV from the active-row form
    N, d = w.shape
    dw = np.zeros((N, d))
    dv = np.zeros((N, d))
    dw[gr["active"]] = gr["dw"]
    dv[gr["active"]] = gr["dv"]
    analytic = {"x": gr["dx"], "wr": gr["dwr"], "wc": gr["dwc"], "w": dw, "v": dv,
                "rb": gr["drb"], "cb": gr["dcb"]}
    eps = 1e-6
    for name, arr in p.items():
        num = np.zeros_like(arr)
        flat = arr.reshape(-1)
        for i in range(flat.size):
            keep = flat[i]
            flat[i] = keep + eps
            up = _loss(p, idx, dy)
            flat[i] = keep - eps
            dn = _loss(p, idx, dy)
            flat[i] = keep
            num.reshape(-1)[i] = (up - dn) / (2 * eps)
        err = np.abs(num - analytic[name]).max()
        scale = max(1.0, np.abs(num).max())
        assert err <= 1e-6 * scale, (name, err, scale)


def test_single_expert_closed_form():
    # K = 1: the gate is 1 whatever the score, so the router gets no gradient
    rng = np.random.default_rng(7)
    d = 5
    x = rng.standard_normal((1, d))
    w = rng.standard_normal((6, d))
    v = rng.standard_normal((6, d))
    wr = rng.standard_normal((2, d))
    wc = rng.standard_normal((3, d))
    dy = rng.standard_normal((1, d))
    idx = np.array([[4]], np.int32)
    gr = OB.backward(x, wr, wc, w, v, idx, np.ones((1, 1)), dy)
    h = float(w[4] @ x[0])
    s = h / (1 + np.exp(-h))
    sg = 1 / (1 + np.exp(-h))
    ds = sg * (1 + h * (1 - sg))
    u = float(dy[0] @ v[4])
    np.testing.assert_allclose(gr["dv"][0], s * dy[0], rtol=1e-12)
    np.testing.assert_allclose(gr["dw"][0], u * ds * x[0], rtol=1e-12)
    np.testing.assert_allclose(gr["dx"][0], u * ds * w[4], rtol=1e-12, atol=1e-15)
    assert np.abs(gr["dwr"]).max() == 0 and np.abs(gr["dwc"]).max() == 0
    assert np.abs(gr["dscore"]).max() == 0


def test_silu_grad_is_the_derivative():
    h = np.linspace(-8, 8, 101)
    eps = 1e-6
    num = (O.silu(h + eps) - O.silu(h - eps)) / (2 * eps)
    np.testing.assert_allclose(OB.silu_grad(h), num, rtol=1e-8, atol=1e-10)


def test_log_softmax_correction_vanishes():
    # sum_k dS_k = 0 (softmax backward), so every row of da sums to zero and the
    # log-softmax backward returns da itself: the router logit gradient is
    # sparse, nonzero only on the rows / columns of selected experts
    x, wr, wc, w, v, rb, cb, idx, dy = _problem(L=6, d=8, Nr=7, Nc=6, K=5, seed=3)
    _, g = OB.forward_fixed_f64(x, wr, wc, w, v, idx, rb, cb)
    gr = OB.backward(x, wr, wc, w, v, idx, g, dy, rb, cb)
    assert np.abs(gr["dscore"].sum(axis=1)).max() < 1e-14
    da, db = OB.score_backward(idx, gr["dscore"], 7, 6)
    assert np.abs(gr["dzr"] - da).max() < 1e-14
    assert np.abs(gr["dzc"] - db).max() < 1e-14
    sel_rows = np.zeros((6, 7), bool)
    for t in range(6):
        sel_rows[t, idx[t] // 6] = True
    assert np.abs(gr["dzr"][~sel_rows]).max() < 1e-14


def test_backward_is_linear_in_dy():
    x, wr, wc, w, v, rb, cb, idx, dy = _problem(seed=5)
    _, g = OB.forward_fixed_f64(x, wr, wc, w, v, idx, rb, cb)
    dy2 = np.random.default_rng(9).standard_normal(dy.shape)
    a = OB.backward(x, wr, wc, w, v, idx, g, dy, rb, cb)
    b = OB.backward(x, wr, wc, w, v, idx, g, dy2, rb, cb)
    c = OB.backward(x, wr, wc, w, v, idx, g, dy + 2 * dy2, rb, cb)
    for k in ("dx", "dwr", "dwc", "drb", "dcb", "dw", "dv", "dgate"):
        np.testing.assert_allclose(c[k], a[k] + 2 * b[k], rtol=1e-10, atol=1e-12)


def test_gates_of_the_fixed_forward_match_the_product_topk_gates():
    # the fixed-selection forward uses the same gate definition as the oracle's
    # forward when the selection is the product top-K's own
    x, wr, wc, w, v, rb, cb, _, dy = _problem(L=4, d=8, Nr=6, Nc=6, K=4, seed=11)
    a, b = O.router_logp(x.astype(np.float32), wr.astype(np.float32), wc.astype(np.float32),
                         rb.astype(np.float32), cb.astype(np.float32))
    idx, score, gate, _, _ = O.product_topk(a, b, 6, 4)
    _, g = OB.forward_fixed_f64(x.astype(np.float32).astype(np.float64),
                                wr.astype(np.float32).astype(np.float64),
                                wc.astype(np.float32).astype(np.float64), w, v, idx,
                                rb.astype(np.float32).astype(np.float64),
                                cb.astype(np.float32).astype(np.float64))
    np.testing.assert_allclose(g, gate, rtol=2e-6, atol=1e-7)


def test_log_softmax_backward_matches_finite_differences():
    # a general upstream gradient (not summing to zero), so the correction
    # term matters here
    rng = np.random.default_rng(4)
    z = rng.standard_normal((3, 7))
    dl = rng.standard_normal((3, 7))
    got = OB.log_softmax_backward(z, dl)
    eps = 1e-6
    num = np.zeros_like(z)
    for i in range(z.size):
        zp = z.copy().reshape(-1)
        zm = z.copy().reshape(-1)
        zp[i] += eps
        zm[i] -= eps
        num.reshape(-1)[i] = ((O.log_softmax_rows(zp.reshape(z.shape)) * dl).sum()
                              - (O.log_softmax_rows(zm.reshape(z.shape)) * dl).sum()) / (2 * eps)
    np.testing.assert_allclose(got, num, rtol=1e-7, atol=1e-9)
