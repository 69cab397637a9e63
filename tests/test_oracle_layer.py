"""Pins of the whole-layer oracle (shared dense MLP + routed branch), CPU only:
a hand-worked example, limits with closed forms, invariants, and the layer
sum reducing to either branch when the other one is zeroed."""
import json
import os

import numpy as np

from oracle import omni_layer as OL
from oracle import omni_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _mlp(L=5, d=6, d_ff=7, seed=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((L, d))
    wg = rng.standard_normal((d_ff, d)) / np.sqrt(d)
    wu = rng.standard_normal((d_ff, d)) / np.sqrt(d)
    wd = rng.standard_normal((d, d_ff)) / np.sqrt(d_ff)
    return x, wg, wu, wd


def test_hand_worked_example():
    fx = json.load(open(os.path.join(GOLDEN, "shared_mlp_example.json")))
    got = OL.shared_mlp_f64(np.array(fx["x"]), np.array(fx["w_gate"]), np.array(fx["w_up"]),
                            np.array(fx["w_down"]))
    np.testing.assert_allclose(got, np.array(fx["expect_y"]), rtol=0, atol=fx["abs_tol"])


def test_zero_up_or_down_projection_gives_zero():
    x, wg, wu, wd = _mlp()
    assert np.abs(OL.shared_mlp_f64(x, wg, np.zeros_like(wu), wd)).max() == 0
    assert np.abs(OL.shared_mlp_f64(x, wg, wu, np.zeros_like(wd))).max() == 0


def test_single_hidden_unit_closed_form():
    x, wg, wu, wd = _mlp(d_ff=1, seed=3)
    g = x @ wg[0]
    u = x @ wu[0]
    want = (g / (1 + np.exp(-g)) * u)[:, None] * wd[:, 0][None, :]
    np.testing.assert_allclose(OL.shared_mlp_f64(x, wg, wu, wd), want, rtol=1e-13, atol=1e-15)


def test_saturated_gate_is_a_relu_on_the_gate_projection():
    # silu(c z) / c -> max(z, 0) as c grows: the scaled branch becomes
    # sum_j relu(x . wg_j) (x . wu_j) Wd[:, j], which tells the gate from the up
    # projection (a swap puts the relu on the wrong factor)
    _, _, wu, wd = _mlp(L=5, d=5, d_ff=9, seed=4)
    x = np.eye(5)                          # gate values = entries of wg, |.| >= 0.1
    rng = np.random.default_rng(6)
    wg = rng.choice([-1.0, 1.0], size=(9, 5)) * (0.1 + rng.random((9, 5)))
    c = 1e3
    with np.errstate(over="ignore"):       # exp(-c z) = inf for z < 0 gives silu = -0
        got = OL.shared_mlp_f64(x, c * wg, wu, wd) / c
    want = (np.maximum(x @ wg.T, 0) * (x @ wu.T)) @ wd.T
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_loop_form_matches():
    x, wg, wu, wd = _mlp(L=3, d=4, d_ff=5, seed=8)
    np.testing.assert_allclose(OL.shared_mlp_f64(x, wg, wu, wd),
                               OL.shared_mlp_literal(x, wg, wu, wd), rtol=1e-12, atol=1e-14)


def test_homogeneous_in_up_and_down_and_token_equivariant():
    x, wg, wu, wd = _mlp(L=6, seed=9)
    m = OL.shared_mlp_f64(x, wg, wu, wd)
    np.testing.assert_allclose(OL.shared_mlp_f64(x, wg, 2.5 * wu, wd), 2.5 * m, rtol=1e-12)
    np.testing.assert_allclose(OL.shared_mlp_f64(x, wg, wu, -3.0 * wd), -3.0 * m, rtol=1e-12)
    perm = np.random.default_rng(1).permutation(6)
    np.testing.assert_allclose(OL.shared_mlp_f64(x[perm], wg, wu, wd), m[perm], rtol=1e-12)


def _layer_problem(seed=0):
    rng = np.random.default_rng(seed)
    L, d, Nr, Nc, d_ff = 12, 16, 6, 5, 24
    f = lambda *s: rng.standard_normal(s).astype(np.float32)
    return dict(x=f(L, d), wr_t=f(Nr, d) / 4, wc_t=f(Nc, d) / 4, w=f(Nr * Nc, d) / 4,
                v=f(Nr * Nc, d) / 4, w_gate=f(d_ff, d) / 4, w_up=f(d_ff, d) / 4,
                w_down=f(d, d_ff) / 5)


def test_layer_reduces_to_each_branch():
    p = _layer_problem()
    kw = dict(kprime=4, K=4, B=3)
    zero_down = dict(p, w_down=np.zeros_like(p["w_down"]))
    out = OL.layer_forward(**zero_down, **kw)
    routed = O.forward(p["x"], p["wr_t"], p["wc_t"], p["w"], p["v"], 4, 4, 3)
    np.testing.assert_array_equal(out["expert_idx"], routed["expert_idx"])
    np.testing.assert_array_equal(out["y"], routed["y"])
    zero_w = dict(p, w=np.zeros_like(p["w"]))
    out = OL.layer_forward(**zero_w, **kw)
    np.testing.assert_array_equal(out["y"], OL.shared_mlp(p["x"], p["w_gate"], p["w_up"],
                                                          p["w_down"]))


def test_layer_is_the_sum_of_its_branches():
    p = _layer_problem(seed=2)
    out = OL.layer_forward(**p, kprime=5, K=4, B=2)
    both = out["y_routed"] + out["y_shared"]
    np.testing.assert_allclose(out["y"], both, rtol=1e-6, atol=1e-6)
    assert np.abs(out["y_routed"]).max() > 0 and np.abs(out["y_shared"]).max() > 0
