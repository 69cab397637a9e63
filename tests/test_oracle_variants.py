"""Pins of the variant oracles (CPU only): the SwiGLU-gated atomic expert and
the flat router baseline."""
import numpy as np

from oracle import omni_oracle as O
from oracle import omni_variants as OV
from tests.conftest import load_golden


def test_glu_expert_hand_worked_example():
    g = load_golden("glu_expert_example.json")
    y = OV.atomic_forward_glu_f64(np.array(g["x"]), np.array(g["w"]), np.array(g["u"]),
                                  np.array(g["v"]), np.array(g["expert_idx"]),
                                  np.array(g["gate"], np.float32))
    np.testing.assert_allclose(y, np.array(g["expect_y"]), rtol=0, atol=g["abs_tol"])


def _glu_problem(L=5, d=8, N=20, K=4, seed=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((L, d))
    w, u, v = (rng.standard_normal((N, d)) / np.sqrt(d) for _ in range(3))
    idx = np.stack([rng.choice(N, K, replace=False) for _ in range(L)]).astype(np.int32)
    gate = rng.random((L, K)).astype(np.float32)
    return x, w, u, v, idx, gate


def test_glu_with_unit_up_projection_is_the_silu_expert():
    # u_e = x / (x . x) makes x . u_e = 1: the gated expert becomes the SiLU one
    x, w, u, v, idx, gate = _glu_problem(L=1, seed=1)
    u = np.tile(x[0] / (x[0] @ x[0]), (u.shape[0], 1))
    np.testing.assert_allclose(OV.atomic_forward_glu_f64(x, w, u, v, idx, gate),
                               O.atomic_forward_f64(x, w, v, idx, gate), rtol=1e-12, atol=1e-14)


def test_glu_single_expert_closed_form_and_linearity():
    x, w, u, v, _, _ = _glu_problem(L=3, seed=2)
    idx = np.array([[7], [7], [3]], np.int32)
    gate = np.ones((3, 1), np.float32)
    y = OV.atomic_forward_glu_f64(x, w, u, v, idx, gate)
    for t in range(3):
        e = idx[t, 0]
        a = x[t] @ w[e]
        want = a / (1 + np.exp(-a)) * (x[t] @ u[e]) * v[e]
        np.testing.assert_allclose(y[t], want, rtol=1e-13, atol=1e-15)
    x, w, u, v, idx, gate = _glu_problem(seed=3)
    y = OV.atomic_forward_glu_f64(x, w, u, v, idx, gate)
    np.testing.assert_allclose(OV.atomic_forward_glu_f64(x, w, 3 * u, v, idx, gate), 3 * y,
                               rtol=1e-12)
    np.testing.assert_allclose(OV.atomic_forward_glu_f64(x, w, u, -2 * v, idx, gate), -2 * y,
                               rtol=1e-12)


def test_glu_saturated_gate_tells_w_from_u():
    # silu(c a) / c -> max(a, 0): the relu lands on the x . W factor
    x, w, u, v, idx, gate = _glu_problem(seed=4)
    a = np.einsum("td,tkd->tk", x, w[idx])
    assert np.abs(a).min() > 1e-3
    c = 1e4
    with np.errstate(over="ignore"):
        got = OV.atomic_forward_glu_f64(x, c * w, u, v, idx, gate) / c
    b = np.einsum("td,tkd->tk", x, u[idx])
    want = np.einsum("tk,tkd->td", gate.astype(np.float64) * np.maximum(a, 0) * b, v[idx])
    np.testing.assert_allclose(got, want, rtol=1e-9, atol=1e-12)


def test_flat_router_hand_worked_example():
    g = load_golden("flat_router_example.json")
    logp = O.log_softmax_rows(np.array(g["logits"])).astype(np.float32)
    for key, K in (("K2", 2), ("K3", 3)):
        idx, score, gate = OV.flat_topk(logp, K)
        assert idx.tolist() == g[key]["expert_idx"]
        np.testing.assert_allclose(gate, np.array(g[key]["gate"]), rtol=0, atol=g["gate_tol"])


def test_flat_router_with_additive_logits_is_the_product_router():
    # logits z[i Nc + j] = z_r[i] + z_c[j] make the flat log-softmax the sum of
    # the per-axis ones (the log-sum-exp over the grid factorises), so the flat
    # top-K over all N equals the product top-K over the grid
    rng = np.random.default_rng(5)
    L, d, Nr, Nc, K = 6, 16, 9, 7, 12
    x = rng.standard_normal((L, d)).astype(np.float32)
    wr = (rng.standard_normal((Nr, d)) / 2).astype(np.float32)
    wc = (rng.standard_normal((Nc, d)) / 2).astype(np.float32)
    wf = (wr[:, None, :].astype(np.float64) + wc[None, :, :]).reshape(Nr * Nc, d)
    logp = OV.flat_router_logp(x, wf)
    a, b = O.router_logp(x, wr, wc)
    np.testing.assert_allclose(logp, (a[:, :, None] + b[:, None, :]).reshape(L, -1),
                               rtol=0, atol=2e-5)
    idx, _, gate = OV.flat_topk(logp, K)
    bidx, bscore = O.brute_force_topk(a, b, K)
    bgate = O.gates(bscore)
    np.testing.assert_array_equal(idx, bidx)
    np.testing.assert_allclose(gate, bgate, rtol=0, atol=2e-5)


def test_flat_router_edge_cases():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((4, 8)).astype(np.float32)
    # all logits equal: the K lowest ids, equal gates
    idx, _, gate = OV.flat_topk(OV.flat_router_logp(x, np.zeros((10, 8))), 3)
    assert (idx == np.arange(3)).all()
    np.testing.assert_allclose(gate, 1 / 3, rtol=1e-6)
    # K = N selects every expert; log p sums (in probability) to one
    wf = rng.standard_normal((6, 8)).astype(np.float32)
    logp = OV.flat_router_logp(x, wf)
    np.testing.assert_allclose(np.exp(logp.astype(np.float64)).sum(axis=1), 1, rtol=1e-6)
    idx, _, gate = OV.flat_topk(logp, 6)
    assert all(sorted(r) == list(range(6)) for r in idx.tolist())
    np.testing.assert_allclose(gate.sum(axis=1), 1, rtol=1e-6)


def test_flat_router_bias_is_a_log_prior():
    # Wf = 0 and bias = log p: the logits are the bias, so log p comes back
    # (softmax of log p is p) and the top-K follows p
    rng = np.random.default_rng(8)
    p = rng.random(12) + 0.05
    p /= p.sum()
    x = rng.standard_normal((3, 8)).astype(np.float32)
    logp = OV.flat_router_logp(x, np.zeros((12, 8)), np.log(p).astype(np.float32))
    np.testing.assert_allclose(logp, np.tile(np.log(p), (3, 1)), rtol=0, atol=2e-6)
    idx, _, _ = OV.flat_topk(logp, 4)
    assert (idx == np.argsort(-p, kind="stable")[:4]).all()
