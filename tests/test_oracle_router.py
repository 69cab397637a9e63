"""Pins of the oracle's router stages (log-probabilities, per-axis search,
product top-K, gates) against facts that do not come from the oracle itself:
one-hot and identity special cases, closed forms, invariants, brute force over
all N cells on tiny grids, and hand-worked fixtures."""
import math

import numpy as np
import pytest

from oracle import omni_oracle as O
from synth import normal, custom, make_inputs, f32_to_bf16_bits, bf16_bits_to_f32
from tests.conftest import load_golden


# ------------------------------------------------------------------ O1 / O2


def test_onehot_input_reads_router_columns():
    # x = e_c picks the weights of input feature c for every grid row / column.
    # Non-square Nr != Nc != d so a transposed operand cannot pass.
    d, Nr, Nc = 7, 5, 3
    wr = normal((Nr, d), 11)
    wc = normal((Nc, d), 12)
    x = np.eye(d, dtype=np.float32)
    zr, zc = O.router_logits_f64(x, wr, wc)
    for c in range(d):
        np.testing.assert_array_equal(zr[c], wr[:, c].astype(np.float64))
        np.testing.assert_array_equal(zc[c], wc[:, c].astype(np.float64))


def test_identity_router_returns_input():
    d = Nr = Nc = 16
    x = normal((9, d), 3)
    eye = np.eye(d, dtype=np.float32)
    zr, zc = O.router_logits_f64(x, eye, eye)
    np.testing.assert_array_equal(zr, x.astype(np.float64))
    np.testing.assert_array_equal(zc, x.astype(np.float64))


def test_bias_only_router_recovers_log_probabilities():
    # x = 0 leaves only the bias; a bias equal to log p of a distribution p
    # must come back as log p (closed form of the log-softmax).
    rng = np.random.default_rng(5)
    Nr, Nc, d = 6, 4, 8
    pr = rng.random(Nr) + 0.1
    pr /= pr.sum()
    pc = rng.random(Nc) + 0.1
    pc /= pc.sum()
    x = np.zeros((2, d), np.float32)
    a, b = O.router_logp(x, normal((Nr, d), 1), normal((Nc, d), 2),
                         np.log(pr), np.log(pc))
    np.testing.assert_allclose(a, np.log(pr)[None].repeat(2, 0), rtol=0, atol=2e-7)
    np.testing.assert_allclose(b, np.log(pc)[None].repeat(2, 0), rtol=0, atol=2e-7)


def test_log_softmax_normalises_and_is_shift_invariant():
    wl = custom(L=13, d=32, Nr=8, Nc=16, kprime=4, K=4, B=4)
    inp = make_inputs(wl, ("x", "wr", "wc"))
    a, b = O.router_logp(inp["x"], inp["wr"], inp["wc"])
    for t in (a, b):
        s = np.exp(t.astype(np.float64)).sum(axis=1)
        np.testing.assert_allclose(s, 1.0, atol=1e-6)
        assert (t <= 0).all()
    # a constant bias shifts every logit of a row: log-probabilities unchanged
    a2, b2 = O.router_logp(inp["x"], inp["wr"], inp["wc"],
                           np.full(8, 3.5, np.float32), np.full(16, -2.0, np.float32))
    np.testing.assert_allclose(a2, a, atol=1e-6)
    np.testing.assert_allclose(b2, b, atol=1e-6)
    # uniform logits: log(1/n)
    u, _ = O.router_logp(np.zeros((1, 32), np.float32), inp["wr"], inp["wc"])
    np.testing.assert_allclose(u, math.log(1 / 8), atol=1e-7)


def test_router_is_linear_in_x():
    wl = custom(L=5, d=24, Nr=6, Nc=10, kprime=2, K=2, B=2)
    inp = make_inputs(wl, ("x", "wr", "wc"))
    x2 = normal((5, 24), 77)
    z1 = O.router_logits_f64(inp["x"], inp["wr"], inp["wc"])
    z2 = O.router_logits_f64(x2, inp["wr"], inp["wc"])
    z12 = O.router_logits_f64(inp["x"].astype(np.float64) + x2, inp["wr"], inp["wc"])
    for p, q, r in zip(z1, z2, z12):
        np.testing.assert_allclose(p + q, r, atol=1e-12)


def test_bf16_inputs_are_widened_exactly():
    f = normal((3, 8), 9)
    bits = f32_to_bf16_bits(f)
    np.testing.assert_array_equal(O.widen(bits), bf16_bits_to_f32(bits).astype(np.float64))
    # round to nearest even on a constructed halfway case: 1 + 2^-8 -> 1.0
    half = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8], np.float32)
    np.testing.assert_array_equal(bf16_bits_to_f32(f32_to_bf16_bits(half)),
                                  np.array([1.0, 1.0 + 2.0 ** -6], np.float32))


# ------------------------------------------------------------------ O3


def _rank_by_counting(row):
    # rank(i) = #{j : v_j > v_i} + #{j < i : v_j == v_i}  (brute force, O(n^2))
    n = len(row)
    return [sum(1 for j in range(n) if row[j] > row[i]) +
            sum(1 for j in range(i) if row[j] == row[i]) for i in range(n)]


@pytest.mark.parametrize("quant", [0.0, 0.5])
def test_axis_topk_matches_counting_ranks(quant):
    rng = np.random.default_rng(1)
    logp = rng.standard_normal((20, 37)).astype(np.float32)
    if quant:
        logp = (np.round(logp / quant) * quant).astype(np.float32)   # many ties
    for k in (1, 5, 37):
        idx, val = O.axis_topk(logp, k)
        for t in range(logp.shape[0]):
            r = _rank_by_counting(list(logp[t]))
            want = sorted(range(37), key=lambda i: r[i])[:k]
            assert list(idx[t]) == want
            np.testing.assert_array_equal(val[t], logp[t][want])


def test_axis_topk_golden_ties():
    g = load_golden("axis_order_ties.json")
    for c in g["cases"]:
        idx, _ = O.axis_topk(np.array([c["row"]], np.float32), c["k"])
        assert list(idx[0]) == c["expect_idx"], c


# ------------------------------------------------------------------ O4


def _tiny_logp(L, Nr, Nc, seed, quant=0.0):
    rng = np.random.default_rng(seed)
    zr = rng.standard_normal((L, Nr))
    zc = rng.standard_normal((L, Nc))
    if quant:
        zr = np.round(zr / quant) * quant
        zc = np.round(zc / quant) * quant
    return O.log_softmax_rows(zr).astype(np.float32), O.log_softmax_rows(zc).astype(np.float32)


@pytest.mark.parametrize("Nr,Nc,kp,K", [(4, 8, 4, 4), (8, 4, 3, 3), (6, 6, 6, 5),
                                        (5, 7, 5, 1), (16, 16, 8, 8), (9, 3, 3, 3)])
@pytest.mark.parametrize("quant", [0.0, 0.25])
def test_factored_topk_equals_brute_force(Nr, Nc, kp, K, quant):
    # Theorem: with k' >= K the per-axis search loses nothing, because any cell
    # outside the k' x k' block is dominated by at least K cells inside it.
    kp = max(kp, min(K, min(Nr, Nc)))
    if K > kp * kp:
        pytest.skip("K > k'^2")
    a, b = _tiny_logp(50, Nr, Nc, seed=Nr * 100 + Nc * 10 + K, quant=quant)
    if kp < K:
        pytest.skip("needs k' >= K")
    idx, score, *_ = O.product_topk(a, b, kp, K)
    bidx, bscore = O.brute_force_topk(a, b, K)
    np.testing.assert_array_equal(idx, bidx)
    np.testing.assert_array_equal(score, bscore)


def test_rounding_collapse_is_the_documented_exception():
    # fl32(a1 + b) == fl32(a0 + b) although a1 > a0: the brute force sees a tie
    # and keeps the lower id e = 0; the factored search already cut row 0.
    a0 = np.float32(-1.0)
    a1 = np.nextafter(a0, np.float32(0))                  # a1 > a0 by one ulp
    b0 = np.float32(-1e4)
    assert np.float32(a0 + b0) == np.float32(a1 + b0)
    a = np.array([[a0, a1, np.float32(-50.0)]], np.float32)
    b = np.array([[b0, np.float32(-2e4), np.float32(-3e4)]], np.float32)
    idx, *_ = O.product_topk(a, b, 1, 1)
    bidx, _ = O.brute_force_topk(a, b, 1)
    assert int(idx[0, 0]) == 1 * 3 + 0        # factored: row 1 (a1), column 0
    assert int(bidx[0, 0]) == 0               # brute force: tie -> lower e


def test_product_topk_structure():
    a, b = _tiny_logp(40, 32, 16, seed=3)
    kp = K = 8
    idx, score, gate, R, C = O.product_topk(a, b, kp, K)
    Nc = 16
    for t in range(40):
        assert len(set(idx[t])) == K and (idx[t] < 32 * 16).all()
        assert (np.diff(score[t]) <= 0).all()
        for k in range(K):
            i, j = divmod(int(idx[t, k]), Nc)
            assert score[t, k] == np.float32(a[t, i] + b[t, j])
            r = list(R[t]).index(i)
            c = list(C[t]).index(j)
            assert (r + 1) * (c + 1) <= K          # staircase (no ties here)


# ------------------------------------------------------------------ O5


def test_gates_are_a_normalised_product_of_axis_probabilities():
    a, b = _tiny_logp(30, 12, 20, seed=8)
    idx, score, gate, *_ = O.product_topk(a, b, 6, 6)
    Nc = 20
    np.testing.assert_allclose(gate.astype(np.float64).sum(1), 1.0, atol=1e-6)
    assert (np.diff(gate, axis=1) <= 0).all()
    # independent route: p_r[i] * p_c[j] renormalised over the selected cells
    pr = np.exp(a.astype(np.float64))
    pc = np.exp(b.astype(np.float64))
    i, j = np.divmod(idx.astype(np.int64), Nc)
    prod = np.take_along_axis(pr, i, 1) * np.take_along_axis(pc, j, 1)
    np.testing.assert_allclose(gate, prod / prod.sum(1, keepdims=True), rtol=2e-6, atol=1e-7)


def test_single_expert_gate_is_one():
    a, b = _tiny_logp(7, 5, 5, seed=2)
    _, _, gate, *_ = O.product_topk(a, b, 1, 1)
    np.testing.assert_array_equal(gate, 1.0)


def test_router_cost_ratio_matches_printed_value():
    g = load_golden("router_cost_ratio.json")
    pct = 100 * O.router_cost_ratio(g["Nr"], g["Nc"])
    assert g["Nr"] * g["Nc"] == g["N"]
    assert round(pct, g["printed_decimals"]) == g["printed_percent"]
