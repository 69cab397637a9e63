"""Pins of the oracle's scheduling and execution stages: a hand-worked
schedule, count identities and ordering invariants, the traffic model, the
closed-form single-expert case, linearity, and the expert-centric order
computing the same function as the token-centric one."""
import math

import numpy as np
import pytest

from oracle import omni_oracle as O
from synth import custom, make_inputs, normal
from tests.conftest import load_golden


def test_schedule_golden_worked_example():
    g = load_golden("schedule_worked_example.json")
    s = O.build_schedule(np.array(g["expert_idx"]), np.array(g["gate"], np.float32),
                         g["N"], g["B"])
    e = g["expect"]
    assert s["n_active"] == e["n_active"] and s["n_groups"] == e["n_groups"]
    for key in ("active", "group_offsets", "task_index", "task_token", "task_expert"):
        assert list(s[key]) == e[key], key
    np.testing.assert_array_equal(s["task_gate"], np.array(e["task_gate"], np.float32))
    L, K = np.array(g["expert_idx"]).shape
    tr = O.traffic_elements(g["d"], L, K, s["n_active"])
    assert tr["token_centric"] == e["traffic_token_centric"]
    assert tr["expert_centric"] == e["traffic_expert_centric"]


def _random_routing(L, K, N, seed, hot=0):
    rng = np.random.default_rng(seed)
    idx = np.empty((L, K), np.int64)
    for t in range(L):
        if hot:
            pool = rng.choice(min(N, hot), size=K, replace=False)
        else:
            pool = rng.choice(N, size=K, replace=False)
        idx[t] = pool
    gate = rng.random((L, K)).astype(np.float32)
    return idx.astype(np.int32), gate


@pytest.mark.parametrize("L,K,N,B,hot", [(37, 5, 200, 7, 0), (64, 8, 1024, 16, 0),
                                         (50, 6, 64, 64, 0), (40, 4, 4096, 3, 30),
                                         (1, 1, 1, 1, 0), (9, 3, 10, 1, 0)])
def test_schedule_invariants(L, K, N, B, hot):
    idx, gate = _random_routing(L, K, N, seed=L + K + N + B, hot=hot)
    s = O.build_schedule(idx, gate, N, B)
    M = L * K
    G = O.max_groups(N, L, K, B)
    offs = s["group_offsets"]
    assert len(offs) == G + 1 and offs[0] == 0 and offs[-1] == M
    assert (np.diff(offs) >= 0).all()
    assert (offs[s["n_groups"]:] == M).all()
    # the sorted tasks are a permutation of the flat task list
    assert sorted(s["task_index"]) == list(range(M))
    np.testing.assert_array_equal(s["task_token"], s["task_index"] // K)
    np.testing.assert_array_equal(s["task_expert"], idx.reshape(-1)[s["task_index"]])
    np.testing.assert_array_equal(s["task_gate"], gate.reshape(-1)[s["task_index"]])
    # active list: strictly increasing, exactly the set of used experts
    act = s["active"]
    assert (np.diff(act) > 0).all() and set(act) == set(idx.reshape(-1))
    assert s["n_groups"] == math.ceil(len(act) / B)
    for g in range(s["n_groups"]):
        lo, hi = offs[g], offs[g + 1]
        ex = s["task_expert"][lo:hi]
        members = act[g * B:(g + 1) * B]
        assert set(ex) == set(members)                  # group = B consecutive actives
        assert len(set(ex)) <= B
        assert (np.diff(s["task_token"][lo:hi]) >= 0).all()   # tokens ascending
        # ties inside one (group, token) keep flatten order
        ti = s["task_index"][lo:hi]
        tok = s["task_token"][lo:hi]
        for a_, b_, ta, tb in zip(ti[:-1], ti[1:], tok[:-1], tok[1:]):
            if ta == tb:
                assert a_ < b_
    # groups are disjoint contiguous id ranges
    for g in range(s["n_groups"] - 1):
        assert act[min(len(act) - 1, (g + 1) * B - 1)] < act[(g + 1) * B]


def test_window_grouping_golden_worked_examples():
    g = load_golden("schedule_window_example.json")
    for ex in g["examples"]:
        idx = np.array(ex["expert_idx"])
        gate = np.array(ex["gate"], np.float32)
        s = O.build_schedule(idx, gate, ex["N"], ex["B"], grouping="window")
        e = ex["expect"]
        assert s["n_groups"] == e["n_groups"]
        for key in ("group_offsets", "task_index", "task_token", "task_expert"):
            assert list(s[key]) == e[key], (ex["note"], key)
        np.testing.assert_array_equal(s["task_gate"], np.array(e["task_gate"], np.float32))
        if "expect_active_grouping" in ex:
            r = O.build_schedule(idx, gate, ex["N"], ex["B"])
            assert r["n_groups"] == ex["expect_active_grouping"]["n_groups"]
            assert list(r["task_index"]) == ex["expect_active_grouping"]["task_index"]


@pytest.mark.parametrize("L,K,N,B,hot", [(37, 5, 200, 7, 0), (40, 4, 4096, 3, 30),
                                         (50, 6, 64, 64, 0), (9, 3, 10, 1, 0),
                                         (1, 1, 1, 1, 0), (12, 4, 100, 1000, 0)])
def test_window_grouping_invariants(L, K, N, B, hot):
    idx, gate = _random_routing(L, K, N, seed=3 * L + K + N + B, hot=hot)
    s = O.build_schedule(idx, gate, N, B, grouping="window")
    M = L * K
    G = O.max_groups(N, L, K, B, "window")
    assert s["n_groups"] == G == math.ceil(N / B)
    offs = s["group_offsets"]
    assert len(offs) == G + 1 and offs[0] == 0 and offs[-1] == M
    assert sorted(s["task_index"]) == list(range(M))
    for g in range(G):
        lo, hi = offs[g], offs[g + 1]
        ex = s["task_expert"][lo:hi]
        assert ((ex >= g * B) & (ex < (g + 1) * B)).all()       # the id window
        # every task of the window is in the group
        assert hi - lo == int(((idx >= g * B) & (idx < (g + 1) * B)).sum())
        assert (np.diff(s["task_token"][lo:hi]) >= 0).all()
        ti, tok = s["task_index"][lo:hi], s["task_token"][lo:hi]
        assert all(a_ < b_ for a_, b_, ta, tb in zip(ti[:-1], ti[1:], tok[:-1], tok[1:])
                   if ta == tb)
    # B = 1: windows are single experts, the same order as ranking the actives
    if B == 1:
        r = O.build_schedule(idx, gate, N, 1)
        np.testing.assert_array_equal(s["task_index"], r["task_index"])
    # one window holding every expert: flatten order unchanged
    if B >= N:
        np.testing.assert_array_equal(s["task_index"], np.arange(M))


def test_expert_centric_equals_token_centric_and_counts_traffic():
    # The ablation table of the explainer: removing expert-centric scheduling
    # leaves model quality unchanged -> both orders compute the same y.
    wl = custom(L=48, d=32, Nr=8, Nc=16, kprime=6, K=6, B=5)
    inp = make_inputs(wl)
    out = O.forward(inp["x"], inp["wr"], inp["wc"], inp["w"], inp["v"], 6, 6, 5)
    s = out["schedule"]
    y_tok = O.atomic_forward_f64(inp["x"], inp["w"], inp["v"], out["expert_idx"], out["gate"])
    y_exp, loaded = O.atomic_forward_expert_centric(inp["x"], inp["w"], inp["v"], s, 48,
                                                    count_loads=True)
    np.testing.assert_allclose(y_exp, y_tok, rtol=1e-12, atol=1e-12)
    tr = O.traffic_elements(32, 48, 6, s["n_active"])
    assert loaded == tr["expert_centric"] == 2 * 32 * s["n_active"]
    assert tr["token_centric"] == 2 * 32 * 48 * 6
    # literal scalar loop agrees with the vectorised sum
    y_lit = O.atomic_forward_literal(inp["x"], inp["w"], inp["v"], out["expert_idx"], out["gate"])
    np.testing.assert_allclose(y_lit, y_tok, rtol=1e-12, atol=1e-12)


def test_single_expert_closed_form():
    x = normal((1, 16), 1)
    w = normal((3, 16), 2)
    v = normal((3, 16), 3)
    y = O.atomic_forward_f64(x, w, v, np.array([[2]]), np.array([[1.0]], np.float32))
    h = float(np.dot(x[0].astype(np.float64), w[2].astype(np.float64)))
    np.testing.assert_allclose(y[0], h / (1 + math.exp(-h)) * v[2].astype(np.float64),
                               rtol=1e-14)


def test_zero_w_gives_zero_and_y_is_linear_in_v():
    wl = custom(L=10, d=16, Nr=4, Nc=4, kprime=3, K=3, B=2)
    inp = make_inputs(wl)
    out = O.forward(inp["x"], inp["wr"], inp["wc"], inp["w"], inp["v"], 3, 3, 2)
    idx, g = out["expert_idx"], out["gate"]
    z = O.atomic_forward_f64(inp["x"], np.zeros_like(inp["w"]), inp["v"], idx, g)
    assert np.all(z == 0)
    v2 = normal(inp["v"].shape, 99)
    y1 = O.atomic_forward_f64(inp["x"], inp["w"], inp["v"], idx, g)
    y2 = O.atomic_forward_f64(inp["x"], inp["w"], v2, idx, g)
    y3 = O.atomic_forward_f64(inp["x"], inp["w"], 2 * inp["v"].astype(np.float64) + v2, idx, g)
    np.testing.assert_allclose(y3, 2 * y1 + y2, atol=1e-12)


def test_golden_atomic_expert_sum():
    g = load_golden("atomic_expert_example.json")
    y = O.atomic_forward_f64(np.array(g["x"]), np.array(g["w"]), np.array(g["v"]),
                             np.array(g["expert_idx"]), np.array(g["gate"], np.float32))
    np.testing.assert_allclose(y, np.array(g["expect_y"]), rtol=0, atol=g["abs_tol"])


def test_token_permutation_equivariance():
    # Routing and the expert sum act per token: permuting the tokens permutes y.
    wl = custom(L=20, d=32, Nr=8, Nc=8, kprime=4, K=4, B=3)
    inp = make_inputs(wl)
    perm = np.random.default_rng(0).permutation(20)
    o1 = O.forward(inp["x"], inp["wr"], inp["wc"], inp["w"], inp["v"], 4, 4, 3)
    o2 = O.forward(inp["x"][perm], inp["wr"], inp["wc"], inp["w"], inp["v"], 4, 4, 3)
    np.testing.assert_array_equal(o2["expert_idx"], o1["expert_idx"][perm])
    np.testing.assert_array_equal(o2["y"], o1["y"][perm])


def test_full_tiny_workload_runs_fast():
    from synth import WORKLOADS
    import time
    wl = WORKLOADS["tiny"]
    inp = make_inputs(wl)
    t0 = time.time()
    out = O.forward(inp["x"], inp["wr"], inp["wc"], inp["w"], inp["v"], wl.kprime, wl.K, wl.B)
    assert time.time() - t0 < 5
    assert out["y"].shape == (64, 128)
    s = out["schedule"]
    assert s["group_offsets"][-1] == 64 * 8
    # factored == brute force on the real tiny workload (k' = K)
    bidx, _ = O.brute_force_topk(out["a"], out["b"], wl.K)
    np.testing.assert_array_equal(out["expert_idx"], bidx)
