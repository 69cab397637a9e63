"""GPU parity of omni_routed_backward against the float64 backward oracle, on
the GPU forward's own selection (expert ids and gates), for seeded upstream
gradients dy.  Active experts bit-exact; every gradient within the forward's
bars (max|d| / max|ref| <= 1e-4 float32, <= 2e-2 bf16)."""
import numpy as np
import pytest
import torch

from oracle import omni_backward as OB
from synth import WORKLOADS, custom, make_inputs
from tests.gpu_helpers import dev, host, log, rel_err

pytestmark = pytest.mark.gpu

B = pytest.importorskip("cartesian_routed_atomic_amd.binding")

TOL = {"f32": 1e-4, "bf16": 2e-2}

CASES = {
    "tiny": WORKLOADS["tiny"],
    "ragged_f32": custom(L=77, d=256, Nr=48, Nc=40, kprime=12, K=10, B=7, dtype="f32",
                         index=301),
    "ragged_bf16": custom(L=131, d=512, Nr=200, Nc=72, kprime=64, K=64, B=300, dtype="bf16",
                          index=302),
    "zipf_bf16": custom(L=300, d=256, Nr=64, Nc=64, kprime=16, K=16, B=8, dtype="bf16",
                        zipf_s=1.1, index=303),
    "k1": custom(L=40, d=128, Nr=16, Nc=16, kprime=1, K=1, B=1, dtype="bf16", index=304),
    "small": WORKLOADS["small"],
}


def _run(wl, seed):
    inp = make_inputs(wl)
    t = {k: dev(v) for k, v in inp.items()}
    out = B.forward(t["x"], t["wr"], t["wc"], t["w"], t["v"], wl.kprime, wl.K, wl.B,
                    t["row_bias"], t["col_bias"])
    dy = np.random.default_rng(seed).standard_normal((wl.L, wl.d)).astype(np.float32)
    g = B.routed_backward(t["x"], t["wr"], t["wc"], t["w"], t["v"], out["expert_idx"],
                          out["gate"], dev(dy))
    torch.cuda.synchronize()
    return inp, out, dy, g


@pytest.mark.parametrize("name", list(CASES))
def test_backward_parity(name):
    wl = CASES[name]
    log(f"[backward] {name}: L={wl.L} d={wl.d} grid={wl.Nr}x{wl.Nc} K={wl.K} {wl.dtype}")
    inp, out, dy, g = _run(wl, seed=wl.index)
    idx = host(out["expert_idx"])
    gate = host(out["gate"])
    ref = OB.backward(inp["x"], inp["wr"], inp["wc"], inp["w"], inp["v"], idx, gate, dy,
                      inp["row_bias"], inp["col_bias"])
    n = int(host(g["counts"])[0])
    assert n == len(ref["active"])
    np.testing.assert_array_equal(host(g["active"])[:n], ref["active"])
    tol = TOL[wl.dtype]
    errs = {}
    for key, got in (("dx", g["dx"]), ("dwr", g["dwr"]), ("dwc", g["dwc"]), ("drb", g["drb"]),
                     ("dcb", g["dcb"]), ("dgate", g["dgate"])):
        errs[key] = rel_err(host(got), ref[key])
    errs["dw"] = rel_err(host(g["dw"])[:n], ref["dw"])
    errs["dv"] = rel_err(host(g["dv"])[:n], ref["dv"])
    log("  " + " ".join(f"{k} {v:.1e}" for k, v in errs.items()) + f" (tol {tol})")
    for k, v in errs.items():
        assert v <= tol, (k, v)


def test_backward_is_deterministic():
    wl = CASES["zipf_bf16"]
    _, _, _, g1 = _run(wl, seed=1)
    n = int(host(g1["counts"])[0])
    # rows of active / dw / dv from n_active on are unspecified (left untouched)
    cut = lambda k, a: a[:n] if k in ("active", "dw", "dv") else a
    r1 = {k: cut(k, host(v)).copy() for k, v in g1.items() if k != "workspace"}
    _, _, _, g2 = _run(wl, seed=1)
    for k, v in r1.items():
        np.testing.assert_array_equal(v.view(np.uint8), cut(k, host(g2[k])).view(np.uint8))


def test_backward_of_an_empty_batch():
    # No tokens: the router gradients are sums over no tokens (zero), no
    # expert is active; outputs prefilled with NaN / -1 must be overwritten.
    wl = custom(L=40, d=128, Nr=16, Nc=16, kprime=4, K=4, B=1, dtype="bf16", index=305)
    t = {k: dev(v) for k, v in make_inputs(wl).items()}
    K, d = wl.K, wl.d
    empty = lambda shape, dtype: torch.empty(shape, dtype=dtype, device="cuda")
    nan = lambda shape: torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    out = {"dwr": nan((wl.Nr, d)), "dwc": nan((wl.Nc, d)), "drb": nan((wl.Nr,)),
           "dcb": nan((wl.Nc,)),
           "counts": torch.full((2,), -1, dtype=torch.int32, device="cuda")}
    g = B.routed_backward(t["x"][:0], t["wr"], t["wc"], t["w"], t["v"],
                          empty((0, K), torch.int32), empty((0, K), torch.float32),
                          empty((0, d), torch.float32), out=out)
    torch.cuda.synchronize()
    assert host(g["counts"]).tolist() == [0, 0]
    for k in ("dwr", "dwc", "drb", "dcb"):
        np.testing.assert_array_equal(host(g[k]), 0.0)
