"""Backward parity at the full workload sizes, in the launch configuration the
benchmark times (binding.routed_backward on the forward's own selection).

The float64 oracle checks:
  - the active expert list in full (bit-exact);
  - dx and dgate on sampled tokens (each token's are its own: the oracle
    runs on that token alone);
  - dW and dV on sampled active experts (the oracle runs on the tokens that
    use the expert);
  - dWr, dWc and the bias gradients in full (they sum over every token: the
    oracle's executor backward runs over all tokens in batches for the gate
    gradients, then its router backward runs once).
Bars as for the small cases: max|d| / max|ref| <= 2e-2 (bf16)."""
import time

import numpy as np
import pytest
import torch

from oracle import omni_backward as OB
from oracle import omni_oracle as O
from synth import WORKLOADS, make_inputs
from tests.gpu_helpers import dev, host, log, rel_err

pytestmark = pytest.mark.gpu

B = pytest.importorskip("cartesian_routed_atomic_amd.binding")

TOL = {"f32": 1e-4, "bf16": 2e-2}


@pytest.mark.parametrize("name", ["large", "mid"])
def test_backward_full_size(name):
    wl = WORKLOADS[name]
    tol = TOL[wl.dtype]
    log(f"[backward full] {name}: L={wl.L} d={wl.d} grid={wl.Nr}x{wl.Nc} K={wl.K}")
    t0 = time.time()
    inp = make_inputs(wl)
    t = {k: dev(v) for k, v in inp.items()}
    out = B.forward(t["x"], t["wr"], t["wc"], t["w"], t["v"], wl.kprime, wl.K, wl.B,
                    t["row_bias"], t["col_bias"])
    dy = np.random.default_rng(wl.index + 77).standard_normal((wl.L, wl.d)).astype(np.float32)
    g = B.routed_backward(t["x"], t["wr"], t["wc"], t["w"], t["v"], out["expert_idx"],
                          out["gate"], dev(dy))
    torch.cuda.synchronize()
    idx = host(out["expert_idx"])
    gate = host(out["gate"])
    got = {k: host(v) for k, v in g.items() if k != "workspace"}
    del t, out, g
    log(f"  gpu done in {time.time() - t0:.1f}s")
    x, wr, wc, w, v = inp["x"], inp["wr"], inp["wc"], inp["w"], inp["v"]
    rb, cb = inp["row_bias"], inp["col_bias"]

    active = np.unique(idx)
    n = int(got["counts"][0])
    assert n == len(active)
    np.testing.assert_array_equal(got["active"][:n], active)

    rng = np.random.default_rng(5)
    # dx, dgate: sampled tokens
    toks = np.sort(rng.choice(wl.L, size=48, replace=False))
    dx_ref = np.zeros((len(toks), wl.d))
    dg_ref = np.zeros((len(toks), wl.K))
    for i, tk in enumerate(toks):
        r = OB.backward(x[tk:tk + 1], wr, wc, w, v, idx[tk:tk + 1], gate[tk:tk + 1],
                        dy[tk:tk + 1], rb, cb)
        dx_ref[i] = r["dx"][0]
        dg_ref[i] = r["dgate"][0]
    e_dx = rel_err(got["dx"][toks], dx_ref)
    e_dg = rel_err(got["dgate"][toks], dg_ref)
    log(f"  dx {e_dx:.1e} dgate {e_dg:.1e} on {len(toks)} tokens")
    assert e_dx <= tol and e_dg <= tol

    # dW, dV: sampled active experts
    pos = np.sort(rng.choice(n, size=48, replace=False))
    dw_ref = np.zeros((len(pos), wl.d))
    dv_ref = np.zeros((len(pos), wl.d))
    for i, p in enumerate(pos):
        e = active[p]
        users = np.nonzero((idx == e).any(axis=1))[0]
        r = OB.executor_backward(x[users], w, v, idx[users], gate[users], dy[users])
        j = int(np.searchsorted(r["active"], e))
        dw_ref[i] = r["dw"][j]
        dv_ref[i] = r["dv"][j]
    e_dw = rel_err(got["dw"][pos], dw_ref)
    e_dv = rel_err(got["dv"][pos], dv_ref)
    log(f"  dW {e_dw:.1e} dV {e_dv:.1e} on {len(pos)} experts")
    assert e_dw <= tol and e_dv <= tol

    # router gradients, in full
    dgate = np.zeros((wl.L, wl.K))
    for s in range(0, wl.L, 512):
        r = OB.executor_backward(x[s:s + 512], w, v, idx[s:s + 512], gate[s:s + 512],
                                 dy[s:s + 512])
        dgate[s:s + 512] = r["dgate"]
    dS = OB.gate_backward(gate, dgate)
    da, db = OB.score_backward(idx, dS, wl.Nr, wl.Nc)
    zr, zc = O.router_logits_f64(x, wr, wc, rb, cb)
    dzr = OB.log_softmax_backward(zr, da)
    dzc = OB.log_softmax_backward(zc, db)
    _, dwr, dwc, drb, dcb = OB.router_backward(x, wr, wc, dzr, dzc)
    errs = {"dwr": rel_err(got["dwr"], dwr), "dwc": rel_err(got["dwc"], dwc),
            "drb": rel_err(got["drb"], drb), "dcb": rel_err(got["dcb"], dcb)}
    log("  " + " ".join(f"{k} {e:.1e}" for k, e in errs.items()) + f" (tol {tol})")
    for k, e in errs.items():
        assert e <= tol, (k, e)
    log(f"  done in {time.time() - t0:.1f}s")
