"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (binding.forward on one stream).  The oracle checks the whole
router output, the top-K of every token (fed the GPU's own log-probabilities),
the whole schedule, and y of every token for the form auto picks and for the
grouped form."""
import time

import pytest
import torch

from oracle import omni_oracle as O
from synth import WORKLOADS, make_inputs
from tests.gpu_helpers import dev, host, log, rel_err
from tests.test_gpu_a_parity import TOL_Y, check_router, check_schedule, check_topk

pytestmark = pytest.mark.gpu

B = pytest.importorskip("cartesian_routed_atomic_amd.binding")


@pytest.mark.parametrize("name", ["mid", "large", "decode"])
def test_full_size_parity(name):
    wl = WORKLOADS[name]
    log(f"[full] {name}: L={wl.L} d={wl.d} N={wl.N} K={wl.K} B={wl.B}")
    t0 = time.time()
    inp = make_inputs(wl)
    log(f"  inputs generated in {time.time() - t0:.1f}s")
    t = {k: dev(v) for k, v in inp.items()}
    out = B.forward(t["x"], t["wr"], t["wc"], t["w"], t["v"], wl.kprime, wl.K, wl.B,
                    t["row_bias"], t["col_bias"])
    torch.cuda.synchronize()
    # the form auto did not pick, on the same schedule: must give the same bits
    auto = B.atomic_forward_mode(t["x"].dtype, wl.L, wl.d, wl.N, wl.K, wl.B)
    other = "expert" if auto == "token" else "token"
    y2 = B.atomic_forward(t["x"], t["w"], t["v"], out["schedule"], mode=other)
    torch.cuda.synchronize()
    assert torch.equal(y2.view(torch.int32), out["y"].view(torch.int32))
    log(f"  y of the {auto}-centric (auto) and {other}-centric forms bit-identical")
    # the token-centric form with its lists inverted from the sorted schedule
    # instead of read from the flattened selection: the same bits
    s = out["schedule"]
    flat = (s.flat_expert, s.flat_gate)
    s.flat_expert = s.flat_gate = None
    y3 = B.atomic_forward(t["x"], t["w"], t["v"], s, mode="token")
    s.flat_expert, s.flat_gate = flat
    torch.cuda.synchronize()
    assert torch.equal(y3.view(torch.int32), out["y"].view(torch.int32))
    log("  token lists from the selection and from the schedule give bit-identical y")
    # the grouped form (hot experts of each token tile on MFMA) on the same schedule
    yh = B.atomic_forward(t["x"], t["w"], t["v"], out["schedule"], mode="grouped")
    yh2 = B.atomic_forward(t["x"], t["w"], t["v"], out["schedule"], mode="grouped")
    torch.cuda.synchronize()
    assert torch.equal(yh.view(torch.int32), yh2.view(torch.int32))
    log("  grouped form: two calls bit-identical")
    del t, y2, y3, yh2
    log(f"  gpu done {time.time() - t0:.1f}s")
    check_router(inp, out)
    check_topk(out["row_logp"], out["col_logp"], out, wl.kprime, wl.K)
    log(f"  top-K of all {wl.L} tokens checked ({time.time() - t0:.1f}s)")
    want = check_schedule(out, out["schedule"], wl.N, wl.B)
    log(f"  expert usage {want['n_active'] / wl.N:.4f}; traffic "
        f"{O.traffic_elements(wl.d, wl.L, wl.K, want['n_active'])}")
    # y of every token, the oracle evaluated once for both forms
    ywant = O.atomic_forward(inp["x"], inp["w"], inp["v"], host(out["expert_idx"]),
                             host(out["gate"]))
    for label, y in (("auto", out["y"]), ("grouped", yh)):
        e = rel_err(host(y), ywant)
        log(f"  y ({label}) of all tokens: max|d|/max|y| {e:.2e} (tol {TOL_Y[wl.dtype]})")
        assert e <= TOL_Y[wl.dtype]
    log(f"  done in {time.time() - t0:.1f}s")
