"""GPU parity of the variants against their float64 oracles: the
SwiGLU-gated atomic expert (omni_atomic_forward_glu).  Bars as for the
routed output: max|d| / max|ref| <= 1e-4 (float32) or 2e-2 (bf16)."""
import numpy as np
import pytest
import torch

from oracle import omni_variants as OV
from synth import WORKLOADS, custom, make_inputs
from tests.gpu_helpers import dev, host, log, rel_err

pytestmark = pytest.mark.gpu

B = pytest.importorskip("cartesian_routed_atomic_amd.binding")

TOL = {"f32": 1e-4, "bf16": 2e-2}
PARTS = ("x", "wr", "wc", "w", "v", "u")

GLU_CASES = {
    "tiny": WORKLOADS["tiny"],
    "ragged_bf16": custom(L=77, d=256, Nr=48, Nc=40, kprime=12, K=10, B=7, dtype="bf16",
                          index=501),
    "ragged_f32": custom(L=33, d=512, Nr=20, Nc=30, kprime=9, K=9, B=5, dtype="f32", index=502),
    "k1": custom(L=40, d=128, Nr=16, Nc=16, kprime=1, K=1, B=1, dtype="bf16", index=503),
    "small": WORKLOADS["small"],
    "large": WORKLOADS["large"],
}


@pytest.mark.parametrize("name", list(GLU_CASES))
def test_glu_expert_parity(name):
    wl = GLU_CASES[name]
    log(f"[glu] {name}: L={wl.L} d={wl.d} N={wl.N} K={wl.K} {wl.dtype}")
    inp = make_inputs(wl, parts=PARTS)
    t = {k: dev(v) for k, v in inp.items()}
    out = B.forward(t["x"], t["wr"], t["wc"], t["w"], t["v"], wl.kprime, wl.K, wl.B,
                    t["row_bias"], t["col_bias"])
    y = B.atomic_forward_glu(t["x"], t["w"], t["u"], t["v"], out["schedule"])
    y0 = np.random.default_rng(wl.index).standard_normal((wl.L, wl.d)).astype(np.float32)
    y2 = B.atomic_forward_glu(t["x"], t["w"], t["u"], t["v"], out["schedule"], y=dev(y0),
                              accumulate=True)
    torch.cuda.synchronize()
    idx, gate = host(out["expert_idx"]), host(out["gate"])
    toks = np.arange(wl.L) if wl.L <= 512 else np.sort(
        np.random.default_rng(3).choice(wl.L, 128, replace=False))
    ref = OV.atomic_forward_glu_f64(inp["x"], inp["w"], inp["u"], inp["v"], idx, gate,
                                    tokens=toks)
    e1 = rel_err(host(y)[toks], ref)
    e2 = rel_err(host(y2)[toks], ref + y0[toks])
    log(f"  y {e1:.1e}, accumulated {e2:.1e} (tol {TOL[wl.dtype]}) on {len(toks)} tokens")
    assert e1 <= TOL[wl.dtype] and e2 <= TOL[wl.dtype]


def test_glu_expert_is_deterministic_and_rejects_unsupported_rows():
    wl = GLU_CASES["ragged_bf16"]
    inp = make_inputs(wl, parts=PARTS)
    t = {k: dev(v) for k, v in inp.items()}
    out = B.forward(t["x"], t["wr"], t["wc"], t["w"], t["v"], wl.kprime, wl.K, wl.B)
    a = B.atomic_forward_glu(t["x"], t["w"], t["u"], t["v"], out["schedule"])
    b = B.atomic_forward_glu(t["x"], t["w"], t["u"], t["v"], out["schedule"])
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    # rows over 4 KiB are refused before anything is launched
    x4 = torch.zeros((2, 4096), dtype=torch.bfloat16, device="cuda")
    w4 = torch.zeros((8, 4096), dtype=torch.bfloat16, device="cuda")
    s4 = B.schedule_tasks(torch.zeros((2, 1), dtype=torch.int32, device="cuda"),
                          torch.ones((2, 1), dtype=torch.float32, device="cuda"), 8, 1)
    with pytest.raises(B.OmniError):
        B.atomic_forward_glu(x4, w4, w4, w4, s4)
