"""GPU parity of the shared dense MLP (omni_shared_mlp) and of the whole
OmniMoE layer (shared MLP + routed branch) against the float64 oracle.

Bars as for the routed output: max|d| / max|ref| <= 1e-4 (float32 workloads)
or 2e-2 (bf16)."""
import numpy as np
import pytest
import torch

from oracle import omni_layer as OL
from oracle import omni_oracle as O
from synth import WORKLOADS, custom, make_inputs
from tests.gpu_helpers import dev, host, log, rel_err

pytestmark = pytest.mark.gpu

B = pytest.importorskip("cartesian_routed_atomic_amd.binding")

TOL = {"f32": 1e-4, "bf16": 2e-2}
MLP = ("x", "wg", "wu", "wd")

CASES = {
    "tiny": WORKLOADS["tiny"],
    # d not a multiple of 32 (the 128 x 128 kernel), d_ff not a multiple of 16
    # (the interleaved gate / up blocks end inside a block), ragged L
    "ragged_bf16": custom(L=131, d=264, Nr=16, Nc=16, kprime=8, K=8, B=8, dtype="bf16",
                          index=401, dff=200),
    "ragged_f32": custom(L=77, d=132, Nr=8, Nc=8, kprime=4, K=4, B=4, dtype="f32",
                         index=402, dff=100),
    # the 256 x 256 kernel: d a multiple of 32 and enough tiles
    "small": WORKLOADS["small"],
    "one_token": custom(L=1, d=256, Nr=8, Nc=8, kprime=4, K=4, B=4, dtype="bf16", index=403,
                        dff=64),
    # few tokens: the down product is split over d_ff (8 chunks)
    "decode_shape": custom(L=256, d=2048, Nr=16, Nc=16, kprime=4, K=4, B=4, dtype="bf16",
                           index=405, dff=5632),
}
# the routed branch needs d = 64 * 2^p: a ragged layer case of its own
LAYER_CASES = {
    "tiny": WORKLOADS["tiny"],
    "ragged_bf16": custom(L=131, d=256, Nr=16, Nc=12, kprime=8, K=8, B=8, dtype="bf16",
                          index=404, dff=200),
    "small": WORKLOADS["small"],
}


@pytest.mark.parametrize("name", list(CASES))
def test_shared_mlp_parity(name):
    wl = CASES[name]
    log(f"[shared mlp] {name}: L={wl.L} d={wl.d} d_ff={wl.d_ff} {wl.dtype}")
    inp = make_inputs(wl, parts=MLP)
    t = {k: dev(inp[k]) for k in MLP}
    y = B.shared_mlp(t["x"], t["wg"], t["wu"], t["wd"])
    # accumulate onto a seeded y
    y0 = np.random.default_rng(wl.index).standard_normal((wl.L, wl.d)).astype(np.float32)
    y2 = B.shared_mlp(t["x"], t["wg"], t["wu"], t["wd"], y=dev(y0), accumulate=True)
    torch.cuda.synchronize()
    toks = np.arange(wl.L) if wl.L <= 512 else np.sort(
        np.random.default_rng(0).choice(wl.L, 512, replace=False))
    ref = OL.shared_mlp_f64(inp["x"][toks], inp["wg"], inp["wu"], inp["wd"])
    e1 = rel_err(host(y)[toks], ref)
    e2 = rel_err(host(y2)[toks], ref + y0[toks])
    log(f"  y {e1:.1e}, accumulated {e2:.1e} (tol {TOL[wl.dtype]}) on {len(toks)} tokens")
    assert e1 <= TOL[wl.dtype] and e2 <= TOL[wl.dtype]


def test_shared_mlp_full_size_sampled():
    wl = WORKLOADS["large"]
    log(f"[shared mlp] large: L={wl.L} d={wl.d} d_ff={wl.d_ff}")
    inp = make_inputs(wl, parts=MLP)
    t = {k: dev(inp[k]) for k in MLP}
    y = B.shared_mlp(t["x"], t["wg"], t["wu"], t["wd"])
    torch.cuda.synchronize()
    toks = np.sort(np.random.default_rng(1).choice(wl.L, 256, replace=False))
    ref = OL.shared_mlp_f64(inp["x"][toks], inp["wg"], inp["wu"], inp["wd"])
    e = rel_err(host(y)[toks], ref)
    log(f"  y {e:.1e} on {len(toks)} tokens")
    assert e <= TOL[wl.dtype]


def test_shared_mlp_is_deterministic_and_empty_batch_is_a_no_op():
    wl = CASES["ragged_bf16"]
    inp = make_inputs(wl, parts=MLP)
    t = {k: dev(inp[k]) for k in MLP}
    a = B.shared_mlp(t["x"], t["wg"], t["wu"], t["wd"])
    b = B.shared_mlp(t["x"], t["wg"], t["wu"], t["wd"])
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    y = B.shared_mlp(t["x"][:0], t["wg"], t["wu"], t["wd"])
    torch.cuda.synchronize()
    assert y.shape == (0, wl.d)


@pytest.mark.parametrize("name", list(LAYER_CASES))
def test_layer_forward_parity(name):
    wl = LAYER_CASES[name]
    log(f"[layer] {name}: L={wl.L} d={wl.d} d_ff={wl.d_ff} grid={wl.Nr}x{wl.Nc} K={wl.K}")
    inp = make_inputs(wl, parts=("x", "wr", "wc", "w", "v") + MLP[1:])
    t = {k: dev(v) for k, v in inp.items()}
    out = B.layer_forward(t["x"], t["wr"], t["wc"], t["w"], t["v"], t["wg"], t["wu"], t["wd"],
                          wl.kprime, wl.K, wl.B, t["row_bias"], t["col_bias"])
    torch.cuda.synchronize()
    # the routed branch on the GPU's own selection (its parity is tested on
    # its own); the layer output must be the sum of the two branches
    idx, gate = host(out["expert_idx"]), host(out["gate"])
    toks = np.arange(wl.L) if wl.L <= 512 else np.sort(
        np.random.default_rng(2).choice(wl.L, 256, replace=False))
    ref = (OL.shared_mlp_f64(inp["x"][toks], inp["wg"], inp["wu"], inp["wd"])
           + O.atomic_forward_f64(inp["x"], inp["w"], inp["v"], idx, gate, tokens=toks))
    e = rel_err(host(out["y"])[toks], ref)
    log(f"  layer y {e:.1e} (tol {TOL[wl.dtype]}) on {len(toks)} tokens")
    assert e <= TOL[wl.dtype]
