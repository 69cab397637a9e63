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
    # d = 64 m not a power of two, and rows over 4 KiB (the chunked kernels)
    "d768": custom(L=300, d=768, Nr=40, Nc=50, kprime=10, K=16, B=8, dtype="bf16", index=504),
    "d4096": custom(L=70, d=4096, Nr=32, Nc=32, kprime=8, K=12, B=8, dtype="bf16", index=505),
    "f32_d1536": custom(L=40, d=1536, Nr=16, Nc=24, kprime=6, K=9, B=4, dtype="f32",
                        index=506),
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
    # token lists inverted from the sorted schedule instead of read from the
    # flattened selection: the same bits
    s = out["schedule"]
    flat = (s.flat_expert, s.flat_gate)
    s.flat_expert = s.flat_gate = None
    y3 = B.atomic_forward_glu(t["x"], t["w"], t["u"], t["v"], s)
    s.flat_expert, s.flat_gate = flat
    torch.cuda.synchronize()
    assert torch.equal(y3.view(torch.int32), y.view(torch.int32))
    idx, gate = host(out["expert_idx"]), host(out["gate"])
    toks = np.arange(wl.L) if wl.L <= 512 else np.sort(
        np.random.default_rng(3).choice(wl.L, 128, replace=False))
    ref = OV.atomic_forward_glu_f64(inp["x"], inp["w"], inp["u"], inp["v"], idx, gate,
                                    tokens=toks)
    e1 = rel_err(host(y)[toks], ref)
    e2 = rel_err(host(y2)[toks], ref + y0[toks])
    log(f"  y {e1:.1e}, accumulated {e2:.1e} (tol {TOL[wl.dtype]}) on {len(toks)} tokens")
    assert e1 <= TOL[wl.dtype] and e2 <= TOL[wl.dtype]


def test_glu_expert_is_deterministic_and_rejects_unsupported_widths():
    wl = GLU_CASES["ragged_bf16"]
    inp = make_inputs(wl, parts=PARTS)
    t = {k: dev(v) for k, v in inp.items()}
    out = B.forward(t["x"], t["wr"], t["wc"], t["w"], t["v"], wl.kprime, wl.K, wl.B)
    a = B.atomic_forward_glu(t["x"], t["w"], t["u"], t["v"], out["schedule"])
    b = B.atomic_forward_glu(t["x"], t["w"], t["u"], t["v"], out["schedule"])
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    # a width that is not a multiple of 64 is refused before anything is launched
    x4 = torch.zeros((2, 72), dtype=torch.bfloat16, device="cuda")
    w4 = torch.zeros((8, 72), dtype=torch.bfloat16, device="cuda")
    s4 = B.schedule_tasks(torch.zeros((2, 1), dtype=torch.int32, device="cuda"),
                          torch.ones((2, 1), dtype=torch.float32, device="cuda"), 8, 1)
    with pytest.raises(B.OmniError):
        B.atomic_forward_glu(x4, w4, w4, w4, s4)


# ------------------------------------------------------------ flat router

from synth import normal  # noqa: E402

FLAT_CASES = {
    # name: (L, d, N, K, dtype, kind)
    "tiny_f32": (64, 128, 1024, 8, "f32", "gauss"),
    "ragged_bf16": (77, 264, 1920, 10, "bf16", "gauss"),
    "dup_rows": (40, 256, 3000, 16, "bf16", "dup"),        # exact ties: ids e, e+1, e+2 equal
    "all_equal": (8, 128, 5000, 64, "bf16", "zero"),       # more than 2048 tied: the fallback
    "quantised_bias": (16, 128, 8192, 33, "f32", "qbias"),  # few distinct values: the fallback
    "million": (32, 2048, 1 << 20, 64, "bf16", "gauss"),   # the large workload's N
}


def _flat_inputs(L, d, N, dtype, kind, seed):
    x = normal((L, d), 1000 * seed, 1.0, dtype)
    if kind == "zero" or kind == "qbias":
        wf = np.zeros((N, d), np.uint16 if dtype == "bf16" else np.float32)
    elif kind == "dup":
        base = normal((N // 3 + 1, d), 1000 * seed + 1, 1 / np.sqrt(d), dtype)
        wf = np.ascontiguousarray(np.repeat(base, 3, axis=0)[:N])
    else:
        wf = normal((N, d), 1000 * seed + 1, 1 / np.sqrt(d), dtype)
    bias = None
    if kind == "qbias":
        bias = (np.round(np.random.default_rng(seed).standard_normal(N)) * 0.5).astype(np.float32)
    return x, wf, bias


@pytest.mark.parametrize("name", list(FLAT_CASES))
def test_flat_router_parity(name):
    L, d, N, K, dtype, kind = FLAT_CASES[name]
    log(f"[flat router] {name}: L={L} d={d} N={N} K={K} {dtype} {kind}")
    x, wf, bias = _flat_inputs(L, d, N, dtype, kind, seed=600 + len(name))
    r = B.flat_router_topk(dev(x), dev(wf), K, bias=dev(bias), want_logp=True)
    torch.cuda.synchronize()
    logp = host(r["logp"])
    # selection: bit-exact for the GPU's own log-probabilities
    idx, score, gate = OV.flat_topk(logp, K)
    np.testing.assert_array_equal(host(r["expert_idx"]), idx)
    np.testing.assert_array_equal(host(r["score"]).view(np.uint32), score.view(np.uint32))
    dg = float(np.abs(host(r["gate"]) - gate).max())
    assert dg <= 2e-6, dg
    # log-probabilities against the float64 oracle (a sample of tokens at large N)
    toks = np.arange(L) if L * N <= 1 << 22 else np.arange(4)
    want = OV.flat_router_logp(x[toks], wf, bias)
    dl = float(np.abs(logp[toks] - want).max())
    log(f"  selection bit-exact; gates max|d| {dg:.1e}; log p max|d| {dl:.1e}")
    assert dl <= 1e-4  # the router bar; measured <= 3.8e-6 (N = 2^20)
