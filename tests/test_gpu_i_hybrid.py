"""The hybrid executor form through the C ABI: the experts with many tasks
as two dense MFMA products over all tokens, every other task per token.

* within the float tolerance of the oracle on sampled tokens, with and
  without accumulation onto a seeded y0;
* deterministic run to run, and the same bits whether the token lists come
  from the flattened selection or from the inverted schedule;
* bit-identical to the token-centric form when no expert reaches the
  threshold (the hot products then write nothing);
* shapes that take each token-centric kernel for the cold tasks, more than
  64 tasks per token, d = 64 (a half-empty column tile) and a hot set at
  its 2048-expert cap.
"""
import numpy as np
import pytest
import torch

from oracle import omni_oracle as O
from synth import custom, make_inputs, normal
from tests.gpu_helpers import dev, host, log, rel_err
from tests.test_gpu_a_parity import TOL_Y, _zipf_ids, run_pipeline, check_y

pytestmark = pytest.mark.gpu

B = pytest.importorskip("cartesian_routed_atomic_amd.binding")


def threshold(cnt, L):
    """Tasks an expert needs to be hot, as the header states it: ceil(L / 128)
    (at least 2), doubled until no more than 2048 experts reach it."""
    thr = max(2, -(-L // 128))
    while (cnt >= thr).sum() > 2048:
        thr *= 2
    return thr


def _hotset_ids(L, K, N, seed):
    """K distinct ids per token; half the tokens draw from 64 hot experts."""
    rng = np.random.default_rng(seed)
    hot = rng.choice(N, size=64, replace=False)
    idx = np.empty((L, K), np.int32)
    for t in range(L):
        pool = hot if (rng.random() < 0.5 and K <= 64) else N
        idx[t] = rng.choice(pool, size=K, replace=False)
    return idx


def _uniform_ids(L, K, N, seed):
    rng = np.random.default_rng(seed)
    return np.stack([rng.choice(N, size=K, replace=False) for _ in range(L)]).astype(np.int32)


def _cap_ids(L, K, N, seed):
    """Every expert exactly L K / N times (a full hot set when that is the
    threshold)."""
    del seed
    return ((np.arange(L)[:, None] * K + np.arange(K)[None, :]) % N).astype(np.int32)


IDS = {"zipf": lambda L, K, N, s: _zipf_ids(L, K, N, 1.1, s), "hotset": _hotset_ids,
       "uniform": _uniform_ids, "cap": _cap_ids}

# (L, d, N, K, kind)
SHAPES = [
    (2000, 512, 20000, 32, "zipf"),
    (1000, 2048, 5000, 17, "hotset"),
    (8205, 256, 30000, 8, "zipf"),       # cold tasks: four tokens per wave, ragged
    (300, 64, 3000, 70, "zipf"),         # several waves per token, K > 64, d = 64
    (4096, 1024, 2048, 64, "uniform"),   # every expert reaches ceil(L / 128)
    (2048, 512, 4000, 64, "zipf"),
    (2048, 256, 2048, 64, "cap"),        # all 2048 experts hot: the cap
    (3000, 256, 3000, 64, "cap"),        # 3000 reach the threshold: it doubles
    (513, 128, 1 << 20, 64, "uniform"),  # nothing hot
    (500, 128, 1000, 1, "zipf"),         # one task per token
    (5, 128, 50, 8, "zipf"),             # 5 tokens: a 256-row tile of clamped rows
]


@pytest.mark.parametrize("L,d,N,K,kind", SHAPES)
def test_hybrid_form(L, d, N, K, kind):
    seed = L * 3 + d + K
    idx = IDS[kind](L, K, N, seed)
    cnt = np.bincount(idx.ravel(), minlength=N)
    thr = threshold(cnt, L)
    n_hot = int((cnt >= thr).sum())
    cover = cnt[cnt >= thr].sum() / idx.size
    log(f"[hybrid] L={L} d={d} N={N} K={K} {kind}: {n_hot} hot experts "
        f"(threshold {thr}) take {cover:.1%} of the tasks")
    gate = np.random.default_rng(seed + 1).random((L, K)).astype(np.float32)
    gate /= gate.sum(axis=1, keepdims=True)
    x = normal((L, d), seed + 2, 1.0, "bf16")
    w = normal((N, d), seed + 3, float(d) ** -0.5, "bf16")
    v = normal((N, d), seed + 4, float(d) ** -0.5, "bf16")
    tx, tw, tv = dev(x), dev(w), dev(v)
    sched = B.schedule_tasks(dev(idx), dev(gate), N, 16)
    yh = B.atomic_forward(tx, tw, tv, sched, mode="hybrid")
    yh2 = B.atomic_forward(tx, tw, tv, sched, mode="hybrid")
    yt = B.atomic_forward(tx, tw, tv, sched, mode="token")
    flat = (sched.flat_expert, sched.flat_gate)
    sched.flat_expert = sched.flat_gate = None
    yh3 = B.atomic_forward(tx, tw, tv, sched, mode="hybrid")
    sched.flat_expert, sched.flat_gate = flat
    torch.cuda.synchronize()
    assert torch.equal(yh.view(torch.int32), yh2.view(torch.int32)), "not deterministic"
    assert torch.equal(yh.view(torch.int32), yh3.view(torch.int32)), "inverted lists differ"
    if n_hot == 0:
        assert torch.equal(yh.view(torch.int32), yt.view(torch.int32))
        log("  nothing hot: bit-identical to the token-centric form")
    toks = np.sort(np.random.default_rng(seed + 5).choice(L, size=min(L, 256), replace=False))
    want = O.atomic_forward(x, w, v, idx, gate, tokens=toks)
    e = rel_err(host(yh)[toks], want)
    et = rel_err(host(yh), host(yt))
    log(f"  max|d|/max|y|: {e:.2e} against the oracle, {et:.2e} against the token form "
        f"(tol {TOL_Y['bf16']})")
    assert e <= TOL_Y["bf16"]
    y0 = np.random.default_rng(seed + 6).standard_normal((L, d)).astype(np.float32)
    ya = B.atomic_forward(tx, tw, tv, sched, y=dev(y0), accumulate=True, mode="hybrid")
    torch.cuda.synchronize()
    ea = rel_err(host(ya)[toks], want + y0[toks])
    log(f"  accumulate onto y0: {ea:.2e}")
    assert ea <= TOL_Y["bf16"]


def test_hybrid_full_pipeline_zipf():
    """Router, top-K, schedule and the hybrid executor on a Zipf-routed
    workload (row and column logits biased as in the skewed workload)."""
    wl = custom(L=4096, d=1024, Nr=128, Nc=128, kprime=32, K=32, B=64, dtype="bf16",
                zipf_s=1.1, index=220)
    inp = make_inputs(wl)
    out = run_pipeline(wl, inp)
    t = {k: dev(inp[k]) for k in ("x", "w", "v")}
    yh = B.atomic_forward(t["x"], t["w"], t["v"], out["schedule"], mode="hybrid")
    torch.cuda.synchronize()
    idx = host(out["expert_idx"])
    cnt = np.bincount(idx.ravel(), minlength=wl.N)
    thr = threshold(cnt, wl.L)
    log(f"[hybrid pipeline] {int((cnt >= thr).sum())} hot experts take "
        f"{cnt[cnt >= thr].sum() / idx.size:.1%} of the tasks")
    toks = np.sort(np.random.default_rng(1).choice(wl.L, size=256, replace=False))
    check_y(inp, out, yh, "bf16", tokens=toks)


def test_hybrid_rejects_float32():
    x = torch.zeros((4, 128), device="cuda")
    w = torch.zeros((64, 128), device="cuda")
    idx = torch.zeros((4, 2), dtype=torch.int32, device="cuda")
    idx[:, 1] = 1
    gate = torch.full((4, 2), 0.5, device="cuda")
    sched = B.schedule_tasks(idx, gate, 64, 4)
    with pytest.raises(B.OmniError) as err:
        B.atomic_forward(x, w, w, sched, mode="hybrid")
    assert err.value.code == B.OMNI_ERR_UNSUPPORTED
