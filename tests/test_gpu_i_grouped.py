"""The grouped executor form through the C ABI: per tile of 64 tokens, the
experts the schedule counts most tasks for (the hot set) as two bf16 MFMA
products, every other task per task, y written once.

* within the bf16 tolerance of the oracle on every token, with and without
  accumulation onto a seeded y0;
* deterministic run to run, and the same bits whether the token lists come
  from the flattened selection or from the inverted schedule;
* bit-identical to the token-centric form when no expert reaches the
  threshold (every task then takes the token-centric arithmetic);
* skewed, hot-set, capped and uniform routings; ragged last tiles; d from 64
  to 2048; one task per token; the whole pipeline on a Zipf-routed workload.
The hot-set rule itself is checked exactly on the CPU model of the kernels
(tests/test_host_sim_grouped.py).
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


def hot_set(idx, L, N):
    """The hot set the header states: experts with at least tau tasks, tau =
    max(2, ceil(L / 64)) doubled until at most 512 experts reach it."""
    cnt = np.bincount(idx.ravel(), minlength=N)
    tau = max(2, -(-L // 64))
    while (cnt >= tau).sum() > 512:
        tau *= 2
    return cnt >= tau, cnt


def _hotset_ids(L, K, N, seed):
    """K distinct ids per token; half the tokens draw from 64 hot experts."""
    rng = np.random.default_rng(seed)
    hot = rng.choice(N, size=64, replace=False)
    idx = np.empty((L, K), np.int32)
    for t in range(L):
        pool = hot if rng.random() < 0.5 else N
        idx[t] = rng.choice(pool, size=K, replace=False)
    return idx


def _uniform_ids(L, K, N, seed):
    rng = np.random.default_rng(seed)
    return np.stack([rng.choice(N, size=K, replace=False) for _ in range(L)]).astype(np.int32)


def _cap_ids(L, K, N, seed):
    """Every expert exactly L K / N times."""
    del seed
    return ((np.arange(L)[:, None] * K + np.arange(K)[None, :]) % N).astype(np.int32)


IDS = {"zipf": lambda L, K, N, s: _zipf_ids(L, K, N, 1.1, s), "hotset": _hotset_ids,
       "uniform": _uniform_ids, "cap": _cap_ids}

# (L, d, N, K, kind)
SHAPES = [
    (2000, 512, 20000, 32, "zipf"),
    (1000, 2048, 5000, 17, "hotset"),
    (8205, 256, 30000, 8, "zipf"),       # ragged last tile (8205 = 128 * 64 + 13)
    (300, 64, 3000, 64, "zipf"),         # d = 64: one output block, for wave 0
    (4096, 1024, 2048, 64, "uniform"),   # every expert has ~128 tasks: the cap doubles tau
    (2048, 256, 2048, 64, "cap"),        # all 2048 experts reach tau: doubles until none
    (3000, 256, 6000, 64, "cap"),        # 32 tasks each: 6000 reach tau, then none
    (513, 128, 1 << 20, 64, "uniform"),  # nothing hot
    (500, 128, 1000, 1, "zipf"),         # one task per token
    (5, 128, 50, 8, "zipf"),             # 5 tokens: one tile of mostly missing rows
]


@pytest.mark.parametrize("L,d,N,K,kind", SHAPES)
def test_grouped_form(L, d, N, K, kind):
    seed = L * 3 + d + K
    idx = IDS[kind](L, K, N, seed)
    hot, cnt = hot_set(idx, L, N)
    n_hot = int(hot.sum())
    cover = cnt[hot].sum() / idx.size
    log(f"[grouped] L={L} d={d} N={N} K={K} {kind}: {n_hot} hot experts take {cover:.1%} "
        f"of the tasks")
    gate = np.random.default_rng(seed + 1).random((L, K)).astype(np.float32)
    gate /= gate.sum(axis=1, keepdims=True)
    x = normal((L, d), seed + 2, 1.0, "bf16")
    w = normal((N, d), seed + 3, float(d) ** -0.5, "bf16")
    v = normal((N, d), seed + 4, float(d) ** -0.5, "bf16")
    tx, tw, tv = dev(x), dev(w), dev(v)
    sched = B.schedule_tasks(dev(idx), dev(gate), N, 16)
    yg = B.atomic_forward(tx, tw, tv, sched, mode="grouped")
    yg2 = B.atomic_forward(tx, tw, tv, sched, mode="grouped")
    yt = B.atomic_forward(tx, tw, tv, sched, mode="token") if d <= 2048 else None
    flat = (sched.flat_expert, sched.flat_gate)
    sched.flat_expert = sched.flat_gate = None
    yg3 = B.atomic_forward(tx, tw, tv, sched, mode="grouped")
    sched.flat_expert, sched.flat_gate = flat
    torch.cuda.synchronize()
    assert torch.equal(yg.view(torch.int32), yg2.view(torch.int32)), "not deterministic"
    assert torch.equal(yg.view(torch.int32), yg3.view(torch.int32)), "inverted lists differ"
    if n_hot == 0:
        assert torch.equal(yg.view(torch.int32), yt.view(torch.int32))
        log("  nothing hot: bit-identical to the token-centric form")
    want = O.atomic_forward(x, w, v, idx, gate)
    e = rel_err(host(yg), want)
    et = rel_err(host(yg), host(yt))
    log(f"  max|d|/max|y| of all tokens: {e:.2e} against the oracle, {et:.2e} against the "
        f"token form (tol {TOL_Y['bf16']})")
    assert e <= TOL_Y["bf16"]
    y0 = np.random.default_rng(seed + 6).standard_normal((L, d)).astype(np.float32)
    ya = B.atomic_forward(tx, tw, tv, sched, y=dev(y0), accumulate=True, mode="grouped")
    torch.cuda.synchronize()
    ea = rel_err(host(ya), want + y0)
    log(f"  accumulate onto y0: {ea:.2e}")
    assert ea <= TOL_Y["bf16"]


def test_grouped_full_pipeline_zipf():
    """Router, top-K, schedule and the grouped executor on a Zipf-routed
    workload (row and column logits biased as in the skewed workload)."""
    wl = custom(L=4096, d=1024, Nr=128, Nc=128, kprime=32, K=32, B=64, dtype="bf16",
                zipf_s=1.1, index=220)
    inp = make_inputs(wl)
    out = run_pipeline(wl, inp)
    t = {k: dev(inp[k]) for k in ("x", "w", "v")}
    yg = B.atomic_forward(t["x"], t["w"], t["v"], out["schedule"], mode="grouped")
    torch.cuda.synchronize()
    idx = host(out["expert_idx"])
    hot, cnt = hot_set(idx, wl.L, wl.N)
    log(f"[grouped pipeline] {int(hot.sum())} hot experts take "
        f"{cnt[hot].sum() / idx.size:.1%} of the tasks")
    check_y(inp, out, yg, "bf16")


@pytest.mark.parametrize("dtype,d,K", [(torch.float32, 128, 2), (torch.bfloat16, 128, 65),
                                       (torch.bfloat16, 4096, 2)])
def test_grouped_rejects_what_it_does_not_cover(dtype, d, K):
    # float32, more than 64 tasks per token, rows over 4 KiB
    L, N = 4, 256
    x = torch.zeros((L, d), device="cuda", dtype=dtype)
    w = torch.zeros((N, d), device="cuda", dtype=dtype)
    idx = (torch.arange(L * K, device="cuda", dtype=torch.int32) % N).reshape(L, K)
    gate = torch.full((L, K), 1.0 / K, device="cuda")
    sched = B.schedule_tasks(idx, gate, N, 4)
    with pytest.raises(B.OmniError) as err:
        B.atomic_forward(x, w, w, sched, mode="grouped")
    assert err.value.code == B.OMNI_ERR_UNSUPPORTED
