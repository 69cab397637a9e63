"""Seeded random shapes through the C ABI.

* The schedule, both groupings, bit-exact against the oracle, over shapes that
  fall on both sides of every launch-path choice (one or several radix passes,
  at most 32 sort tiles or more, at most 8 expert tiles or more).
* The executor: the expert-centric and token-centric forms bit-identical to
  each other, and within the float tolerance of the oracle on sampled tokens,
  over row widths 64..2048 and token counts that take each token-centric
  kernel (several waves per token below 4096 tokens, one from 4096, four
  tokens per wave from 8192, with a ragged last wave); and over widths
  d = 64 m that are not powers of two or whose rows are too long for the
  register-resident kernels (the chunked kernels: d = 192 .. 4096).
"""
import numpy as np
import pytest
import torch

from oracle import omni_oracle as O
from synth import normal
from tests.gpu_helpers import dev, host, log, rel_err
from tests.test_gpu_a_parity import TOL_Y, check_schedule

pytestmark = pytest.mark.gpu

B = pytest.importorskip("cartesian_routed_atomic_amd.binding")


def _ids(L, K, N, seed):
    """K distinct ids per token; half the tokens draw from a small hot set so
    that experts repeat across tokens."""
    rng = np.random.default_rng(seed)
    hot = rng.choice(N, size=min(N, max(K, 64)), replace=False)
    idx = np.empty((L, K), np.int32)
    for t in range(L):
        pool = hot if (rng.random() < 0.5 and len(hot) >= K) else N
        idx[t] = rng.choice(pool, size=K, replace=False)
    return idx


def _schedule_shapes(seed, n):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        K = int(rng.integers(1, 65))
        L = int(rng.integers(1, 4000))
        N = int(rng.integers(K, 300000))
        Bg = int(rng.choice([1, 2, 3, 7, 16, 64, 100, 256, 1000]))
        out.append((L, K, N, Bg))
    return out


# plus shapes with at most 8 expert tiles (N <= 32768) and a minimal one, and
# decode-sized, 16,384 tasks with K = 1, ids up to 2^24, one group per expert
SCHEDULE_SHAPES = _schedule_shapes(7, 12) + [(1500, 20, 20000, 8), (700, 64, 32768, 64),
                                              (5, 3, 7, 1), (256, 64, 1 << 20, 64),
                                              (16384, 1, 50, 7), (129, 64, 1 << 24, 16),
                                              (500, 20, 3000, 1)]


@pytest.mark.parametrize("grouping", ["active", "window"])
@pytest.mark.parametrize("L,K,N,Bg", SCHEDULE_SHAPES)
def test_random_schedule_is_bit_exact(L, K, N, Bg, grouping):
    log(f"[random schedule] L={L} K={K} N={N} B={Bg} {grouping}")
    idx = _ids(L, K, N, seed=L * 131 + K)
    gate = np.random.default_rng(L + K).random((L, K)).astype(np.float32)
    sched = B.schedule_tasks(dev(idx), dev(gate), N, Bg, grouping=grouping)
    torch.cuda.synchronize()
    check_schedule({"expert_idx": dev(idx), "gate": dev(gate)}, sched, N, Bg,
                   grouping=grouping)


# (L, d, N, K, dtype): widths 64..2048 (float32 rows up to 1024 for the token
# form), token counts for every token-centric kernel
EXEC_SHAPES = [
    (1, 64, 3000, 5, "bf16"),
    (37, 128, 9000, 64, "f32"),
    (300, 2048, 20000, 33, "bf16"),
    (1000, 512, 50000, 17, "bf16"),
    (2999, 1024, 8000, 8, "f32"),
    (4096, 256, 30000, 12, "bf16"),
    (5001, 2048, 6000, 3, "bf16"),
    (8203, 128, 40000, 9, "bf16"),
    (8200, 1024, 12000, 4, "f32"),
    # 327,680 tasks over 600,000 experts: the expert rows are streamed
    (8192, 256, 600000, 40, "bf16"),
    # more than 64 tasks per token (the kernels walk them 64 at a time)
    (8193, 128, 40000, 70, "bf16"),
    (100, 256, 5000, 100, "bf16"),
    # d = 64 m, m not a power of two (chunks of 64 .. 512 elements), and rows
    # longer than 4 KiB (token form chunked; the expert form holds d = 4096
    # and float32 d = 2048 in registers, with the same sums in the same order)
    (33, 192, 5000, 7, "bf16"),
    (700, 768, 20000, 64, "bf16"),
    (257, 1536, 9000, 70, "f32"),
    (4100, 3072, 30000, 16, "bf16"),
    (8192, 768, 600000, 40, "bf16"),
    (64, 4096, 3000, 8, "bf16"),
    (300, 2048, 5000, 9, "f32"),
    (5, 320, 100, 3, "f32"),
]


@pytest.mark.parametrize("L,d,N,K,dt", EXEC_SHAPES)
def test_random_executor_forms_agree(L, d, N, K, dt):
    log(f"[random executor] L={L} d={d} N={N} K={K} {dt}")
    seed = L * 7 + d
    idx = _ids(L, K, N, seed=seed)
    gate = np.random.default_rng(seed + 1).random((L, K)).astype(np.float32)
    gate /= gate.sum(axis=1, keepdims=True)
    x = normal((L, d), seed + 2, 1.0, dt)
    w = normal((N, d), seed + 3, float(d) ** -0.5, dt)
    v = normal((N, d), seed + 4, float(d) ** -0.5, dt)
    tx, tw, tv = dev(x), dev(w), dev(v)
    sched = B.schedule_tasks(dev(idx), dev(gate), N, 16)
    ys = {"expert": B.atomic_forward(tx, tw, tv, sched, mode="expert"),
          "token": B.atomic_forward(tx, tw, tv, sched, mode="token")}
    # the token lists inverted from the sorted schedule instead of read from
    # the flattened selection
    flat = (sched.flat_expert, sched.flat_gate)
    sched.flat_expert = sched.flat_gate = None
    ys["token_inverted"] = B.atomic_forward(tx, tw, tv, sched, mode="token")
    sched.flat_expert, sched.flat_gate = flat
    torch.cuda.synchronize()
    ref = host(ys["expert"])
    for name, y in ys.items():
        np.testing.assert_array_equal(host(y).view(np.uint32), ref.view(np.uint32),
                                      err_msg=name)
    toks = np.sort(np.random.default_rng(seed + 5).choice(L, size=min(L, 256), replace=False))
    want = O.atomic_forward(x, w, v, idx, gate, tokens=toks)
    e = rel_err(ref[toks], want)
    log(f"  forms {sorted(ys)} bit-identical; y max|d|/max|y| {e:.2e} (tol {TOL_Y[dt]})")
    assert e <= TOL_Y[dt]
    # accumulate onto a seeded y0: every form the same bits, y0 + routed output
    y0 = np.random.default_rng(seed + 6).standard_normal((L, d)).astype(np.float32)
    modes = ["expert", "token"]
    acc = {m: B.atomic_forward(tx, tw, tv, sched, y=dev(y0), accumulate=True, mode=m)
           for m in modes}
    torch.cuda.synchronize()
    ra = host(acc["expert"])
    for m, y in acc.items():
        np.testing.assert_array_equal(host(y).view(np.uint32), ra.view(np.uint32), err_msg=m)
    ea = rel_err(ra[toks], want + y0[toks])
    log(f"  accumulate: forms bit-identical, max|d|/max|y| {ea:.2e}")
    assert ea <= TOL_Y[dt]
