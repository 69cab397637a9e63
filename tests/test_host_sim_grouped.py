"""The grouped executor form (csrc/grouped.hip), compiled for the host and run
on the wave model of tests/host_sim/: every LDS and global index checked by
the address and array-bounds sanitizers, the hot set exact against its rule,
y within the bf16 bar of the oracle.  CPU only.

The model evaluates v_mfma_f32_16x16x32_bf16 from its lane layout (A[m][k] in
lane m + 16 (k / 8), B[k][n] in lane n + 16 (k / 8), D[m][n] in lane
n + 16 (m / 4)), the layout the router's MFMA kernel uses on the GPU.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import omni_oracle as O
from synth import normal

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SIM = os.path.join(ROOT, "tests", "host_sim")
CSRC = os.path.join(ROOT, "cartesian_routed_atomic_amd", "csrc")
CLANG = "/opt/rocm/llvm/bin/clang++"
HOT_MAX, HOT_DIV = 512, 64


@pytest.fixture(scope="module")
def sim(tmp_path_factory):
    if not os.path.exists(CLANG):
        pytest.skip("ROCm clang++ not installed")
    tmp = str(tmp_path_factory.mktemp("grouped_sim"))
    exe = os.path.join(tmp, "grouped_sim")
    r = subprocess.run([CLANG, "-std=c++20", "-O1", "-g", "-fno-sanitize-recover=all",
                        "-fsanitize=address,undefined", "-fsanitize=array-bounds", "-I", SIM,
                        "-I", CSRC, "-I", os.path.join(ROOT, "include"),
                        os.path.join(SIM, "grouped_sim.cpp"), "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    yield {"exe": exe, "tmp": tmp}
    shutil.rmtree(tmp, ignore_errors=True)


def _routing(L, K, N, s, seed):
    """K distinct experts per token: Zipf(s) over ids (s = 0: uniform)."""
    rng = np.random.default_rng(seed)
    p = 1.0 / np.arange(1, N + 1) ** s
    p /= p.sum()
    idx = np.empty((L, K), np.int32)
    for t in range(L):
        idx[t] = rng.choice(N, size=K, replace=False, p=p)
    g = rng.random((L, K)).astype(np.float32) + np.float32(0.05)
    g /= g.sum(axis=1, keepdims=True)
    return idx, g.astype(np.float32)


def _hot_rule(idx, L, N):
    """The hot set the form documents: experts with at least tau tasks, tau =
    max(2, ceil(L / 64)) doubled until at most 512 experts reach it."""
    cnt = np.bincount(idx.ravel(), minlength=N)
    tau = max(2, -(-L // HOT_DIV))
    while (cnt >= tau).sum() > HOT_MAX:
        tau *= 2
    return np.flatnonzero(cnt >= tau).astype(np.int32), tau


def _run(sim, tag, L, K, d, N, s, seed, accumulate=False, fill=0, nt=False):
    x = normal((L, d), seed, 1.0, "bf16")
    w = normal((N, d), seed + 1, d ** -0.5, "bf16")
    v = normal((N, d), seed + 2, d ** -0.5, "bf16")
    idx, g = _routing(L, K, N, s, seed + 3)
    sched = O.build_schedule(idx, g, N, 16)
    y0 = (np.random.default_rng(seed + 4).standard_normal((L, d)).astype(np.float32)
          if accumulate else np.zeros((L, d), np.float32))
    fin = os.path.join(sim["tmp"], f"in_{tag}.bin")
    fout = os.path.join(sim["tmp"], f"out_{tag}.bin")
    with open(fin, "wb") as f:
        np.array([L, K, d, N, int(accumulate)], np.int32).tofile(f)
        for a in (x, w, v):
            a.tofile(f)
        idx.tofile(f)
        g.tofile(f)
        sched["task_expert"].astype(np.int32).tofile(f)
        y0.tofile(f)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([sim["exe"], fin, fout, str(fill), str(int(nt))], capture_output=True,
                       text=True, env=env, timeout=900)
    assert r.returncode == 0, f"{tag}: exit {r.returncode}\n{r.stderr[-4000:]}"
    b = np.fromfile(fout, np.uint8)
    y = b[:L * d * 4].view(np.float32).reshape(L, d)
    misc = b[L * d * 4:L * d * 4 + 16].view(np.int32)
    hot = b[L * d * 4 + 16:].view(np.int32)
    want = O.atomic_forward(x, w, v, idx, g) + y0
    err = float(np.abs(y - want).max() / np.abs(want).max())
    return {"y": y, "misc": misc, "hot": hot, "err": err, "idx": idx}


# (tag, L, K, d, N, zipf s, seed, accumulate): a ragged last tile and a hot set;
# the 512 cap reached (the threshold doubles); no hot expert (every task per
# task); accumulate onto y; one task per token (and rows of one 64-column
# chunk); the larger tiles; rows of several x chunk rounds
CASES = [("skew", 150, 16, 128, 2048, 1.1, 11, False),
         ("cap", 200, 64, 128, 1024, 0.8, 21, False),
         ("uniform", 130, 8, 64, 65536, 0.0, 31, False),
         ("accumulate", 129, 12, 256, 512, 1.0, 41, True),
         ("k1", 64, 1, 64, 64, 1.2, 51, False),
         # 32- and 64-token tiles (from 8192 and 16384 tokens), ragged last tiles
         ("tile32", 8200, 2, 64, 512, 1.1, 61, False),
         ("tile64", 16400, 2, 64, 1024, 1.1, 71, True),
         # rows of 8 x 64 columns: the first product's x ring runs several rounds
         ("d512", 96, 8, 512, 256, 1.1, 81, False)]


def test_grouped_form_in_bounds_hot_set_exact_y_within_bar(sim):
    with cf.ThreadPoolExecutor(min(len(CASES), os.cpu_count() or 1)) as ex:
        futs = {c[0]: ex.submit(_run, sim, *c) for c in CASES}
        outs = {k: f.result() for k, f in futs.items()}
    for tag, L, K, d, N, s, seed, acc in CASES:
        o = outs[tag]
        hot, tau = _hot_rule(o["idx"], L, N)
        print(f"{tag}: |H| {len(hot)} tau {tau}; y max|d|/max|y| {o['err']:.2e}")
        assert int(o["misc"][1]) == len(hot) and int(o["misc"][2]) == tau, (tag, o["misc"])
        np.testing.assert_array_equal(o["hot"][:len(hot)], hot)
        assert o["err"] <= 2e-2, (tag, o["err"])
    assert len(_hot_rule(outs["uniform"]["idx"], 130, 65536)[0]) == 0
    assert len(_hot_rule(outs["skew"]["idx"], 150, 2048)[0]) > 0
    assert _hot_rule(outs["cap"]["idx"], 200, 1024)[1] > max(2, -(-200 // HOT_DIV))


def test_grouped_form_does_not_read_unwritten_lds(sim):
    a = _run(sim, "fill0", 150, 16, 128, 2048, 1.1, 11, fill=0)
    b = _run(sim, "fill255", 150, 16, 128, 2048, 1.1, 11, fill=255)
    np.testing.assert_array_equal(a["y"].view(np.uint32), b["y"].view(np.uint32))
    # the cold kernel with the nontemporal hint on its rows: the same bits
    c = _run(sim, "nt", 150, 16, 128, 2048, 1.1, 11, nt=True)
    np.testing.assert_array_equal(a["y"].view(np.uint32), c["y"].view(np.uint32))
