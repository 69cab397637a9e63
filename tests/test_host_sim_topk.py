"""The product top-K kernels, compiled for the host and run on a model of the
gfx950 wavefront (tests/host_sim/): every index into LDS and global memory
checked, results bit-exact against the oracle.  CPU only.

csrc/topk.hip is compiled unchanged with clang++ for x86 against
tests/host_sim/hip/hip_runtime.h, which runs each work-item as a fiber and
evaluates every cross-lane operation (ballot, readlane, DPP, shuffle) from all
live lanes at once, as the hardware does in lockstep.  Two builds:
  * address + array-bounds sanitizers: any LDS index outside its array (the
    kernels pass LDS arrays by reference with their sizes) or any global
    index outside its exact-size host buffer stops the run;
  * array-bounds only (fast): the same inputs with LDS filled with other bytes
    before every workgroup (a result that changes would be a read of LDS no
    lane wrote) and with the log-sum-exp shifted by +-1 float32 ulp (the
    device's approximate log may differ from the host's in the last bit).

The main case is the tie-heavy 64 x 64 grid, k' = 16, K = 12, logits in
steps of 0.25 over 97 tokens, where 28 tokens tie at the staircase threshold
and take the exact walk over all k'^2 cells.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import omni_oracle as O
from synth import tie_case

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SIM = os.path.join(ROOT, "tests", "host_sim")
CSRC = os.path.join(ROOT, "cartesian_routed_atomic_amd", "csrc")
CLANG = "/opt/rocm/llvm/bin/clang++"

# (Nr, Nc, k', K, step): the tie cases of the GPU top-K test that fit a CPU run
CASES = [(64, 64, 16, 12, 0.25), (40, 24, 8, 8, 0.5), (128, 96, 64, 64, 1.0),
         (33, 65, 5, 25, 0.5), (64, 64, 16, 12, 0.5), (100, 80, 32, 20, 0.25),
         (64, 64, 64, 64, 0.25), (64, 64, 16, 1, 0.25), (256, 48, 48, 64, 2.0)]
L_TOKENS = 97   # the GPU test's token count, for the main case
L_OTHER = 48    # the other cases: the first 48 of those tokens


def _build(tmp, name, sanitize):
    exe = os.path.join(tmp, name)
    cmd = [CLANG, "-std=c++20", "-O1", "-g", "-fno-sanitize-recover=all", *sanitize,
           "-I", SIM, "-I", CSRC, "-I", os.path.join(ROOT, "include"),
           os.path.join(SIM, "topk_sim.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return exe


@pytest.fixture(scope="module")
def sims(tmp_path_factory):
    if not os.path.exists(CLANG):
        pytest.skip("ROCm clang++ not installed")
    tmp = str(tmp_path_factory.mktemp("topk_sim"))
    with cf.ThreadPoolExecutor(2) as ex:
        asan = ex.submit(_build, tmp, "topk_asan",
                         ["-fsanitize=address,undefined", "-fsanitize=array-bounds"])
        ubsan = ex.submit(_build, tmp, "topk_ubsan",
                          ["-fsanitize=undefined", "-fsanitize=array-bounds"])
        yield {"asan": asan.result(), "ubsan": ubsan.result(), "tmp": tmp}
    shutil.rmtree(tmp, ignore_errors=True)


def _run(exe, tmp, tag, za, zb, kp, K, fill=0, ulps=0):
    L, Nr = za.shape
    Nc = zb.shape[1]
    fin = os.path.join(tmp, f"in_{tag}.bin")
    fout = os.path.join(tmp, f"out_{tag}.bin")
    with open(fin, "wb") as f:
        np.array([L, Nr, Nc, kp, K], np.int32).tofile(f)
        za.tofile(f)
        zb.tofile(f)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe, fin, fout, str(fill), str(ulps)], capture_output=True, text=True,
                       env=env, timeout=600)
    assert r.returncode == 0, f"{tag}: exit {r.returncode}\n{r.stderr[-4000:]}"
    b = open(fout, "rb").read()
    out, o = {}, 0
    for name, dt, n in (("idx", np.int32, L * K), ("score", np.float32, L * K),
                        ("gate", np.float32, L * K), ("a", np.float32, L * Nr),
                        ("b", np.float32, L * Nc), ("R", np.int32, L * kp),
                        ("C", np.int32, L * kp), ("tie", np.int32, L)):
        out[name] = np.frombuffer(b, dt, n, o)
        o += n * 4
    out["raw"] = b
    return out


def _check_against_oracle(out, za, zb, kp, K):
    L, Nr = za.shape
    Nc = zb.shape[1]
    a, b = out["a"].reshape(L, Nr), out["b"].reshape(L, Nc)
    assert float(np.abs(a - O.log_softmax_rows(za)).max()) <= 1e-5
    assert float(np.abs(b - O.log_softmax_rows(zb)).max()) <= 1e-5
    idx, score, gate, R, C = O.product_topk(a, b, kp, K)
    np.testing.assert_array_equal(out["R"].reshape(L, kp), R)
    np.testing.assert_array_equal(out["C"].reshape(L, kp), C)
    np.testing.assert_array_equal(out["idx"].reshape(L, K), idx)
    np.testing.assert_array_equal(out["score"].reshape(L, K).view(np.uint32),
                                  score.view(np.uint32))
    assert float(np.abs(out["gate"].reshape(L, K) - gate).max()) <= 2e-6


def test_tie_cases_stay_in_bounds_and_match_the_oracle(sims):
    jobs = []
    with cf.ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        for i, (Nr, Nc, kp, K, step) in enumerate(CASES):
            za, zb = tie_case(L_TOKENS if i == 0 else L_OTHER, Nr, Nc, step)
            jobs.append((i, za, zb, kp, K,
                         ex.submit(_run, sims["asan"], sims["tmp"], f"a{i}", za, zb, kp, K)))
        flagged = {}
        for i, za, zb, kp, K, fut in jobs:
            out = fut.result()
            _check_against_oracle(out, za, zb, kp, K)
            flagged[CASES[i]] = int(out["tie"].sum())
    print("tokens taking the exact fix-up per case:", flagged)
    # the main case exercises the fix-up kernel on a good share of its tokens
    assert flagged[CASES[0]] >= 10


def test_tie_case_does_not_read_unwritten_lds_and_holds_under_log_ulps(sims):
    Nr, Nc, kp, K, step = CASES[0]
    za, zb = tie_case(L_TOKENS, Nr, Nc, step)
    with cf.ThreadPoolExecutor(5) as ex:
        f = {(fill, ulps): ex.submit(_run, sims["ubsan"], sims["tmp"], f"u{fill}_{ulps}", za,
                                     zb, kp, K, fill, ulps)
             for fill, ulps in ((0, 0), (255, 0), (90, 0), (90, 1), (90, -1))}
        outs = {k: v.result() for k, v in f.items()}
    # the LDS fill byte changes nothing
    assert outs[(0, 0)]["raw"] == outs[(255, 0)]["raw"] == outs[(90, 0)]["raw"]
    for k, out in outs.items():
        _check_against_oracle(out, za, zb, kp, K)
        assert int(out["tie"].sum()) >= 10, k
