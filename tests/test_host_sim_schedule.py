"""The one-workgroup schedule (csrc/schedule_small.hip, at most 16,384 tasks
and groups), compiled for the host and run on the wave model of
tests/host_sim/: every LDS and global index checked by the address and
array-bounds sanitizers, every output bit-exact against the oracle's
build_schedule, LDS fill bytes without effect.  CPU only.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import omni_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SIM = os.path.join(ROOT, "tests", "host_sim")
CSRC = os.path.join(ROOT, "cartesian_routed_atomic_amd", "csrc")
CLANG = "/opt/rocm/llvm/bin/clang++"


@pytest.fixture(scope="module")
def sim(tmp_path_factory):
    if not os.path.exists(CLANG):
        pytest.skip("ROCm clang++ not installed")
    tmp = str(tmp_path_factory.mktemp("schedule_sim"))
    exe = os.path.join(tmp, "schedule_sim")
    r = subprocess.run([CLANG, "-std=c++20", "-O1", "-g", "-fno-sanitize-recover=all",
                        "-fsanitize=address,undefined", "-fsanitize=array-bounds", "-I", SIM,
                        "-I", CSRC, "-I", os.path.join(ROOT, "include"),
                        os.path.join(SIM, "schedule_sim.cpp"), "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    yield {"exe": exe, "tmp": tmp}
    shutil.rmtree(tmp, ignore_errors=True)


def _ids(L, K, N, seed, zipf):
    """K distinct ids per token, uniform or Zipf-skewed over the ids."""
    rng = np.random.default_rng(seed)
    if zipf:
        p = 1.0 / np.arange(1, N + 1) ** 1.1
        p /= p.sum()
        return np.stack([rng.choice(N, size=K, replace=False, p=p)
                         for _ in range(L)]).astype(np.int32)
    if K * 4 <= N:  # rejection-free enough: draw, then fix duplicates per token
        idx = rng.integers(0, N, size=(L, K), dtype=np.int64)
        for t in range(L):
            while len(set(idx[t])) < K:
                idx[t] = rng.choice(N, size=K, replace=False)
        return idx.astype(np.int32)
    return np.stack([rng.choice(N, size=K, replace=False) for _ in range(L)]).astype(np.int32)


def _run(sim, tag, L, K, N, B, grouping, seed, zipf, fill=0):
    idx = _ids(L, K, N, seed, zipf)
    gate = np.random.default_rng(seed + 1).random((L, K)).astype(np.float32)
    G = O.max_groups(N, L, K, B, grouping)
    fin = os.path.join(sim["tmp"], f"in_{tag}.bin")
    fout = os.path.join(sim["tmp"], f"out_{tag}.bin")
    with open(fin, "wb") as f:
        np.array([L, K, N, B, int(grouping == "window"), G], np.int32).tofile(f)
        idx.tofile(f)
        gate.tofile(f)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([sim["exe"], fin, fout, str(fill)], capture_output=True, text=True,
                       env=env, timeout=900)
    assert r.returncode == 0, f"{tag}: exit {r.returncode}\n{r.stderr[-4000:]}"
    M = L * K
    b = np.fromfile(fout, np.uint8)
    sizes = [("counts", np.int32, 2), ("active", np.int32, min(N, M)), ("off", np.int32, G + 1),
             ("task_token", np.int32, M), ("task_expert", np.int32, M),
             ("task_gate", np.float32, M), ("task_index", np.int32, M)]
    out, o = {}, 0
    for name, dt, n in sizes:
        out[name] = b[o:o + 4 * n].view(dt)
        o += 4 * n
    assert o == b.size
    return out, O.build_schedule(idx, gate, N, B, grouping)


# (tag, L, K, N, B, grouping, seed, zipf): decode-sized (16,384 tasks over 2^20
# ids, three id passes); ids up to 2^24 (four passes); one task; the task
# limit with K = 1; id windows (empty windows included); B = 1 (a group per
# expert, more than 256 groups: two key passes); Zipf-skewed ids
CASES = [("decode", 256, 64, 1 << 20, 64, "active", 1, False),
         ("ids24", 129, 64, 1 << 24, 16, "active", 2, False),
         ("one", 1, 1, 1, 1, "active", 3, False),
         ("k1", 16384, 1, 50, 7, "active", 4, False),
         ("window", 37, 16, 300, 1, "window", 5, False),
         ("window64", 250, 64, 16384, 64, "window", 6, False),
         ("b1", 500, 20, 3000, 1, "active", 7, False),
         ("zipf", 300, 32, 5000, 16, "active", 8, True)]


def _check(tag, got, want):
    n = want["n_active"]
    assert int(got["counts"][0]) == n and int(got["counts"][1]) == want["n_groups"], tag
    np.testing.assert_array_equal(got["active"][:n], want["active"], err_msg=tag)
    np.testing.assert_array_equal(got["off"], want["group_offsets"], err_msg=tag)
    for k in ("task_token", "task_expert", "task_index"):
        np.testing.assert_array_equal(got[k], want[k], err_msg=f"{tag} {k}")
    np.testing.assert_array_equal(got["task_gate"].view(np.uint32),
                                  want["task_gate"].view(np.uint32), err_msg=tag)


def test_small_schedule_bit_exact(sim):
    with cf.ThreadPoolExecutor(min(len(CASES), os.cpu_count() or 1)) as ex:
        futs = {c[0]: ex.submit(_run, sim, *c) for c in CASES}
        outs = {k: f.result() for k, f in futs.items()}
    for c in CASES:
        got, want = outs[c[0]]
        _check(c[0], got, want)
        print(f"{c[0]}: {want['n_active']} active, {want['n_groups']} groups: bit-exact")


def test_small_schedule_does_not_read_unwritten_lds(sim):
    a, want = _run(sim, "fill255", 100, 9, 700, 5, "active", 9, True, fill=255)
    _check("fill255", a, want)
