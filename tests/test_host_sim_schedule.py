"""Expert-Centric Scheduling (csrc/schedule.hip), compiled for the host and
run on the wave model of tests/host_sim/: every LDS and global index checked
by the address and array-bounds sanitizers, every output bit-exact against
the oracle's schedule.  CPU only.

The cases reach each launch sequence of the pipeline: at most 32 sort
tiles (the scatter sums its rows of tile counts itself) and more (a
separate row scan); a single pass (offsets from the digit bases) with
digits of 7 to 11 bits, two and three passes (offsets from the sorted
keys); the separate tile count and the inline count; both groupings.
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


def _routing(L, K, N, s, seed):
    """K distinct experts per token: Zipf(s) over a random permutation of the
    ids (s = 0: uniform)."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(N)
    p = 1.0 / np.arange(1, N + 1) ** s
    p /= p.sum()
    idx = np.empty((L, K), np.int32)
    for t in range(L):
        idx[t] = perm[rng.choice(N, size=K, replace=False, p=p)]
    g = rng.random((L, K)).astype(np.float32)
    return idx, g


def _run(sim, tag, L, K, N, B, window, s, seed, fill):
    idx, g = _routing(L, K, N, s, seed)
    fin = os.path.join(sim["tmp"], f"in_{tag}.bin")
    fout = os.path.join(sim["tmp"], f"out_{tag}.bin")
    with open(fin, "wb") as f:
        np.array([L, K, N, B, int(window)], np.int32).tofile(f)
        idx.tofile(f)
        g.tofile(f)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([sim["exe"], fin, fout, str(fill)], capture_output=True, text=True,
                       env=env, timeout=900)
    assert r.returncode == 0, f"{tag}: exit {r.returncode}\n{r.stderr[-4000:]}"
    M = L * K
    n_act = min(M, N)
    G = O.max_groups(N, L, K, B, "window" if window else "active")
    b = np.fromfile(fout, np.int32)
    out, o = {}, 0
    for name, n in (("counts", 2), ("active", n_act), ("group_offsets", G + 1),
                    ("task_token", M), ("task_expert", M), ("task_gate", M),
                    ("task_index", M), ("rank", N)):
        out[name] = b[o:o + n]
        o += n
    out["task_gate"] = out["task_gate"].view(np.float32)
    return idx, g, out


# (tag, L, K, N, B, window, zipf s, seed)
CASES = [
    # one 2048-task tile, 7-bit digits, 16 expert tiles (separate count)
    ("decode", 64, 16, 1 << 16, 8, False, 0.0, 1),
    # inline count (one expert tile), a ragged sort tile
    ("inline", 50, 8, 2000, 4, False, 0.0, 2),
    # heavy duplicates: Zipf routing, 16 tiles, 11-bit digits
    ("zipf", 1024, 32, 1 << 16, 16, False, 1.2, 3),
    # id windows, empty windows
    ("window", 40, 8, 3000, 16, True, 0.0, 4),
    # exactly 2048 possible groups: one 11-bit pass, offsets up to G = 2048
    ("g2048", 64, 32, 1 << 12, 1, False, 0.0, 5),
    # two 6-bit passes (2400 possible groups), offsets from the sorted keys
    ("twopass", 300, 8, 5000, 1, False, 0.0, 6),
    # two passes over id windows, most windows empty
    ("window2", 20, 4, 10000, 2, True, 0.0, 7),
    # 35 tiles of 2048: the separate row scan, offsets from the digit bases
    ("wide", 1100, 64, 1 << 17, 64, False, 0.0, 8),
    # three 6-bit passes (70,400 possible groups), Zipf routing
    ("threepass", 1100, 64, 1 << 17, 1, False, 0.8, 10),
]


def test_schedule_in_bounds_and_exact(sim):
    with cf.ThreadPoolExecutor(min(len(CASES), os.cpu_count() or 1)) as ex:
        futs = {c[0]: ex.submit(_run, sim, *c, 0xA5 if i % 2 else 0)
                for i, c in enumerate(CASES)}
        outs = {k: f.result() for k, f in futs.items()}
    for tag, L, K, N, B, window, s, seed in CASES:
        idx, g, out = outs[tag]
        want = O.build_schedule(idx, g, N, B, "window" if window else "active")
        na = want["n_active"]
        assert out["counts"].tolist() == [na, want["n_groups"]], tag
        assert np.array_equal(out["active"][:na], want["active"]), tag
        assert np.array_equal(out["group_offsets"], want["group_offsets"]), tag
        for k in ("task_token", "task_expert", "task_index"):
            assert np.array_equal(out[k], want[k]), (tag, k)
        assert np.array_equal(out["task_gate"].view(np.int32),
                              want["task_gate"].view(np.int32)), tag
        assert np.array_equal(out["rank"][want["active"]], np.arange(na)), tag
