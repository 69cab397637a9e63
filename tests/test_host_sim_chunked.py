"""The chunked executor kernels (csrc/chunked.hip: rows of any d = 64 m, the
row taken in chunks), compiled for the host and run on the wave model of
tests/host_sim/: every global index checked by the address and array-bounds
sanitizers, y within the float32-accumulation bar of the oracle, and the
expert- and token-centric forms bit-identical to each other.  CPU only.

Widths: m = 3, 5, 12, 24 and 48 (d = 192, 320, 768, 1536, 3072: chunks of 64,
64, 256, 512 and 512 elements, so 1 to 8 elements per lane and 3 to 6 chunks
a row), bf16 and float32; K below, at and above one wave of tasks (64).
"""
import concurrent.futures as cf
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import omni_oracle as O
from oracle import omni_variants as OV
from synth import normal

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SIM = os.path.join(ROOT, "tests", "host_sim")
CSRC = os.path.join(ROOT, "cartesian_routed_atomic_amd", "csrc")
CLANG = "/opt/rocm/llvm/bin/clang++"
BAR = 1e-4  # max |y - y_oracle| / max |y_oracle| (float32 sums of exact products)


@pytest.fixture(scope="module")
def sim(tmp_path_factory):
    if not os.path.exists(CLANG):
        pytest.skip("ROCm clang++ not installed")
    tmp = str(tmp_path_factory.mktemp("chunked_sim"))
    exe = os.path.join(tmp, "chunked_sim")
    r = subprocess.run([CLANG, "-std=c++20", "-O1", "-g", "-fno-sanitize-recover=all",
                        "-fsanitize=address,undefined", "-fsanitize=array-bounds", "-I", SIM,
                        "-I", CSRC, "-I", os.path.join(ROOT, "include"),
                        os.path.join(SIM, "chunked_sim.cpp"), "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    yield {"exe": exe, "tmp": tmp}
    shutil.rmtree(tmp, ignore_errors=True)


def _inputs(L, K, d, N, dtype, seed, glu):
    x = normal((L, d), seed, 1.0, dtype)
    w = normal((N, d), seed + 1, d ** -0.5, dtype)
    u = normal((N, d), seed + 2, d ** -0.5, dtype) if glu else None
    v = normal((N, d), seed + 3, d ** -0.5, dtype)
    rng = np.random.default_rng(seed + 4)
    idx = np.stack([rng.choice(N, size=K, replace=False) for _ in range(L)]).astype(np.int32)
    g = (rng.random((L, K)) + 0.05).astype(np.float32)
    g /= g.sum(axis=1, keepdims=True)
    return x, w, u, v, idx, g.astype(np.float32)


def _run(sim, tag, L, K, d, N, dtype, form, glu, acc, flat, seed):
    x, w, u, v, idx, g = _inputs(L, K, d, N, dtype, seed, glu)
    s = O.build_schedule(idx, g, N, 8)
    y0 = (np.random.default_rng(seed + 5).standard_normal((L, d)).astype(np.float32)
          if acc else np.zeros((L, d), np.float32))
    fin = os.path.join(sim["tmp"], f"in_{tag}.bin")
    fout = os.path.join(sim["tmp"], f"out_{tag}.bin")
    with open(fin, "wb") as f:
        np.array([L, K, d, N, int(dtype == "bf16"), form, int(glu), int(acc), int(flat)],
                 np.int32).tofile(f)
        for a in (x, w, u, v):
            if a is not None:
                a.tofile(f)
        idx.ravel().tofile(f)
        g.ravel().tofile(f)
        for k in ("task_token", "task_expert", "task_gate", "task_index"):
            s[k].tofile(f)
        y0.tofile(f)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([sim["exe"], fin, fout], capture_output=True, text=True, env=env,
                       timeout=900)
    assert r.returncode == 0, f"{tag}: exit {r.returncode}\n{r.stderr[-4000:]}"
    y = np.fromfile(fout, np.float32).reshape(L, d)
    want = (OV.atomic_forward_glu(x, w, u, v, idx, g) if glu
            else O.atomic_forward(x, w, v, idx, g)) + y0
    err = float(np.abs(y - want).max() / np.abs(want).max())
    return {"y": y, "err": err}


# (tag, L, K, d, N, dtype, accumulate, seed)
SHAPES = [("m3", 9, 7, 192, 40, "bf16", False, 11),
          ("m5", 6, 64, 320, 96, "bf16", True, 21),
          ("m12", 5, 70, 768, 128, "bf16", False, 31),
          ("m24", 3, 13, 1536, 32, "bf16", False, 41),
          ("m48", 3, 9, 3072, 24, "bf16", True, 51),
          ("f32m3", 7, 5, 192, 16, "f32", False, 61),
          ("f32m24", 3, 66, 1536, 80, "f32", False, 71)]


def test_chunked_forms_in_bounds_within_bar_and_identical(sim):
    jobs = {}
    with cf.ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        for tag, L, K, d, N, dt, acc, seed in SHAPES:
            # expert-centric form; token-centric with and without the flattened selection
            for form, flat in ((1, 1), (2, 1), (2, 0)):
                jobs[(tag, form, flat)] = ex.submit(_run, sim, f"{tag}_{form}{flat}", L, K, d, N,
                                                    dt, form, False, acc, flat, seed)
        outs = {k: f.result() for k, f in jobs.items()}
    for tag, L, K, d, N, dt, acc, seed in SHAPES:
        e, t, tu = outs[(tag, 1, 1)], outs[(tag, 2, 1)], outs[(tag, 2, 0)]
        print(f"{tag}: d={d} K={K} {dt}: max|dy|/max|y| {e['err']:.1e}")
        assert e["err"] <= BAR, (tag, e["err"])
        np.testing.assert_array_equal(e["y"].view(np.uint32), t["y"].view(np.uint32))
        np.testing.assert_array_equal(t["y"].view(np.uint32), tu["y"].view(np.uint32))


def test_chunked_gated_variant(sim):
    for tag, L, K, d, N, dt in (("glu_m3", 5, 9, 192, 24, "bf16"),
                                ("glu_m12", 4, 65, 768, 96, "bf16"),
                                ("glu_f32m5", 3, 6, 320, 12, "f32")):
        o = _run(sim, tag, L, K, d, N, dt, 2, True, False, 1, 81)
        print(f"{tag}: max|dy|/max|y| {o['err']:.1e}")
        assert o["err"] <= BAR, (tag, o["err"])
