"""Seeded synthetic workloads for the OmniMoE routed atomic-expert layer.

This module is shared input plumbing: it holds the five workload shapes and
the seeded generators that produce their tensors. It contains none of the
layer's arithmetic (no routing, no selection, no scheduling, no expert
evaluation), so both the CPU oracle and the GPU path may take their inputs
from here without sharing any of the method.

Recipe (the same for every workload):
  * seed of tensor j in workload c = 1000 * c + j, with tensor ids
    x = 0, Wr = 1, Wc = 2, W = 3, V = 4;
  * each tensor is cut into fixed row chunks; chunk i draws from
    numpy PCG64 seeded by SeedSequence(seed).spawn(n_chunks)[i], so the bits
    do not depend on how many threads fill the chunks;
  * x ~ N(0, 1); W, V, Wr, Wc ~ N(0, 1/d), drawn as float32
    (standard_normal, then one multiply by 1/sqrt(d));
  * bf16 workloads round each float32 once to bfloat16 (round to nearest
    even) and keep the bits as uint16; the fp32 workload keeps float32.
  * the router weights are produced in the layout the library consumes:
    wr_t[i, :] holds the d weights that score grid row i (i.e. the i-th
    column of Wr in the pages' notation Wr in R^{d x sqrt(N)}), and likewise
    wc_t for grid columns.
  * the skewed workload adds a Zipf-shaped bias -s * ln(i + 1) (s = 1.1) to
    the logits of row i and, identically, of column i.
  * the shared dense MLP branch (gate, up, down projections; tensor ids
    Wg = 5, Wu = 6, Wd = 7) has hidden width d_ff = 256 * ceil(8 d / 768)
    (two thirds of 4 d, rounded up to a multiple of 256) unless a workload
    fixes it; Wg, Wu [d_ff, d] ~ N(0, 1/d), Wd [d, d_ff] ~ N(0, 1/d_ff).
  * the gated-expert variant's third expert matrix U [N, d] (tensor id 8)
    ~ N(0, 1/d) like W and V.
"""
from __future__ import annotations

import concurrent.futures as _cf
import math
import os
from dataclasses import dataclass, field

import numpy as np

TENSOR_IDS = {"x": 0, "wr": 1, "wc": 2, "w": 3, "v": 4, "wg": 5, "wu": 6, "wd": 7, "u": 8}

# rows per generation chunk; fixed so the bits never depend on thread count
_CHUNK_ELEMS = 1 << 22


@dataclass(frozen=True)
class Workload:
    name: str
    index: int          # position in the workload table; enters the seeds
    L: int              # tokens
    d: int              # model width
    Nr: int             # grid rows
    Nc: int             # grid columns
    kprime: int         # per-axis candidates
    K: int              # experts per token
    B: int              # active experts per group
    dtype: str          # "f32" or "bf16"
    zipf_s: float = 0.0  # 0 = no bias; else bias[i] = -zipf_s * ln(i + 1)
    dff: int = 0         # shared-MLP hidden width; 0 = 256 * ceil(8 d / 768)
    note: str = field(default="", compare=False)

    @property
    def d_ff(self) -> int:
        return self.dff if self.dff else 256 * -(-8 * self.d // 768)

    @property
    def N(self) -> int:
        return self.Nr * self.Nc

    @property
    def M(self) -> int:
        return self.L * self.K

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


WORKLOADS = {
    "tiny": Workload("tiny", 0, L=64, d=128, Nr=32, Nc=32, kprime=8, K=8, B=16,
                     dtype="f32", note="Gaussian, fp32"),
    "small": Workload("small", 1, L=4096, d=1024, Nr=128, Nc=128, kprime=32, K=32,
                      B=64, dtype="bf16", note="Gaussian, bf16"),
    "mid": Workload("mid", 2, L=16384, d=2048, Nr=512, Nc=512, kprime=64, K=64,
                    B=128, dtype="bf16", zipf_s=1.1,
                    note="Gaussian + Zipf(1.1) bias on row/column logits"),
    "large": Workload("large", 3, L=8192, d=2048, Nr=1024, Nc=1024, kprime=64, K=64,
                      B=256, dtype="bf16", note="Gaussian, uniform routing, W+V = 8 GiB"),
    "decode": Workload("decode", 4, L=256, d=2048, Nr=1024, Nc=1024, kprime=64, K=64,
                       B=64, dtype="bf16", note="few tokens, mostly unique experts"),
}


def _threads() -> int:
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return max(1, min(16, n or 1))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    r = u + (np.uint32(0x7FFF) + lsb)
    return (r >> 16).astype(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bits (uint16) to float32 exactly."""
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal(shape, seed: int, scale: float = 1.0, dtype: str = "f32",
           threads: int | None = None) -> np.ndarray:
    """Seeded N(0, scale^2) tensor, chunked so bits are thread-count independent.

    dtype "f32" returns float32; "bf16" returns uint16 bfloat16 bits.
    """
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    n_chunks = max(1, -(-n // _CHUNK_ELEMS))
    seqs = np.random.SeedSequence(seed).spawn(n_chunks)
    out = np.empty(n, dtype=np.uint16 if dtype == "bf16" else np.float32)
    sc = np.float32(scale)

    def fill(i):
        lo, hi = i * _CHUNK_ELEMS, min(n, (i + 1) * _CHUNK_ELEMS)
        g = np.random.Generator(np.random.PCG64(seqs[i]))
        v = g.standard_normal(hi - lo, dtype=np.float32)
        if scale != 1.0:
            v *= sc
        if dtype == "bf16":
            out[lo:hi] = f32_to_bf16_bits(v)
        else:
            out[lo:hi] = v

    nt = threads or _threads()
    if nt == 1 or n_chunks == 1:
        for i in range(n_chunks):
            fill(i)
    else:
        with _cf.ThreadPoolExecutor(nt) as ex:
            list(ex.map(fill, range(n_chunks)))
    return out.reshape(shape)


def zipf_bias(n: int, s: float) -> np.ndarray:
    """bias[i] = -s * ln(i + 1) in float32 (hot indices are the low ones)."""
    i = np.arange(n, dtype=np.float64)
    return (-s * np.log1p(i)).astype(np.float32)


def make_inputs(wl: Workload, parts=("x", "wr", "wc", "w", "v"), threads=None) -> dict:
    """Generate the named tensors of a workload on the host (numpy).

    Returns a dict with any of x [L,d], wr [Nr,d], wc [Nc,d], w [N,d], v [N,d],
    wg [d_ff,d], wu [d_ff,d], wd [d,d_ff], u [N,d] (float32 or uint16 bf16 bits), plus
    row_bias / col_bias (float32 or None).
    """
    c = wl.index
    sd = 1.0 / math.sqrt(wl.d)
    shapes = {"x": (wl.L, wl.d), "wr": (wl.Nr, wl.d), "wc": (wl.Nc, wl.d),
              "w": (wl.N, wl.d), "v": (wl.N, wl.d),
              "wg": (wl.d_ff, wl.d), "wu": (wl.d_ff, wl.d), "wd": (wl.d, wl.d_ff),
              "u": (wl.N, wl.d)}
    scales = {"x": 1.0, "wr": sd, "wc": sd, "w": sd, "v": sd, "wg": sd, "wu": sd,
              "wd": 1.0 / math.sqrt(wl.d_ff), "u": sd}
    out = {}
    for p in parts:
        out[p] = normal(shapes[p], 1000 * c + TENSOR_IDS[p], scales[p], wl.dtype, threads)
    if wl.zipf_s:
        out["row_bias"] = zipf_bias(wl.Nr, wl.zipf_s)
        out["col_bias"] = zipf_bias(wl.Nc, wl.zipf_s)
    else:
        out["row_bias"] = None
        out["col_bias"] = None
    return out


def custom(L, d, Nr, Nc, kprime, K, B, dtype="f32", zipf_s=0.0, index=100, name="custom",
           dff=0):
    """A workload of arbitrary shape (tests use it for ragged and edge cases)."""
    return Workload(name, index, L=L, d=d, Nr=Nr, Nc=Nc, kprime=kprime, K=K, B=B,
                    dtype=dtype, zipf_s=zipf_s, dff=dff)


def tied_logits(L: int, n: int, step: float, seed: int) -> np.ndarray:
    """[L, n] float32 logits drawn N(0, 1) and rounded to multiples of `step`,
    so that many values in a row are equal (inputs where ties decide the
    selection order)."""
    rng = np.random.default_rng(seed)
    z = np.round(rng.standard_normal((L, n)) / step) * step
    return z.astype(np.float32)


def tie_case(L: int, Nr: int, Nc: int, step: float):
    """The tie-heavy row / column logits of the top-K tests: tied_logits with
    seeds Nr and Nc + 1, and signed zeros planted in the first token's rows
    (-0 and +0 compare equal)."""
    za = tied_logits(L, Nr, step, Nr)
    zb = tied_logits(L, Nc, step, Nc + 1)
    za[0, :3] = [0.0, -0.0, 0.0]
    zb[0, :2] = [-0.0, 0.0]
    return za, zb
