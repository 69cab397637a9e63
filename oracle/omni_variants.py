"""CPU oracle for variants of the OmniMoE routed layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the GPU library.

Variants:
  * SwiGLU-gated atomic expert.  [EXPL, Atomic Expert] and [GS-ZH §2.1] name
    SwiGLU as the expert's activation while the expert has one input vector
    w_in, which leaves nothing to gate (the default path reads sigma as SiLU).
    The variant gives every expert a third vector u_i, stored as row i of a
    third global matrix U [N, d] next to W and V, and reads the expert as
        E_i(x) = silu(x . w_in) * (x . u_i) * w_out,
    the SwiGLU form silu(a) * b with a = x . w_in (the argument sigma already
    has) and b = x . u_i.  Each expert then has 3d parameters instead of the
    2d the pages state.  PARITY UNPINNED against the pages (a reading); the
    pins fix its arithmetic.
  * Flat router (the baseline the Cartesian Product Router replaces,
    [GS-NL §2.2] and the ablation table of [EXPL]): one logit per expert,
    z = x Wf^T + bias with Wf [N, d]; log-softmax over all N; top-K by
    (log p desc, e asc); gates = softmax over the K selected log p.

Citation keys as in omni_oracle.
"""
from __future__ import annotations

import numpy as np

from oracle.omni_oracle import gates, log_softmax_rows, silu, widen


def atomic_forward_glu_f64(x, w, u, v, expert_idx, gate, tokens=None):
    """y_t = sum_k g_tk silu(x_t . W[e]) (x_t . U[e]) V[e], float64.
    tokens: optional subset of token ids.  Returns [len(tokens) or L, d]."""
    expert_idx = np.asarray(expert_idx)
    gate = np.asarray(gate, dtype=np.float32)
    L = expert_idx.shape[0]
    toks = np.arange(L) if tokens is None else np.asarray(tokens)
    y = np.zeros((len(toks), np.asarray(x).shape[1]))
    for n, t in enumerate(toks):
        xt = widen(x[t])
        rows = expert_idx[t].astype(np.int64)
        a = widen(w[rows]) @ xt
        b = widen(u[rows]) @ xt
        y[n] = (gate[t].astype(np.float64) * silu(a) * b) @ widen(v[rows])
    return y


def atomic_forward_glu(x, w, u, v, expert_idx, gate, tokens=None):
    """atomic_forward_glu_f64 rounded once to float32."""
    return atomic_forward_glu_f64(x, w, u, v, expert_idx, gate, tokens).astype(np.float32)


def flat_router_logp(x, wf, bias=None):
    """log p = log_softmax(x Wf^T + bias) over all N experts: float64 arithmetic,
    rounded to float32 (as the product router's per-axis log-probabilities)."""
    z = widen(x) @ widen(wf).T
    if bias is not None:
        z = z + widen(bias)[None, :]
    return log_softmax_rows(z).astype(np.float32)


def flat_topk(logp, K):
    """Top-K experts of each row of logp [L, N] by (log p desc, e asc), values
    compared as float32 numbers; gates = softmax over the K selected log p.
    Returns idx [L, K] int32, score [L, K] float32, gate [L, K] float32."""
    logp = np.asarray(logp, dtype=np.float32)
    L, N = logp.shape
    idx = np.empty((L, K), np.int32)
    for t in range(L):
        e = np.arange(N)
        order = np.lexsort((e, -logp[t].astype(np.float64)))
        idx[t] = order[:K]
    score = np.take_along_axis(logp, idx.astype(np.int64), axis=1)
    return idx, score, gates(score)
