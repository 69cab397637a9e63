"""CPU oracle for the whole OmniMoE layer: shared dense MLP + routed branch.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the GPU library.

[GS-NL §2] the layer is hybrid: a dense MLP branch that every token passes
through, shared by all inputs, next to the pool of routed atomic experts;
[GS-NL §2.1] "Shared Dense MLP" calls it a standard dense MLP that handles
general semantics while the routed branch handles long-tail knowledge;
[GS-ZH §2.1] and [EXPL, Atomic Expert] say the same.

Readings taken where the pages leave a step open (each is a choice):
  * the dense MLP has the gated SwiGLU form used by current dense language
    models: m(x) = (silu(x Wg^T) * (x Wu^T)) Wd^T.  [EXPL, Atomic Expert]
    names SwiGLU as the activation, which a rank-1 atomic expert (one input
    projection) cannot use; a dense MLP can.  PARITY UNPINNED against the
    pages (they print no formula for this branch); the pins below fix the
    arithmetic of the form chosen.
  * storage: Wg, Wu [d_ff, d] (row j = hidden unit j's input weights),
    Wd [d, d_ff] (row c = output feature c's weights over the hidden units).
  * the layer output is the plain sum m(x) + y_routed(x) (the pages weight
    neither branch).
  * hidden width d_ff is a free parameter.

Citation keys as in omni_oracle.
"""
from __future__ import annotations

import numpy as np

from oracle.omni_oracle import atomic_forward_f64, build_schedule, product_topk, router_logp
from oracle.omni_oracle import silu, widen


def shared_mlp_f64(x, w_gate, w_up, w_down):
    """m(x) = (silu(x Wg^T) * (x Wu^T)) Wd^T in float64.  [GS-NL §2.1]
    x [L, d]; w_gate, w_up [d_ff, d]; w_down [d, d_ff] (float32 or bf16 bits).
    Returns [L, d] float64."""
    xf = widen(x)
    g = xf @ widen(w_gate).T           # [L, d_ff] gate pre-activations
    u = xf @ widen(w_up).T             # [L, d_ff] up projections
    return (silu(g) * u) @ widen(w_down).T


def shared_mlp(x, w_gate, w_up, w_down):
    """shared_mlp_f64 rounded once to float32."""
    return shared_mlp_f64(x, w_gate, w_up, w_down).astype(np.float32)


def shared_mlp_literal(x, w_gate, w_up, w_down):
    """The same branch as scalar loops over (token, hidden unit, feature),
    float64 (self-check for small inputs)."""
    xf = widen(x)
    wg, wu, wd = widen(w_gate), widen(w_up), widen(w_down)
    L, d = xf.shape
    d_ff = wg.shape[0]
    y = np.zeros((L, wd.shape[0]))
    for t in range(L):
        for j in range(d_ff):
            a = 0.0
            b = 0.0
            for c in range(d):
                a += xf[t, c] * wg[j, c]
                b += xf[t, c] * wu[j, c]
            hj = float(silu(a)) * b
            for o in range(wd.shape[0]):
                y[t, o] += hj * wd[o, j]
    return y


def layer_forward(x, wr_t, wc_t, w, v, w_gate, w_up, w_down, kprime, K, B,
                  row_bias=None, col_bias=None):
    """The whole layer: routed branch (router -> product top-K + gates ->
    schedule -> y_routed) plus the shared dense MLP, summed in float64 and
    rounded once to float32.  [GS-NL §2]"""
    a, b = router_logp(x, wr_t, wc_t, row_bias, col_bias)
    idx, score, gate, R, C = product_topk(a, b, kprime, K)
    N = np.asarray(wr_t).shape[0] * np.asarray(wc_t).shape[0]
    sched = build_schedule(idx, gate, N, B)
    yr = atomic_forward_f64(x, w, v, idx, gate)
    ys = shared_mlp_f64(x, w_gate, w_up, w_down)
    return {"expert_idx": idx, "gate": gate, "schedule": sched,
            "y_routed": yr, "y_shared": ys, "y": (yr + ys).astype(np.float32)}
