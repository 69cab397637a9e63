"""CPU oracle for the backward pass of the OmniMoE routed atomic-expert layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite uses it.  It shares no code with the
GPU library.

The pages train models with this layer but print no backward pass, so the
gradients here are derived by hand from the forward computation of
omni_oracle (chain rule through every differentiable step, in float64).
The expert selection (the per-axis top-k' and the product top-K) is piecewise
constant in the inputs: it passes no gradient, and is taken as fixed, as
every top-k router does.

Forward, per token t and selected task k (expert e = i * Nc + j):
    z_r = x Wr^T + row_bias,  z_c = x Wc^T + col_bias           [GS-NL §2.2]
    a = log_softmax(z_r),  b = log_softmax(z_c)                  [EXPL router]
    S_k = a[i_k] + b[j_k],  g = softmax_k(S)                     (gate reading)
    h_k = x_t . W[e],  y_t = sum_k g_k silu(h_k) V[e]            [GS-NL §2.1]

Backward, given dy = dL/dy:
    u_k = dy_t . V[e]
    dV[e]  += g_k silu(h_k) dy_t
    dg_k    = silu(h_k) u_k
    dh_k    = g_k silu'(h_k) u_k,     silu'(h) = s(h) (1 + h (1 - s(h))), s = logistic
    dW[e]  += dh_k x_t
    dx_t   += dh_k W[e]
    dS_k    = g_k (dg_k - sum_j g_j dg_j)                        (softmax backward)
    da[i_k] += dS_k,  db[j_k] += dS_k
    dz_r    = da - softmax(z_r) sum(da)                          (log-softmax backward)
    dx_t   += dz_r Wr + dz_c Wc
    dWr     = dz_r^T x,  dWc = dz_c^T x,  d row_bias = sum_t dz_r,  d col_bias = sum_t dz_c

Citation keys as in omni_oracle.
"""
from __future__ import annotations

import numpy as np

from oracle.omni_oracle import widen, silu


def silu_grad(h):
    """d/dh [h s(h)] = s(h) (1 + h (1 - s(h))), s the logistic function, float64."""
    h = np.asarray(h, dtype=np.float64)
    s = 1.0 / (1.0 + np.exp(-h))
    return s * (1.0 + h * (1.0 - s))


def executor_backward(x, w, v, expert_idx, gate, dy):
    """Gradients of y_t = sum_k g_tk silu(x_t . W[e_tk]) V[e_tk] (float64).

    [GS-NL §2.1] Dynamic Expert Assembly, differentiated term by term.
    Returns dict:
      dx [L, d]; dgate [L, K];
      active [n] (sorted unique experts), dw [n, d], dv [n, d] (rows of active);
    all float64.
    """
    expert_idx = np.asarray(expert_idx)
    gate = np.asarray(gate, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    L, K = expert_idx.shape
    xf = widen(x)
    d = xf.shape[1]
    active = np.unique(expert_idx)
    pos = {int(e): i for i, e in enumerate(active)}
    dw = np.zeros((len(active), d))
    dv = np.zeros((len(active), d))
    dx = np.zeros((L, d))
    dgate = np.zeros((L, K))
    for t in range(L):
        rows = expert_idx[t].astype(np.int64)
        Wt = widen(w[rows])                 # [K, d]
        Vt = widen(v[rows])
        h = Wt @ xf[t]
        u = Vt @ dy[t]
        s = silu(h)
        dgate[t] = s * u
        dh = gate[t] * silu_grad(h) * u
        dx[t] = dh @ Wt
        for k in range(K):
            i = pos[int(rows[k])]
            dv[i] += gate[t, k] * s[k] * dy[t]
            dw[i] += dh[k] * xf[t]
    return {"dx": dx, "dgate": dgate, "active": active, "dw": dw, "dv": dv}


def gate_backward(gate, dgate):
    """dS_k = g_k (dg_k - sum_j g_j dg_j): backward of g = softmax over the K
    selected joint scores (the gate reading), float64."""
    g = np.asarray(gate, dtype=np.float64)
    dg = np.asarray(dgate, dtype=np.float64)
    return g * (dg - (g * dg).sum(axis=-1, keepdims=True))


def score_backward(expert_idx, dscore, Nr, Nc):
    """da, db: S_k = a[i_k] + b[j_k] with e = i * Nc + j  [EXPL router]; the
    gradient of every selected score flows to its row and its column."""
    expert_idx = np.asarray(expert_idx).astype(np.int64)
    dS = np.asarray(dscore, dtype=np.float64)
    L = expert_idx.shape[0]
    da = np.zeros((L, Nr))
    db = np.zeros((L, Nc))
    for t in range(L):
        np.add.at(da[t], expert_idx[t] // Nc, dS[t])
        np.add.at(db[t], expert_idx[t] % Nc, dS[t])
    return da, db


def log_softmax_backward(z, dlogp):
    """dz = dlogp - softmax(z) * sum(dlogp), per row, float64."""
    z = np.asarray(z, dtype=np.float64)
    dl = np.asarray(dlogp, dtype=np.float64)
    p = np.exp(z - z.max(axis=-1, keepdims=True))
    p /= p.sum(axis=-1, keepdims=True)
    return dl - p * dl.sum(axis=-1, keepdims=True)


def router_backward(x, wr_t, wc_t, dzr, dzc):
    """Backward of z_r = x Wr^T + row_bias, z_c = x Wc^T + col_bias  [GS-NL §2.2].
    Returns dx [L, d], dwr [Nr, d], dwc [Nc, d], drb [Nr], dcb [Nc], float64."""
    xf = widen(x)
    dzr = np.asarray(dzr, dtype=np.float64)
    dzc = np.asarray(dzc, dtype=np.float64)
    dx = dzr @ widen(wr_t) + dzc @ widen(wc_t)
    return dx, dzr.T @ xf, dzc.T @ xf, dzr.sum(axis=0), dzc.sum(axis=0)


def backward(x, wr_t, wc_t, w, v, expert_idx, gate, dy, row_bias=None, col_bias=None):
    """Whole routed layer, backward, for a fixed selection (expert_idx, gate).

    gate must be the forward's gates (softmax of the selected scores); the
    router logits are recomputed from x, Wr, Wc and the biases.
    Returns dict: dx, dwr, dwc, drb, dcb, active, dw, dv, dgate, dscore,
    dzr, dzc (float64).
    """
    from oracle.omni_oracle import router_logits_f64
    Nr = np.asarray(wr_t).shape[0]
    Nc = np.asarray(wc_t).shape[0]
    ex = executor_backward(x, w, v, expert_idx, gate, dy)
    dS = gate_backward(gate, ex["dgate"])
    da, db = score_backward(expert_idx, dS, Nr, Nc)
    zr, zc = router_logits_f64(x, wr_t, wc_t, row_bias, col_bias)
    dzr = log_softmax_backward(zr, da)
    dzc = log_softmax_backward(zc, db)
    rdx, dwr, dwc, drb, dcb = router_backward(x, wr_t, wc_t, dzr, dzc)
    return {"dx": ex["dx"] + rdx, "dwr": dwr, "dwc": dwc, "drb": drb, "dcb": dcb,
            "active": ex["active"], "dw": ex["dw"], "dv": ex["dv"], "dgate": ex["dgate"],
            "dscore": dS, "dzr": dzr, "dzc": dzc}


def forward_fixed_f64(x, wr_t, wc_t, w, v, expert_idx, row_bias=None, col_bias=None):
    """The forward in float64 with the selection held fixed (for finite-difference
    checks of backward): y_t = sum_k softmax_k(S)_k silu(x_t . W[e]) V[e] with
    S_k = log_softmax(z_r)[i_k] + log_softmax(z_c)[j_k]."""
    from oracle.omni_oracle import log_softmax_rows
    xf = np.asarray(x, dtype=np.float64)
    Nc = np.asarray(wc_t).shape[0]
    zr = xf @ np.asarray(wr_t, dtype=np.float64).T
    zc = xf @ np.asarray(wc_t, dtype=np.float64).T
    if row_bias is not None:
        zr = zr + np.asarray(row_bias, dtype=np.float64)[None, :]
    if col_bias is not None:
        zc = zc + np.asarray(col_bias, dtype=np.float64)[None, :]
    a = log_softmax_rows(zr)
    b = log_softmax_rows(zc)
    idx = np.asarray(expert_idx).astype(np.int64)
    L, K = idx.shape
    S = np.take_along_axis(a, idx // Nc, axis=1) + np.take_along_axis(b, idx % Nc, axis=1)
    g = np.exp(S - S.max(axis=1, keepdims=True))
    g /= g.sum(axis=1, keepdims=True)
    w = np.asarray(w, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    y = np.zeros((L, xf.shape[1]))
    for t in range(L):
        h = w[idx[t]] @ xf[t]
        y[t] = (g[t] * silu(h)) @ v[idx[t]]
    return y, g
