"""CPU oracle for the OmniMoE routed atomic-expert layer (forward pass).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the GPU library.

This is a plain, slow, token-centric restatement of what the layer computes,
in float64 wherever arithmetic happens, rounded to float32 at each stage
boundary.  Every function names the passage it follows.  Citation keys:

  [GS-NL]  "OmniMoE: An Efficient MoE by Orchestrating Atomic Experts at Scale",
           gist.science explainer, Dutch edition, "Technisch Overzicht":
           §2.1 (core components), §2.2 (algorithmic innovations).
  [GS-ZH]  the same explainer, Chinese edition, "技术摘要" §2.1 / §2.2.
  [EXPL]   OmniMoE interactive explainer (omnimoeexpl, manus.space):
           sections "Atomic Expert / DEA", "Cartesian Product Router",
           "Expert-Centric Scheduling" and the ablation table.

Readings taken where the pages leave a step open (each is a choice):
  * sigma is SiLU, h * 1/(1+exp(-h)).  [GS-NL §2.1] writes a generic sigma
    and [EXPL, Atomic Expert] names SwiGLU, which needs two input projections
    a rank-1 expert does not have.  PARITY UNPINNED against the pages.
  * the joint score is log p_r[i] + log p_c[j] with per-axis log-softmax
    ([EXPL, Cartesian Product Router] prints the sum with the logarithm
    dropped while stating it is taken in log space).
  * expert id of grid cell (i, j) is e = i * Nc + j (row-major).
  * per-axis candidates k' (k' >= K); all orders break ties toward the
    lower index: rows by (a desc, i asc), columns by (b desc, j asc), cells by
    (S desc, e asc); values compare as float32 numbers (-0 == +0).
  * S = fl32(a[i] + b[j]), one float32 add, so the factored search and a
    brute-force search over all N cells agree except where float32 rounding
    collapses two different row (or column) values onto one sum.
  * gate = softmax over the K selected scores (the pages name a weight per
    (token, expert) pair but print no formula).
  * grouping: unique active experts sorted by id, B per group; the last
    group may be short.  Each group is then a contiguous id range, so the
    "contiguous ranges of expert ids" wording of [GS-NL §2.2] holds too.
  * task order: stable sort by (group, token); tasks of one token inside one
    group keep their flatten order k (score rank).
  * output y is the routed branch only, float32.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------- helpers


def widen(a) -> np.ndarray:
    """Exact float64 view of float32 data or bfloat16 bits (uint16)."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def silu(h):
    """sigma(h) = h / (1 + exp(-h)), float64 (the SiLU reading of sigma)."""
    h = np.asarray(h, dtype=np.float64)
    return h / (1.0 + np.exp(-h))


# ---------------------------------------------------------------- O1 + O2


def router_logp(x, wr_t, wc_t, row_bias=None, col_bias=None):
    """Row and column log-probabilities of the Cartesian Product Router.

    [GS-NL §2.2, Cartesian Product Router] and [EXPL, Cartesian Product
    Router]: two small projections give independent row and column logits
    over the Nr x Nc grid; each is normalised into a distribution, and the
    router works with their logarithms.

    z_r = x . Wr (+ row_bias), z_c = x . Wc (+ col_bias), then per-axis
    log-softmax, all in float64, rounded once to float32.

    x: [L, d]; wr_t: [Nr, d] (row i = the weights scoring grid row i, i.e.
    column i of Wr in the pages' d x sqrt(N) notation); wc_t: [Nc, d].
    Returns (a [L, Nr], b [L, Nc]) float32.
    """
    xf = widen(x)
    zr = xf @ widen(wr_t).T
    zc = xf @ widen(wc_t).T
    if row_bias is not None:
        zr = zr + widen(row_bias)[None, :]
    if col_bias is not None:
        zc = zc + widen(col_bias)[None, :]
    return log_softmax_rows(zr).astype(np.float32), log_softmax_rows(zc).astype(np.float32)


def router_logits(x, wr_t, wc_t, row_bias=None, col_bias=None):
    """Row and column router logits z_r [L, Nr], z_c [L, Nc], float64 -> float32.

    [GS-NL §2.2, Cartesian Product Router]: two small projections Wr, Wc give
    independent row and column logits.  z_r = x . Wr (+ row_bias).
    """
    zr, zc = router_logits_f64(x, wr_t, wc_t, row_bias, col_bias)
    return zr.astype(np.float32), zc.astype(np.float32)


def router_logits_f64(x, wr_t, wc_t, row_bias=None, col_bias=None):
    """The raw logits z_r, z_c of router_logp, in float64."""
    xf = widen(x)
    zr = xf @ widen(wr_t).T
    zc = xf @ widen(wc_t).T
    if row_bias is not None:
        zr = zr + widen(row_bias)[None, :]
    if col_bias is not None:
        zc = zc + widen(col_bias)[None, :]
    return zr, zc


def log_softmax_rows(z):
    """z - (m + ln sum exp(z - m)) per row, float64, m = row maximum."""
    z = np.asarray(z, dtype=np.float64)
    m = z.max(axis=-1, keepdims=True)
    return z - (m + np.log(np.exp(z - m).sum(axis=-1, keepdims=True)))


# ---------------------------------------------------------------- O3


def axis_topk(logp, k):
    """Per-axis search: the k best indices of each row of logp, rank-ordered.

    [EXPL, Cartesian Product Router]: rows and columns are searched
    separately, so routing costs O(sqrt N) per token instead of O(N).
    Order: value descending, lower index first on equal values (a stable
    sort of the negated values).  Returns (idx [L, k] int32, val [L, k] f32).
    """
    logp = np.asarray(logp, dtype=np.float32)
    order = np.argsort(-logp, axis=-1, kind="stable")[:, :k]
    val = np.take_along_axis(logp, order, axis=-1)
    return order.astype(np.int32), val


# ---------------------------------------------------------------- O4 + O5


def product_topk(a, b, kprime, K):
    """Top-K over the product grid from the per-axis candidates.

    [EXPL, Cartesian Product Router]: with p(i,j|x) ~ p_r(i|x) p_c(j|x) the
    joint score is additive in log space, S_ij = log p_r[i] + log p_c[j], and
    the N-entry score matrix is never formed.  Only the k' x k' cells built
    from the per-axis candidates are scored: S = fl32(a[R_r] + b[C_c]),
    e = R_r * Nc + C_c; the K best by (S desc, e asc) are kept in rank order.

    Returns (expert_idx [L,K] int32, score [L,K] f32, gate [L,K] f32,
    row_sel [L,k'] int32, col_sel [L,k'] int32).
    """
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    L, Nc = b.shape
    R, av = axis_topk(a, kprime)
    C, bv = axis_topk(b, kprime)
    S = (av[:, :, None] + bv[:, None, :]).reshape(L, -1)            # float32 adds
    E = (R.astype(np.int64)[:, :, None] * Nc + C[:, None, :]).reshape(L, -1)
    order = np.lexsort((E, -S), axis=-1)[:, :K]                      # S desc, e asc
    idx = np.take_along_axis(E, order, axis=-1).astype(np.int32)
    score = np.take_along_axis(S, order, axis=-1)
    return idx, score, gates(score), R, C


def brute_force_topk(a, b, K):
    """Top-K over all N = Nr * Nc cells with the same comparator (tiny N only).

    The factored search of product_topk must return the same list whenever
    k' >= K, apart from the float32 collapse case named in the header.
    """
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    L, Nr = a.shape
    Nc = b.shape[1]
    S = (a[:, :, None] + b[:, None, :]).reshape(L, Nr * Nc)
    E = np.broadcast_to(np.arange(Nr * Nc, dtype=np.int64), (L, Nr * Nc))
    order = np.lexsort((E, -S), axis=-1)[:, :K]
    return order.astype(np.int32), np.take_along_axis(S, order, axis=-1)


def gates(score):
    """g_k = exp(S_k - S_0) / sum_j exp(S_j - S_0), float64 -> float32.

    The pages attach a weight to every (token, expert) task ([EXPL,
    Expert-Centric Scheduling]) without a formula; the reading is a softmax
    over the K selected joint scores.  S_0 is the largest (lists are in rank
    order).
    """
    s = np.asarray(score, dtype=np.float64)
    ex = np.exp(s - s[:, :1])
    return (ex / ex.sum(axis=-1, keepdims=True)).astype(np.float32)


# ---------------------------------------------------------------- O6 - O9


def max_groups(N, L, K, B, grouping="active"):
    """Upper bound on the number of groups: ceil(min(N, L*K) / B) when the
    active experts are cut B at a time; ceil(N / B) id windows otherwise."""
    if grouping == "window":
        return -(-N // B)
    return -(-min(N, L * K) // B)


def build_schedule(expert_idx, gate, N, B, grouping="active"):
    """Expert-Centric Scheduling of the L*K routing decisions.

    [EXPL, Expert-Centric Scheduling] and [GS-NL §2.2]:
      1. task collection: flatten every (token, expert, weight) decision into
         M = L * K tasks, task m = t * K + k;
      2. collect the unique active experts, sort them by id, cut them into
         groups of B (the last one may be short);
      3. order the tasks by group id first and token id second (stable, so a
         token's tasks inside one group keep their rank order k);
      4. each group's parameters are then loaded once and reused for all of
         its tokens (the executor's business; here only the CSR offsets).
    grouping="window" is the fixed-window variant: group g holds the experts
    with ids in [g B, (g + 1) B) ([GS-NL §2.2] groups tasks by contiguous
    ranges of expert ids); every window is a group, empty or not, so
    n_groups = ceil(N / B).
    Returns a dict of numpy arrays; group_offsets has max_groups + 1 entries
    and every entry past n_groups equals M.
    """
    expert_idx = np.asarray(expert_idx, dtype=np.int64)
    gate = np.asarray(gate, dtype=np.float32)
    L, K = expert_idx.shape
    M = L * K
    task_token = np.repeat(np.arange(L, dtype=np.int64), K)
    task_expert = expert_idx.reshape(-1)
    task_gate = gate.reshape(-1)

    active = np.unique(task_expert)                     # sorted ascending
    n_active = int(active.size)
    if grouping == "window":
        n_groups = -(-N // B)
        group = task_expert // B                        # the id window
    else:
        n_groups = -(-n_active // B)
        rank = np.searchsorted(active, task_expert)     # position in active list
        group = rank // B

    order = np.lexsort((task_token, group))             # group, then token; stable
    G = max_groups(N, L, K, B, grouping)
    sizes = np.bincount(group, minlength=G)[:G] if M else np.zeros(G, np.int64)
    offsets = np.zeros(G + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(sizes)
    return {
        "n_active": n_active,
        "n_groups": n_groups,
        "active": active.astype(np.int32),
        "group_offsets": offsets.astype(np.int32),
        "task_index": order.astype(np.int32),
        "task_token": task_token[order].astype(np.int32),
        "task_expert": task_expert[order].astype(np.int32),
        "task_gate": task_gate[order],
        "task_group": group[order].astype(np.int32),
    }


def traffic_elements(d, L, K, n_active):
    """Parameter traffic of the two execution orders, in elements.

    [EXPL, Expert-Centric Scheduling]: token-centric execution loads 2d
    values per task, D = 2d*L*K; expert-centric execution loads each active
    expert's two rows once, D = 2d*|E_active|.
    """
    return {"token_centric": 2 * d * L * K, "expert_centric": 2 * d * n_active}


def router_cost_ratio(Nr, Nc):
    """Router projection cost relative to a flat d x N router: (Nr + Nc) / N.

    [EXPL, Cartesian Product Router] quotes 1.56 % at N = 16K.
    """
    return (Nr + Nc) / (Nr * Nc)


# ---------------------------------------------------------------- O10


def atomic_forward(x, w, v, expert_idx, gate, tokens=None):
    """Token-centric Dynamic Expert Assembly, float64 -> float32.

    [GS-NL §2.1] atomic expert E_i(x) = sigma(x . w_in) w_out with w_in,
    w_out rows of the global matrices W, V; for every token the selected rows
    are fetched and assembled into one token-specific block:
        y_t = sum_k g_tk * sigma(x_t . W[e_tk]) * V[e_tk].
    tokens: optional subset of token ids (y rows for those only).
    Returns y [len(tokens) or L, d] float32.
    """
    return atomic_forward_f64(x, w, v, expert_idx, gate, tokens).astype(np.float32)


def atomic_forward_literal(x, w, v, expert_idx, gate):
    """The same sum written as one scalar loop per (token, k), float64."""
    expert_idx = np.asarray(expert_idx)
    L, K = expert_idx.shape
    y = np.zeros((L, np.asarray(x).shape[1]), dtype=np.float64)
    for t in range(L):
        xt = widen(x[t])
        for k in range(K):
            e = int(expert_idx[t, k])
            h = 0.0
            wt = widen(w[e])
            for c in range(xt.size):
                h += xt[c] * wt[c]
            y[t] += float(gate[t, k]) * float(silu(h)) * widen(v[e])
    return y


def atomic_forward_f64(x, w, v, expert_idx, gate, tokens=None):
    """atomic_forward without the final float32 rounding (self-checks)."""
    expert_idx = np.asarray(expert_idx)
    gate = np.asarray(gate, dtype=np.float32)
    L = expert_idx.shape[0]
    toks = np.arange(L) if tokens is None else np.asarray(tokens)
    y = np.zeros((len(toks), np.asarray(x).shape[1]), dtype=np.float64)
    for n, t in enumerate(toks):
        xt = widen(x[t])
        rows = expert_idx[t].astype(np.int64)
        h = widen(w[rows]) @ xt
        y[n] = (gate[t].astype(np.float64) * silu(h)) @ widen(v[rows])
    return y


def atomic_forward_expert_centric(x, w, v, sched, L, count_loads=False):
    """Expert-centric execution of a schedule, float64.

    [EXPL, Expert-Centric Scheduling]: walk the groups; load each group's
    active experts' W and V rows once, then serve every task of the group in
    (token) order from the loaded block.  The ablation table of [EXPL] shows
    removing this scheduling leaves model quality unchanged: it computes the
    same function as atomic_forward (up to float64 summation order).
    Returns y [L, d] float64 (and the number of parameter elements loaded).
    """
    d = np.asarray(x).shape[1]
    y = np.zeros((L, d), dtype=np.float64)
    offs = sched["group_offsets"]
    loaded = 0
    for g in range(sched["n_groups"]):
        lo, hi = int(offs[g]), int(offs[g + 1])
        experts = np.unique(sched["task_expert"][lo:hi])
        block_w = {int(e): widen(w[e]) for e in experts}      # loaded once
        block_v = {int(e): widen(v[e]) for e in experts}
        loaded += 2 * d * len(experts)
        for m in range(lo, hi):
            t = int(sched["task_token"][m])
            e = int(sched["task_expert"][m])
            h = float(widen(x[t]) @ block_w[e])
            y[t] += float(sched["task_gate"][m]) * float(silu(h)) * block_v[e]
    return (y, loaded) if count_loads else y


# ---------------------------------------------------------------- pipeline


def forward(x, wr_t, wc_t, w, v, kprime, K, B, row_bias=None, col_bias=None):
    """Whole routed layer: router -> product top-K + gates -> schedule -> y."""
    a, b = router_logp(x, wr_t, wc_t, row_bias, col_bias)
    idx, score, gate, R, C = product_topk(a, b, kprime, K)
    N = np.asarray(wr_t).shape[0] * np.asarray(wc_t).shape[0]
    sched = build_schedule(idx, gate, N, B)
    y = atomic_forward(x, w, v, idx, gate)
    return {"a": a, "b": b, "expert_idx": idx, "score": score, "gate": gate,
            "row_sel": R, "col_sel": C, "schedule": sched, "y": y}
