"""Thin Python binding of libomni.so (ctypes).

Argument marshalling only: every step of the layer runs in the library's
HIP kernels.  PyTorch supplies device memory and the current stream.  If the
library is missing the import fails; there is no other execution path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("OMNI_LIB", os.path.join(_HERE, "libomni.so"))

OMNI_OK, OMNI_ERR_INVALID_ARG, OMNI_ERR_WORKSPACE, OMNI_ERR_UNSUPPORTED, OMNI_ERR_HIP = range(5)
OMNI_F32, OMNI_BF16 = 0, 1
EXEC_MODES = {"auto": 0, "expert": 1, "token": 2, "grouped": 3}  # omni_exec_mode
GROUPINGS = {"active": 0, "window": 1}             # omni_grouping
ABI_VERSION = 14

# Every symbol the header declares (checked by the CPU test suite).
EXPORTS = (
    "omni_abi_version", "omni_status_string", "omni_router_logits_workspace",
    "omni_router_logits",
    "omni_product_topk_workspace", "omni_product_topk", "omni_schedule_max_groups",
    "omni_schedule_workspace", "omni_schedule_tasks", "omni_atomic_forward_mode",
    "omni_atomic_forward_workspace", "omni_atomic_forward", "omni_routed_backward_workspace",
    "omni_routed_backward", "omni_shared_mlp_workspace", "omni_shared_mlp",
    "omni_atomic_forward_glu", "omni_flat_router_workspace", "omni_flat_router_topk",
    "omni_product_topk_static",
)


class OmniError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__(f"{fn} failed: {msg} (status {code})")
        self.code = code


class ScheduleStruct(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("counts", "active", "group_offsets", "task_token", "task_expert",
                 "task_gate", "task_index", "flat_expert", "flat_gate")]


_vp, _i, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
_SIGS = {
    "omni_abi_version": (_i, []),
    "omni_status_string": (ctypes.c_char_p, [_i]),
    "omni_router_logits_workspace": (_sz, [_i, _i, _i, _i, _i]),
    "omni_router_logits": (_i, [_i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                _vp]),
    "omni_product_topk_workspace": (_sz, [_i, _i, _i, _i, _i]),
    "omni_product_topk": (_i, [_i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                               _vp, _vp, _sz, _vp]),
    "omni_product_topk_static": (_i, [_i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                      _vp, _vp, _vp]),
    "omni_schedule_max_groups": (_i, [_i, _i, _i, _i, _i]),
    "omni_schedule_workspace": (_sz, [_i, _i, _i, _i, _i]),
    "omni_schedule_tasks": (_i, [_i, _i, _i, _i, _i, _vp, _vp, ctypes.POINTER(ScheduleStruct),
                                 _vp, _sz, _vp]),
    "omni_atomic_forward_mode": (_i, [_i, _i, _i, _i, _i, _i]),
    "omni_atomic_forward_workspace": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "omni_atomic_forward": (_i, [_i, _i, _i, _i, _i, _i, _vp, _vp, _vp,
                                 ctypes.POINTER(ScheduleStruct), _vp, _i, _i, _vp, _sz, _vp]),
    "omni_routed_backward_workspace": (_sz, [_i, _i, _i, _i, _i, _i]),
    "omni_routed_backward": (_i, [_i, _i, _i, _i, _i, _i] + [_vp] * 19 + [_sz, _vp]),
    "omni_shared_mlp_workspace": (_sz, [_i, _i, _i, _i]),
    "omni_flat_router_workspace": (_sz, [_i, _i, _i]),
    "omni_flat_router_topk": (_i, [_i, _i, _i, _i, _i] + [_vp] * 8 + [_sz, _vp]),
    "omni_atomic_forward_glu": (_i, [_i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp,
                                     ctypes.POINTER(ScheduleStruct), _vp, _i, _vp, _sz, _vp]),
    "omni_shared_mlp": (_i, [_i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _i, _vp, _sz, _vp]),
}

_lib = None


def lib():
    """Load libomni.so once (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} not found: build it with "
                              f"`python -m cartesian_routed_atomic_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        if h.omni_abi_version() != ABI_VERSION:
            raise ImportError(f"{LIB_PATH} has ABI {h.omni_abi_version()}, this binding "
                              f"expects {ABI_VERSION}: rebuild the library")
        _lib = h
    return _lib


def _check(fn, code):
    if code != OMNI_OK:
        msg = lib().omni_status_string(code).decode()
        raise OmniError(fn, code, msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return OMNI_BF16
    if t.dtype == torch.float32:
        return OMNI_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _req(t, name, dtype=None, shape=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


# ------------------------------------------------------------------ calls


def router_logits(x, wr_t, wc_t, row_bias=None, col_bias=None, row_logits=None,
                  col_logits=None, workspace=None, stream=None):
    """omni_router_logits: returns (row_logits [L,Nr], col_logits [L,Nc]) float32."""
    L, d = x.shape
    Nr, Nc = wr_t.shape[0], wc_t.shape[0]
    _req(x, "x")
    _req(wr_t, "wr_t", x.dtype, (Nr, d))
    _req(wc_t, "wc_t", x.dtype, (Nc, d))
    for b, n, nm in ((row_bias, Nr, "row_bias"), (col_bias, Nc, "col_bias")):
        if b is not None:
            _req(b, nm, torch.float32, (n,))
    if row_logits is None:
        row_logits = torch.empty((L, Nr), dtype=torch.float32, device=x.device)
    if col_logits is None:
        col_logits = torch.empty((L, Nc), dtype=torch.float32, device=x.device)
    _req(row_logits, "row_logits", torch.float32, (L, Nr))
    _req(col_logits, "col_logits", torch.float32, (L, Nc))
    nws = lib().omni_router_logits_workspace(_dtype_code(x), L, d, Nr, Nc)
    ws = workspace
    if nws and (ws is None or ws.numel() < nws):
        ws = torch.empty(nws, dtype=torch.uint8, device=x.device)
    _check("omni_router_logits", lib().omni_router_logits(
        _dtype_code(x), L, d, Nr, Nc, _ptr(x), _ptr(wr_t), _ptr(wc_t), _ptr(row_bias),
        _ptr(col_bias), _ptr(row_logits), _ptr(col_logits), _ptr(ws) if nws else None, nws,
        _stream(stream)))
    return row_logits, col_logits


def product_topk(row_logits, col_logits, kprime, K, want_sel=True, want_logp=True, out=None,
                 stream=None):
    """omni_product_topk: returns dict expert_idx, score, gate, row_logp, col_logp,
    row_sel, col_sel (the last four None unless asked for)."""
    L, Nr = row_logits.shape
    Nc = col_logits.shape[1]
    _req(row_logits, "row_logits", torch.float32)
    _req(col_logits, "col_logits", torch.float32, (L, Nc))
    dev = row_logits.device
    o = dict(out or {})

    def get(name, shape, dtype):
        t = o.get(name)
        if t is None:
            t = torch.empty(shape, dtype=dtype, device=dev)
        _req(t, name, dtype, shape)
        return t
    idx = get("expert_idx", (L, K), torch.int32)
    score = get("score", (L, K), torch.float32)
    gate = get("gate", (L, K), torch.float32)
    rlp = get("row_logp", (L, Nr), torch.float32) if want_logp else None
    clp = get("col_logp", (L, Nc), torch.float32) if want_logp else None
    rsel = get("row_sel", (L, kprime), torch.int32) if want_sel else None
    csel = get("col_sel", (L, kprime), torch.int32) if want_sel else None
    nws = lib().omni_product_topk_workspace(L, Nr, Nc, kprime, K)
    ws = o.get("workspace")
    if nws and (ws is None or ws.numel() < nws):
        ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    _check("omni_product_topk", lib().omni_product_topk(
        L, Nr, Nc, kprime, K, _ptr(row_logits), _ptr(col_logits), _ptr(idx), _ptr(score),
        _ptr(gate), _ptr(rlp), _ptr(clp), _ptr(rsel), _ptr(csel), _ptr(ws),
        nws if ws is not None else 0, _stream(stream)))
    return {"expert_idx": idx, "score": score, "gate": gate, "row_logp": rlp, "col_logp": clp,
            "row_sel": rsel, "col_sel": csel, "workspace": ws}


@dataclass
class Schedule:
    L: int
    K: int
    N: int
    B: int
    grouping: str
    counts: torch.Tensor
    active: torch.Tensor
    group_offsets: torch.Tensor
    task_token: torch.Tensor
    task_expert: torch.Tensor
    task_gate: torch.Tensor
    task_index: torch.Tensor | None
    workspace: torch.Tensor | None
    # the selection the tasks were built from, in flatten order (set by
    # schedule_tasks; the token-centric executor reads the token lists from
    # it; None makes that executor invert the sorted order instead)
    flat_expert: torch.Tensor | None = None
    flat_gate: torch.Tensor | None = None

    def struct(self):
        return ScheduleStruct(*(None if t is None else t.data_ptr() for t in (
            self.counts, self.active, self.group_offsets, self.task_token, self.task_expert,
            self.task_gate, self.task_index, self.flat_expert, self.flat_gate)))


def _grouping(grouping):
    if grouping not in GROUPINGS:
        raise ValueError(f"grouping must be one of {sorted(GROUPINGS)}, got {grouping!r}")
    return GROUPINGS[grouping]


def max_groups(L, K, N, B, grouping="active"):
    return lib().omni_schedule_max_groups(L, K, N, B, _grouping(grouping))


def alloc_schedule(L, K, N, B, device, with_index=True, grouping="active"):
    """Device buffers for a schedule of L*K tasks (and its workspace).
    grouping: "active" (B active experts per group) or "window" (id windows)."""
    M = L * K
    G = max_groups(L, K, N, B, grouping)
    nws = lib().omni_schedule_workspace(L, K, N, B, _grouping(grouping))
    i32 = dict(dtype=torch.int32, device=device)
    return Schedule(L, K, N, B, grouping,
                    counts=torch.zeros(2, **i32),
                    active=torch.empty(max(1, min(N, M)), **i32),
                    group_offsets=torch.empty(G + 1, **i32),
                    task_token=torch.empty(max(1, M), **i32),
                    task_expert=torch.empty(max(1, M), **i32),
                    task_gate=torch.empty(max(1, M), dtype=torch.float32, device=device),
                    task_index=torch.empty(max(1, M), **i32) if with_index else None,
                    workspace=torch.empty(max(1, nws), dtype=torch.uint8, device=device))


def schedule_tasks(expert_idx, gate, N, B, sched=None, stream=None, grouping="active"):
    """omni_schedule_tasks: returns a Schedule of device tensors."""
    L, K = expert_idx.shape
    _req(expert_idx, "expert_idx", torch.int32)
    _req(gate, "gate", torch.float32, (L, K))
    if sched is None:
        sched = alloc_schedule(L, K, N, B, expert_idx.device, grouping=grouping)
    elif sched.grouping != grouping:
        raise ValueError(f"schedule buffers were sized for grouping {sched.grouping!r}")
    st = sched.struct()
    ws = sched.workspace
    _check("omni_schedule_tasks", lib().omni_schedule_tasks(
        L, K, N, B, _grouping(grouping), _ptr(expert_idx), _ptr(gate), ctypes.byref(st), _ptr(ws),
        ws.numel() if ws is not None else 0, _stream(stream)))
    sched.flat_expert, sched.flat_gate = expert_idx, gate
    return sched


def _same_shape_schedule(sched, L, N):
    # the kernels index x, W, V with the schedule's token and expert ids
    if sched.L != L or sched.N != N:
        raise ValueError(f"the schedule was built for L={sched.L}, N={sched.N}; "
                         f"x and the expert matrices give L={L}, N={N}")
    if sched.task_index is None:
        raise ValueError("the schedule must carry task_index")


def _exec_mode(mode):
    if mode not in EXEC_MODES:
        raise ValueError(f"mode must be one of {sorted(EXEC_MODES)}, got {mode!r}")
    return EXEC_MODES[mode]


def atomic_forward_mode(dtype, L, d, N, K, B):
    """omni_atomic_forward_mode: the form mode="auto" runs ("expert" / "token" / "grouped")."""
    code = torch.bfloat16 if dtype == torch.bfloat16 else torch.float32
    m = lib().omni_atomic_forward_mode(OMNI_BF16 if code == torch.bfloat16 else OMNI_F32,
                                       L, d, N, K, B)
    if m == 0:
        raise ValueError("invalid shape for omni_atomic_forward_mode")
    return {1: "expert", 2: "token", 3: "grouped"}[m]


def atomic_forward(x, w, v, sched, y=None, accumulate=False, workspace=None, stream=None,
                   mode="auto"):
    """omni_atomic_forward: returns y [L, d] float32 (y += routed if accumulate).
    mode: "auto", "expert" (expert-centric), "token" (token-centric) or "grouped"
    (per token tile, the most shared experts as two MFMA products and the rest
    per task; bf16 only)."""
    L, d = x.shape
    N = w.shape[0]
    _req(x, "x")
    _req(w, "w", x.dtype, (N, d))
    _req(v, "v", x.dtype, (N, d))
    _same_shape_schedule(sched, L, N)
    code = _exec_mode(mode)
    if y is None:
        y = torch.empty((L, d), dtype=torch.float32, device=x.device)
    _req(y, "y", torch.float32, (L, d))
    st = sched.struct()
    nws = lib().omni_atomic_forward_workspace(_dtype_code(x), L, d, N, sched.K, sched.B, code)
    ws = workspace
    if nws and (ws is None or ws.numel() < nws):
        ws = torch.empty(nws, dtype=torch.uint8, device=x.device)
    _check("omni_atomic_forward", lib().omni_atomic_forward(
        _dtype_code(x), L, d, N, sched.K, sched.B, _ptr(x), _ptr(w), _ptr(v),
        ctypes.byref(st), _ptr(y), int(bool(accumulate)), code, _ptr(ws),
        nws if ws is not None else 0, _stream(stream)))
    return y


def atomic_forward_glu(x, w, u, v, sched, y=None, accumulate=False, workspace=None,
                       stream=None):
    """omni_atomic_forward_glu (SwiGLU-gated experts): returns y [L, d] float32,
    y_t = sum_k g silu(x_t . W[e]) (x_t . U[e]) V[e] (y += that if accumulate)."""
    L, d = x.shape
    N = w.shape[0]
    _req(x, "x")
    for name, t in (("w", w), ("u", u), ("v", v)):
        _req(t, name, x.dtype, (N, d))
    _same_shape_schedule(sched, L, N)
    if y is None:
        y = torch.empty((L, d), dtype=torch.float32, device=x.device)
    _req(y, "y", torch.float32, (L, d))
    st = sched.struct()
    nws = lib().omni_atomic_forward_workspace(_dtype_code(x), L, d, N, sched.K, sched.B,
                                              EXEC_MODES["token"])
    ws = workspace
    if nws and (ws is None or ws.numel() < nws):
        ws = torch.empty(nws, dtype=torch.uint8, device=x.device)
    _check("omni_atomic_forward_glu", lib().omni_atomic_forward_glu(
        _dtype_code(x), L, d, N, sched.K, sched.B, _ptr(x), _ptr(w), _ptr(u), _ptr(v),
        ctypes.byref(st), _ptr(y), int(bool(accumulate)), _ptr(ws),
        nws if ws is not None else 0, _stream(stream)))
    return y


def flat_router_topk(x, wf, K, bias=None, want_logp=False, out=None, workspace=None,
                     stream=None):
    """omni_flat_router_topk (the d x N router baseline): returns dict expert_idx,
    score, gate [L, K] and logp [L, N] (None unless want_logp), workspace."""
    L, d = x.shape
    N = wf.shape[0]
    _req(x, "x")
    _req(wf, "wf", x.dtype, (N, d))
    if bias is not None:
        _req(bias, "bias", torch.float32, (N,))
    o = dict(out or {})
    dev = x.device
    r = {"expert_idx": o.get("expert_idx"), "score": o.get("score"), "gate": o.get("gate")}
    for name, dt in (("expert_idx", torch.int32), ("score", torch.float32),
                     ("gate", torch.float32)):
        if r[name] is None:
            r[name] = torch.empty((L, K), dtype=dt, device=dev)
        _req(r[name], name, dt, (L, K))
    r["logp"] = torch.empty((L, N), dtype=torch.float32, device=dev) if want_logp else None
    code = _dtype_code(x)
    nws = lib().omni_flat_router_workspace(code, L, N)
    ws = workspace
    if ws is None or ws.numel() < nws:
        ws = torch.empty(max(1, nws), dtype=torch.uint8, device=dev)
    _check("omni_flat_router_topk", lib().omni_flat_router_topk(
        code, L, d, N, K, _ptr(x), _ptr(wf), _ptr(bias), _ptr(r["expert_idx"]),
        _ptr(r["score"]), _ptr(r["gate"]), _ptr(r["logp"]), _ptr(ws), nws, _stream(stream)))
    r["workspace"] = ws
    return r


def forward(x, wr_t, wc_t, w, v, kprime, K, B, row_bias=None, col_bias=None, stream=None,
            mode="auto"):
    """The four calls back to back on one stream; returns every intermediate."""
    zr, zc = router_logits(x, wr_t, wc_t, row_bias, col_bias, stream=stream)
    sel = product_topk(zr, zc, kprime, K, stream=stream)
    N = wr_t.shape[0] * wc_t.shape[0]
    sched = schedule_tasks(sel["expert_idx"], sel["gate"], N, B, stream=stream)
    y = atomic_forward(x, w, v, sched, stream=stream, mode=mode)
    return {"row_logits": zr, "col_logits": zc, **sel, "schedule": sched, "y": y}


def shared_mlp(x, w_gate, w_up, w_down, y=None, accumulate=False, workspace=None, stream=None):
    """omni_shared_mlp: y [L, d] float32 = (or +=, if accumulate) the shared dense
    MLP branch Wd (silu(Wg x) * (Wu x)); w_gate, w_up [d_ff, d], w_down [d, d_ff]."""
    L, d = x.shape
    d_ff = w_gate.shape[0]
    _req(x, "x")
    _req(w_gate, "w_gate", x.dtype, (d_ff, d))
    _req(w_up, "w_up", x.dtype, (d_ff, d))
    _req(w_down, "w_down", x.dtype, (d, d_ff))
    if y is None:
        y = torch.empty((L, d), dtype=torch.float32, device=x.device)
    _req(y, "y", torch.float32, (L, d))
    code = _dtype_code(x)
    nws = lib().omni_shared_mlp_workspace(code, L, d, d_ff)
    ws = workspace
    if ws is None or ws.numel() < nws:
        ws = torch.empty(max(1, nws), dtype=torch.uint8, device=x.device)
    _check("omni_shared_mlp", lib().omni_shared_mlp(
        code, L, d, d_ff, _ptr(x), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(y),
        int(bool(accumulate)), _ptr(ws), nws, _stream(stream)))
    return y


def layer_forward(x, wr_t, wc_t, w, v, w_gate, w_up, w_down, kprime, K, B, row_bias=None,
                  col_bias=None, stream=None, mode="auto"):
    """The whole OmniMoE layer on one stream: the shared dense MLP writes y, then
    the routed branch (router, product top-K, schedule) runs and its executor
    adds the routed output onto y.  Returns every intermediate of the routed
    branch and y."""
    y = shared_mlp(x, w_gate, w_up, w_down, stream=stream)
    zr, zc = router_logits(x, wr_t, wc_t, row_bias, col_bias, stream=stream)
    sel = product_topk(zr, zc, kprime, K, stream=stream)
    N = wr_t.shape[0] * wc_t.shape[0]
    sched = schedule_tasks(sel["expert_idx"], sel["gate"], N, B, stream=stream)
    atomic_forward(x, w, v, sched, y=y, accumulate=True, stream=stream, mode=mode)
    return {"row_logits": zr, "col_logits": zc, **sel, "schedule": sched, "y": y}


def routed_backward(x, wr_t, wc_t, w, v, expert_idx, gate, dy, out=None, workspace=None,
                    stream=None):
    """omni_routed_backward: gradients of the routed layer for upstream dy [L, d] float32.

    Returns dict dx [L, d], dwr [Nr, d], dwc [Nc, d], drb [Nr], dcb [Nc],
    counts [2], active [min(N, L*K)], dw, dv [min(N, L*K), d] (row r is the
    gradient of expert active[r], r < counts[0]), dgate [L, K]; all float32
    except counts / active (int32)."""
    L, d = x.shape
    Nr, Nc = wr_t.shape[0], wc_t.shape[0]
    N = Nr * Nc
    K = expert_idx.shape[1]
    _req(x, "x")
    for name, t in (("wr_t", wr_t), ("wc_t", wc_t)):
        _req(t, name, x.dtype)
    _req(w, "w", x.dtype, (N, d))
    _req(v, "v", x.dtype, (N, d))
    _req(expert_idx, "expert_idx", torch.int32, (L, K))
    _req(gate, "gate", torch.float32, (L, K))
    _req(dy, "dy", torch.float32, (L, d))
    dev = x.device
    o = dict(out or {})
    na = max(1, min(N, L * K))

    def get(name, shape, dtype):
        t = o.get(name)
        if t is None:
            t = torch.empty(shape, dtype=dtype, device=dev)
        _req(t, name, dtype, shape)
        return t
    r = {"dx": get("dx", (L, d), torch.float32), "dwr": get("dwr", (Nr, d), torch.float32),
         "dwc": get("dwc", (Nc, d), torch.float32), "drb": get("drb", (Nr,), torch.float32),
         "dcb": get("dcb", (Nc,), torch.float32), "counts": get("counts", (2,), torch.int32),
         "active": get("active", (na,), torch.int32),
         "dw": get("dw", (na, d), torch.float32), "dv": get("dv", (na, d), torch.float32),
         "dgate": get("dgate", (L, K), torch.float32)}
    code = _dtype_code(x)
    nws = lib().omni_routed_backward_workspace(code, L, d, Nr, Nc, K)
    ws = workspace
    if ws is None or ws.numel() < nws:
        ws = torch.empty(max(1, nws), dtype=torch.uint8, device=dev)
    _check("omni_routed_backward", lib().omni_routed_backward(
        code, L, d, Nr, Nc, K, _ptr(x), _ptr(wr_t), _ptr(wc_t), _ptr(w), _ptr(v),
        _ptr(expert_idx), _ptr(gate), _ptr(dy), _ptr(r["dx"]), _ptr(r["dwr"]), _ptr(r["dwc"]),
        _ptr(r["drb"]), _ptr(r["dcb"]), _ptr(r["counts"]), _ptr(r["active"]), _ptr(r["dw"]),
        _ptr(r["dv"]), _ptr(r["dgate"]), _ptr(ws), nws, _stream(stream)))
    r["workspace"] = ws
    return r
