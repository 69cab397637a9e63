#!/usr/bin/env python3
"""Routed tokens/s of one OmniMoE routed atomic-expert layer (forward) on one
MI355X, with the executor's HBM roofline fraction and the CPU oracle's rate.

A step is one pass of the whole path on one batch: router logits ->
product top-K + gates -> expert-centric schedule -> execution of the schedule
(in the form the library's auto mode picks for the shape; the other form is
timed beside it), all four C-ABI calls enqueued back to back on one stream,
inputs resident in HBM, every output buffer allocated before timing.  The
same four calls captured once into a HIP graph are timed beside it
(graph_ms_per_step; --no-graph skips that).

    python bench.py [--steps 50] [--warmup 5] [--workload large]

Prints one JSON line on stdout (progress goes to stderr).
"""
import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed tokens/sec per atomic-expert layer at 1 GPU; % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak
FP32_TFLOPS = 157.3            # MI355X float32 vector peak
CSRC = os.path.join(ROOT, "cartesian_routed_atomic_amd", "csrc")
EXEC_SRCS = {  # the sources each executor form's kernels are built from
    "expert": ("execute.hip", "rowfrag.hpp", "device.hpp"),
    "token": ("execute.hip", "rowfrag.hpp", "device.hpp"),
    "grouped": ("grouped.hip", "rowfrag.hpp", "device.hpp"),
}
TRAFFIC_GLOB = os.path.join(ROOT, "profiles", "atomic_forward_*_traffic.md")
EXEC_KERNELS = {  # what one omni_atomic_forward call launches, per form
    "expert": "omni_atomic_forward, expert-centric: coef_kernel + gather_kernel",
    "token": "omni_atomic_forward, token-centric: one kernel (token_multi_kernel from 8192 "
             "tokens, four tokens per wave; token lists read from the flattened selection the "
             "schedule carries)",
    "grouped": "omni_atomic_forward, grouped: gf_zero, gf_count, gf_level, gf_select (the hot "
               "set from the sorted schedule), gf_pack (W_H, V_H^T in fragment order), "
               "gf_cold_kernel (tasks outside the hot set, token by token; writes y), "
               "gf_tile_kernel (per token tile the hot experts as two MFMA products, y += )",
}


def say(msg):
    print(msg, file=sys.stderr, flush=True)


def exec_src_hash(form):
    """Fingerprint of one executor form's kernel sources (a counter record
    taken on other sources no longer describes the kernel)."""
    h = hashlib.sha256()
    for f in EXEC_SRCS[form]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, form):
    """Counter-derived HBM bytes per executor call, if taken on this kernel
    (records in the profiles/atomic_forward_*_traffic.md summaries)."""
    if form not in EXEC_SRCS:
        return None
    for path in sorted(glob.glob(TRAFFIC_GLOB)):
        for m in re.finditer(r"traffic_record:\s*(\{.*\})", open(path).read()):
            rec = json.loads(m.group(1))
            if (rec.get("workload") == workload and rec.get("form") == form
                    and rec.get("executor_src_sha256_16") == exec_src_hash(form)):
                return rec.get("bytes_per_launch")
    return None


_ORACLE_INPUTS = {}  # the workload, for the forked oracle workers (inherited at fork)


def _one_blas_thread():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover
        pass


def _oracle_tokens(span):
    """The oracle's per-token part of the path on tokens [lo, hi): router
    log-probabilities, product top-K + gates, token-centric y."""
    from oracle import omni_oracle as O
    lo, hi = span
    inp, wl = _ORACLE_INPUTS["inp"], _ORACLE_INPUTS["wl"]
    xs = inp["x"][lo:hi]
    a, b = O.router_logp(xs, inp["wr"], inp["wc"], inp["row_bias"], inp["col_bias"])
    idx, _, gate, _, _ = O.product_topk(a, b, wl.kprime, wl.K)
    O.atomic_forward(xs, inp["w"], inp["v"], idx, gate)
    return idx, gate


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def cpu_baseline(inp, wl, target_s):
    """The oracle, untuned, over the host's cores: tokens split into chunks
    over one worker process per core (one BLAS thread each), then the
    schedule over the whole selection in the parent (one global sort).  The
    workers are forked before this process touches the GPU."""
    import multiprocessing as mp

    import numpy as np
    from oracle import omni_oracle as O
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    cores = max(1, min(int(avail or 1), 16))  # a one-GPU machine's share is 16 cores
    _ORACLE_INPUTS.update(inp=inp, wl=wl)
    with mp.get_context("fork").Pool(cores, initializer=_one_blas_thread) as pool:
        def run(S):
            bounds = np.linspace(0, S, min(S, 4 * cores) + 1).astype(int)
            spans = [(int(bounds[i]), int(bounds[i + 1])) for i in range(len(bounds) - 1)]
            t0 = time.perf_counter()
            parts = pool.map(_oracle_tokens, spans)
            idx = np.concatenate([p[0] for p in parts])
            gate = np.concatenate([p[1] for p in parts])
            O.build_schedule(idx, gate, wl.N, wl.B)
            return time.perf_counter() - t0

        # grow the sample until it takes about target_s or covers the batch
        S = min(wl.L, 8 * cores)
        t = run(S)
        while S < wl.L and t < 0.5 * target_s:
            S = min(wl.L, int(S * min(8.0, target_s / max(t, 1e-3))))
            t = run(S)
    _ORACLE_INPUTS.clear()
    return {"value": S / t, "unit": "routed tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": int(avail or 1),
            "threads": f"{cores} worker processes x 1 BLAS thread; schedule in the parent",
            "sample": f"first {S} of {wl.L} tokens of the {wl.name} workload, whole path "
                      f"(router log-probabilities, product top-K + gates, schedule, "
                      f"token-centric y) in {t:.1f}s; numpy float64 oracle, tokens split "
                      f"over {cores} processes on {cpu_model()}"}


def decode_step(args, B, to_dev):
    """The whole step (router, top-K, schedule, executor in auto's form) at the
    decode workload (256 tokens, N = 2^20), launched one by one and as a HIP
    graph replay, with the per-stage times: the latency-bound end of the
    workloads, where launch overhead is the cost."""
    import torch
    from synth import WORKLOADS, make_inputs

    wl = WORKLOADS["decode"]
    t = {k: to_dev(v) for k, v in make_inputs(wl).items()}
    out = B.forward(t["x"], t["wr"], t["wc"], t["w"], t["v"], wl.kprime, wl.K, wl.B,
                    t["row_bias"], t["col_bias"])
    sel = {k: out[k] for k in ("expert_idx", "score", "gate")}
    sel["workspace"] = torch.empty(
        max(1, B.lib().omni_product_topk_workspace(wl.L, wl.Nr, wl.Nc, wl.kprime, wl.K)),
        dtype=torch.uint8, device="cuda")
    a, b, sched, y = out["row_logits"], out["col_logits"], out["schedule"], out["y"]
    code = 1 if wl.dtype == "bf16" else 0
    rws = torch.empty(max(1, B.lib().omni_router_logits_workspace(code, wl.L, wl.d, wl.Nr, wl.Nc)),
                      dtype=torch.uint8, device="cuda")
    form = B.atomic_forward_mode(t["x"].dtype, wl.L, wl.d, wl.N, wl.K, wl.B)
    ews = torch.empty(max(1, B.lib().omni_atomic_forward_workspace(
        code, wl.L, wl.d, wl.N, wl.K, wl.B, B.EXEC_MODES[form])), dtype=torch.uint8, device="cuda")
    stages = {
        "router": lambda: B.router_logits(t["x"], t["wr"], t["wc"], t["row_bias"], t["col_bias"],
                                          row_logits=a, col_logits=b, workspace=rws),
        "topk": lambda: B.product_topk(a, b, wl.kprime, wl.K, want_sel=False, want_logp=False,
                                       out=sel),
        "schedule": lambda: B.schedule_tasks(sel["expert_idx"], sel["gate"], wl.N, wl.B,
                                             sched=sched),
        "execute": lambda: B.atomic_forward(t["x"], t["w"], t["v"], sched, y=y, workspace=ews),
    }

    def step():
        for f in stages.values():
            f()

    def timed(fn, reps):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        return 1e3 * (time.perf_counter() - t1) / reps

    reps = max(args.steps, 50)
    ms = timed(step, reps)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    graph_ms = timed(graph.replay, reps)
    ev = {}
    for name, f in stages.items():
        s0 = torch.cuda.Event(enable_timing=True)
        e0 = torch.cuda.Event(enable_timing=True)
        s0.record()
        for _ in range(20):
            f()
        e0.record()
        e0.synchronize()
        ev[name] = s0.elapsed_time(e0) / 20
    del t, out, graph
    torch.cuda.empty_cache()
    return {"workload": "decode", "L": wl.L, "ms_per_step": ms, "graph_ms_per_step": graph_ms,
            "tokens_per_s": wl.L / (ms * 1e-3), "executor_form": form, "stages_ms": ev,
            "steps": reps}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="large")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip timing omni_routed_backward on the same batch")
    ap.add_argument("--no-layer", action="store_true",
                    help="skip timing the whole layer (shared dense MLP + routed branch)")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip timing the variants (gated experts, id-window grouping)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip timing the HIP-graph replay of the step")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip timing the decode step (256 tokens), eager and as a graph")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run three device-to-device copies of this many MiB (a "
                         "kernel of known traffic, to calibrate HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the layer's multi-GPU sharding is a design note, not built)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    from synth import WORKLOADS, make_inputs

    wl = WORKLOADS[args.workload]
    say(f"[bench] workload {wl.name}: L={wl.L} d={wl.d} N={wl.N} ({wl.Nr}x{wl.Nc}) "
        f"k'={wl.kprime} K={wl.K} B={wl.B} {wl.dtype}")
    t0 = time.time()
    inp = make_inputs(wl)
    say(f"[bench] inputs generated in {time.time() - t0:.1f}s")

    # the CPU oracle first: its worker processes are forked before anything
    # here touches the GPU
    cpu = None
    if not args.no_cpu_baseline:
        say("[bench] timing the CPU oracle ...")
        cpu = cpu_baseline(inp, wl, args.cpu_seconds)
        say(f"[bench] oracle {cpu['value']:.1f} tokens/s ({cpu['sample']})")

    import torch
    from cartesian_routed_atomic_amd import binding as B

    def to_dev(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.bfloat16)
        return torch.from_numpy(a).to("cuda")

    t = {k: to_dev(v) for k, v in inp.items()}
    x, wr, wc, w, v = t["x"], t["wr"], t["wc"], t["w"], t["v"]
    rb, cb = t["row_bias"], t["col_bias"]
    L, K = wl.L, wl.K
    dev = "cuda"
    a = torch.empty((L, wl.Nr), dtype=torch.float32, device=dev)
    b = torch.empty((L, wl.Nc), dtype=torch.float32, device=dev)
    sel = {"expert_idx": torch.empty((L, K), dtype=torch.int32, device=dev),
           "score": torch.empty((L, K), dtype=torch.float32, device=dev),
           "gate": torch.empty((L, K), dtype=torch.float32, device=dev)}
    sel["workspace"] = torch.empty(
        max(1, B.lib().omni_product_topk_workspace(L, wl.Nr, wl.Nc, wl.kprime, K)),
        dtype=torch.uint8, device=dev)
    sched = B.alloc_schedule(L, K, wl.N, wl.B, dev)
    code = 1 if wl.dtype == "bf16" else 0
    exec_ws = torch.empty(  # large enough for every form (the forms are timed below)
        max(1, *(B.lib().omni_atomic_forward_workspace(code, L, wl.d, wl.N, K, wl.B, m)
                 for m in (1, 2, 3))),
        dtype=torch.uint8, device=dev)
    y = torch.empty((L, wl.d), dtype=torch.float32, device=dev)
    form = B.atomic_forward_mode(x.dtype, L, wl.d, wl.N, K, wl.B)

    router_ws = torch.empty(max(1, B.lib().omni_router_logits_workspace(
        1 if wl.dtype == "bf16" else 0, L, wl.d, wl.Nr, wl.Nc)), dtype=torch.uint8, device=dev)

    def stage_router():
        B.router_logits(x, wr, wc, rb, cb, row_logits=a, col_logits=b, workspace=router_ws)

    def stage_topk():
        B.product_topk(a, b, wl.kprime, K, want_sel=False, want_logp=False, out=sel)

    def stage_schedule():
        B.schedule_tasks(sel["expert_idx"], sel["gate"], wl.N, wl.B, sched=sched)

    def stage_execute():
        B.atomic_forward(x, w, v, sched, y=y, workspace=exec_ws)

    def step():
        stage_router()
        stage_topk()
        stage_schedule()
        stage_execute()

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        return 1e3 * (time.perf_counter() - t1) / args.steps

    # the four calls launched one by one: the timed step
    ms = timed(step)
    say(f"[bench] {args.steps} steps, {ms:.3f} ms/step")
    # the same four calls captured once into a HIP graph and replayed (the
    # library allocates, frees and memsets nothing, so the step is capturable)
    graph_ms = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        graph_ms = timed(graph.replay)
        say(f"[bench] graph replay: {args.steps} replays, {graph_ms:.3f} ms/step")

    # per-stage times (HIP events on the stream the kernels run on), after two
    # untimed calls (a form's first calls in a process run measurably slower)
    def ev_time(fn, reps=10, warmup=2):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        e.synchronize()
        return s.elapsed_time(e) / reps

    stages = {"router": ev_time(stage_router), "topk": ev_time(stage_topk),
              "schedule": ev_time(stage_schedule), "execute": ev_time(stage_execute)}
    # the executor call alone, in each form (the step runs `form`)
    forms_ms = {}
    for f in ("expert", "token", "grouped"):
        try:
            forms_ms[f] = ev_time(lambda: B.atomic_forward(x, w, v, sched, y=y,
                                                           workspace=exec_ws, mode=f), reps=20)
        except B.OmniError:
            forms_ms[f] = None
    exec_ms = ev_time(lambda: B.atomic_forward(x, w, v, sched, y=y, workspace=exec_ws),
                      reps=20)
    counts = sched.counts.cpu().tolist()
    n_active, n_groups = int(counts[0]), int(counts[1])
    # the grouped form's hot set for this batch, by the rule the header states
    # (experts with >= tau tasks, tau = max(2, ceil(L / 64)) doubled until at
    # most 512 reach it), recomputed here from the selection for the record
    cnt = np.bincount(sel["expert_idx"].cpu().numpy().ravel(), minlength=wl.N)
    tau = max(2, -(-L // 64))
    while (cnt >= tau).sum() > 512:
        tau *= 2
    grouped_hot = {"n_hot": int((cnt >= tau).sum()), "tau": int(tau),
                   "task_share": float(cnt[cnt >= tau].sum() / (L * K))}
    s = wl.elem_bytes
    M = L * K
    bytes_alg = 2 * wl.d * s * n_active + L * wl.d * s + 4 * L * wl.d + 12 * M
    achieved = bytes_alg / (exec_ms * 1e-3) / 1e9
    traffic = measured_traffic(wl.name, form)
    router_flop = 2.0 * L * wl.d * (wl.Nr + wl.Nc)
    router_tflops = router_flop / (stages["router"] * 1e-3) / 1e12
    say(f"[bench] stages ms {json.dumps({k: round(v4, 4) for k, v4 in stages.items()})}; "
        f"executor ({form}-centric) {exec_ms:.4f} ms, {achieved:.0f} GB/s "
        f"({100 * achieved / HBM_PEAK_GBS:.1f}% of HBM); n_active={n_active} "
        f"n_groups={n_groups}; forms ms {forms_ms}")

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 18  # float32 elements
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        say(f"[bench] copy probe: 3 copies of {args.copy_probe_mib} MiB")
        del src, dst

    bwd = None
    if not args.no_backward and B.lib().omni_routed_backward_workspace(
            1 if wl.dtype == "bf16" else 0, L, wl.d, wl.Nr, wl.Nc, K) > 0:
        # one backward call of the routed layer for a seeded upstream gradient,
        # on the selection of this batch; outputs and workspace allocated once
        dy = torch.randn((L, wl.d), generator=torch.Generator(device=dev).manual_seed(7),
                         device=dev, dtype=torch.float32)
        gb = B.routed_backward(x, wr, wc, w, v, sel["expert_idx"], sel["gate"], dy)
        bout = {k: t_ for k, t_ in gb.items() if k != "workspace"}
        bws = gb["workspace"]
        bwd_ms = ev_time(lambda: B.routed_backward(x, wr, wc, w, v, sel["expert_idx"],
                                                   sel["gate"], dy, out=bout, workspace=bws),
                         reps=5)
        na = int(gb["counts"].cpu()[0])
        NRC = wl.Nr + wl.Nc
        # what the backward must move at least: each active expert's W and V
        # rows once, x and dy once, dx, dW and dV (float32) once, the router
        # rows once and their float32 gradients, the per-task lists
        bwd_bytes = (2 * wl.d * s * na + L * wl.d * s + 4 * L * wl.d + 4 * L * wl.d
                     + 8 * wl.d * na + NRC * wl.d * s + 4 * NRC * wl.d + 8 * M)
        bwd = {"ms": bwd_ms, "bytes_alg": bwd_bytes,
               "achieved": bwd_bytes / (bwd_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
               "unit": "GB/s", "frac": bwd_bytes / (bwd_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
               "tokens_per_s": L / (bwd_ms * 1e-3), "n_active": na}
        say(f"[bench] backward {bwd_ms:.3f} ms, {bwd['achieved']:.0f} GB/s "
            f"({100 * bwd['frac']:.1f}% of HBM), {bwd['tokens_per_s']:.0f} tokens/s")

    layer = None
    if not args.no_layer:
        # the whole OmniMoE layer: the shared dense MLP writes y, then the routed
        # step runs with its executor adding onto y (one stream)
        mlp = {k: to_dev(a_) for k, a_ in make_inputs(wl, parts=("wg", "wu", "wd")).items()
               if k in ("wg", "wu", "wd")}
        d_ff = wl.d_ff
        mlp_ws = torch.empty(max(1, B.lib().omni_shared_mlp_workspace(
            1 if wl.dtype == "bf16" else 0, L, wl.d, d_ff)), dtype=torch.uint8, device=dev)
        y_layer = torch.empty((L, wl.d), dtype=torch.float32, device=dev)

        def shared():
            B.shared_mlp(x, mlp["wg"], mlp["wu"], mlp["wd"], y=y_layer, workspace=mlp_ws)

        def layer_step():
            shared()
            stage_router()
            stage_topk()
            stage_schedule()
            B.atomic_forward(x, w, v, sched, y=y_layer, accumulate=True, workspace=exec_ws)

        shared()
        layer_step()
        mlp_ms = ev_time(shared)
        layer_ms = ev_time(layer_step)
        mlp_flop = 6.0 * L * wl.d * d_ff
        mlp_tflops = mlp_flop / (mlp_ms * 1e-3) / 1e12
        mlp_peak = MFMA_BF16_TFLOPS if wl.dtype == "bf16" else FP32_TFLOPS
        layer = {"ms": layer_ms, "tokens_per_s": L / (layer_ms * 1e-3), "d_ff": d_ff,
                 "shared_mlp_ms": mlp_ms,
                 "shared_mlp_mfma": {"achieved": mlp_tflops, "peak": mlp_peak,
                                     "unit": "TFLOP/s", "frac": mlp_tflops / mlp_peak},
                 "routed_over_layer": ms / layer_ms}
        say(f"[bench] layer (shared MLP d_ff={d_ff} + routed) {layer_ms:.3f} ms, "
            f"{layer['tokens_per_s']:.0f} tokens/s; shared MLP {mlp_ms:.3f} ms = "
            f"{mlp_tflops:.0f} TFLOP/s; routed-only step / layer = {ms / layer_ms:.3f}")

    variants = None
    if not args.no_variants:
        variants = {}
        # SwiGLU-gated experts: a third expert matrix U, read per task like W
        u = to_dev(make_inputs(wl, parts=("u",))["u"])
        try:
            glu_ms = ev_time(lambda: B.atomic_forward_glu(x, w, u, v, sched, y=y,
                                                          workspace=exec_ws), reps=10)
            glu_bytes = 3 * wl.d * s * n_active + L * wl.d * s + 4 * L * wl.d + 12 * M
            variants["glu_expert"] = {
                "ms": glu_ms, "bytes_alg": glu_bytes,
                "achieved": glu_bytes / (glu_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": glu_bytes / (glu_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        except B.OmniError as exc:
            variants["glu_expert"] = {"unsupported": str(exc)}
        del u
        # the schedule with fixed id windows instead of B active experts per group
        wsched = B.alloc_schedule(L, K, wl.N, wl.B, dev, grouping="window")
        variants["window_schedule_ms"] = ev_time(
            lambda: B.schedule_tasks(sel["expert_idx"], sel["gate"], wl.N, wl.B, sched=wsched,
                                     grouping="window"))
        variants["window_groups"] = int(wsched.counts.cpu()[1])
        # the flat d x N router the Cartesian router replaces: logits for all N
        # experts, exact top-K over N per token (the pages' "without the
        # Cartesian router" ablation row)
        from synth import normal
        wf = to_dev(normal((wl.N, wl.d), 1000 * wl.index + 9, 1.0 / wl.d ** 0.5, wl.dtype))
        fr = B.flat_router_topk(x, wf, K)
        flat_ms = ev_time(lambda: B.flat_router_topk(x, wf, K, out=fr, workspace=fr["workspace"]),
                          reps=2)
        product_ms = stages["router"] + stages["topk"]
        flat_flop = 2.0 * L * wl.d * wl.N
        variants["flat_router"] = {
            "ms": flat_ms, "product_router_ms": product_ms, "ratio": flat_ms / product_ms,
            "gemm_tflops": flat_flop / (flat_ms * 1e-3) / 1e12,
            "logits_bytes": 4 * L * wl.N}
        del wf, fr
        say(f"[bench] variants: {json.dumps(variants)}")

    decode = None
    if not args.no_decode and wl.name != "decode":
        decode = decode_step(args, B, to_dev)
        say(f"[bench] decode step: {json.dumps(decode)}")

    rec = {
        "metric": METRIC,
        "value": L / (ms * 1e-3),
        "unit": "routed tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "graph_ms_per_step": graph_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic: seeded Gaussian x ~ N(0,1), W, V, Wr, Wc ~ N(0,1/d), bf16",
        "config": {"workload": wl.name, "L": L, "d": wl.d, "N": wl.N,
                   "grid": [wl.Nr, wl.Nc], "kprime": wl.kprime, "K": K, "B": wl.B,
                   "zipf_s": wl.zipf_s},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "traffic_over_alg": None if traffic is None else traffic / bytes_alg,
                     "kernel": EXEC_KERNELS[form], "bytes_alg": bytes_alg,
                     "kernel_ms": exec_ms},
        "executor_form": form,
        "executor_forms_ms": forms_ms,
        "grouped_hot_set": grouped_hot,
        "router_mfma": {"achieved": router_tflops, "peak": MFMA_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": router_tflops / MFMA_BF16_TFLOPS,
                        "note": "router call = one MFMA GEMM kernel (bias fused)"},
        "stages_ms": stages,
        "n_active": n_active,
        "expert_usage": n_active / wl.N,
        "backward": bwd,
        "layer": layer,
        "variants": variants,
        "decode_step": decode,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
