"""The schedule built on a second stream while the token-centric executor
runs (the token-centric form reads the flattened selection, not the
schedule): the same schedule and the same y bits as the calls in line, also
when the step is captured into a HIP graph and replayed."""
import numpy as np
import pytest
import torch

from synth import custom, make_inputs
from tests.gpu_helpers import dev, log
from tests.test_gpu_a_parity import run_pipeline

pytestmark = pytest.mark.gpu

B = pytest.importorskip("cartesian_routed_atomic_amd.binding")

FIELDS = ("counts", "active", "group_offsets", "task_token", "task_expert", "task_gate",
          "task_index")


@pytest.mark.parametrize("mode", ["token"])
def test_schedule_overlaps_the_executor(mode):
    wl = custom(L=8200, d=512, Nr=64, Nc=64, kprime=16, K=16, B=32, dtype="bf16",
                zipf_s=1.1, index=230)
    inp = make_inputs(wl)
    ref = run_pipeline(wl, inp)  # router, top-K, schedule, executor in line
    t = {k: dev(inp[k]) for k in ("x", "w", "v")}
    y_ref = B.atomic_forward(t["x"], t["w"], t["v"], ref["schedule"], mode=mode)
    torch.cuda.synchronize()
    sel = {"expert_idx": ref["expert_idx"], "gate": ref["gate"]}
    sched = B.alloc_schedule(wl.L, wl.K, wl.N, wl.B, "cuda")
    y = torch.empty_like(y_ref)
    side = torch.cuda.Stream()

    def step():
        main = torch.cuda.current_stream()
        side.wait_stream(main)
        with torch.cuda.stream(side):
            B.schedule_tasks(sel["expert_idx"], sel["gate"], wl.N, wl.B, sched=sched)
        # the executor needs only the flattened selection
        sched.flat_expert, sched.flat_gate = sel["expert_idx"], sel["gate"]
        B.atomic_forward(t["x"], t["w"], t["v"], sched, y=y, mode=mode)
        main.wait_stream(side)

    def check(what):
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32)), what
        for f in FIELDS:
            got, want = getattr(sched, f), getattr(ref["schedule"], f)
            if f == "active":  # entries from n_active on are unspecified
                n = int(ref["schedule"].counts[0].item())
                got, want = got[:n], want[:n]
            assert torch.equal(got, want), (what, f)

    for rep in range(3):
        y.fill_(np.nan)
        step()
        check(f"eager step {rep}")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        y.fill_(np.nan)
        torch.cuda.synchronize()
        graph.replay()
        check(f"graph replay {rep}")
    log(f"[overlap] {mode}: schedule and y bit-identical to the calls in line, "
        "eagerly and over 3 graph replays")
