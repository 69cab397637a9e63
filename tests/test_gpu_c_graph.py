"""The four calls captured into a HIP graph (through torch's stream capture)
and replayed: every replay, with eager work and synchronisations in between,
must reproduce the eager outputs bit for bit."""
import numpy as np
import pytest
import torch

from synth import WORKLOADS, make_inputs
from tests.gpu_helpers import dev, host, log

pytestmark = pytest.mark.gpu

B = pytest.importorskip("cartesian_routed_atomic_amd.binding")


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_graph_replay_matches_eager(name):
    wl = WORKLOADS[name]
    inp = make_inputs(wl)
    t = {k: dev(v) for k, v in inp.items()}
    L, K = wl.L, wl.K
    zr = torch.empty((L, wl.Nr), dtype=torch.float32, device="cuda")
    zc = torch.empty((L, wl.Nc), dtype=torch.float32, device="cuda")
    sel = {"expert_idx": torch.empty((L, K), dtype=torch.int32, device="cuda"),
           "score": torch.empty((L, K), dtype=torch.float32, device="cuda"),
           "gate": torch.empty((L, K), dtype=torch.float32, device="cuda"),
           "workspace": torch.empty(
               max(1, B.lib().omni_product_topk_workspace(L, wl.Nr, wl.Nc, wl.kprime, K)),
               dtype=torch.uint8, device="cuda")}
    sched = B.alloc_schedule(L, K, wl.N, wl.B, "cuda")
    code = 1 if wl.dtype == "bf16" else 0
    ws = torch.empty(max(1, B.lib().omni_atomic_forward_workspace(code, L, wl.d, wl.N, K, wl.B, 0)),
                     dtype=torch.uint8, device="cuda")
    y = torch.empty((L, wl.d), dtype=torch.float32, device="cuda")

    def step():
        B.router_logits(t["x"], t["wr"], t["wc"], t["row_bias"], t["col_bias"],
                        row_logits=zr, col_logits=zc)
        B.product_topk(zr, zc, wl.kprime, K, want_sel=False, want_logp=False, out=sel)
        B.schedule_tasks(sel["expert_idx"], sel["gate"], wl.N, wl.B, sched=sched)
        B.atomic_forward(t["x"], t["w"], t["v"], sched, y=y, workspace=ws)

    outs = lambda: [host(a).copy() for a in (zr, zc, sel["expert_idx"], sel["score"],
                                             sel["gate"], sched.counts, sched.task_index,
                                             sched.task_token, sched.group_offsets, y)]
    step()
    torch.cuda.synchronize()
    want = outs()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for a in (zr, zc, y, sel["gate"]):  # poison the outputs between replays
            a.fill_(float("nan"))
        sched.task_index.fill_(-7)
        _ = (t["x"].float() * 2).sum().item()  # unrelated eager work + a sync
        g.replay()
        torch.cuda.synchronize()
        got = outs()
        for w_, g_ in zip(want, got):
            np.testing.assert_array_equal(w_.view(np.uint8), g_.view(np.uint8))
        log(f"  {name}: graph replay {rep} bit-identical to eager")
