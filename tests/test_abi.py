"""The C-ABI library loads, exports every symbol include/omni.h declares, and
rejects bad arguments on the host (these calls return before any HIP call, so
they need no GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "omni.h")

B = pytest.importorskip("cartesian_routed_atomic_amd.binding")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(omni_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail(f"{B.LIB_PATH} missing: run __graft_entry__.build() first")
    return B.lib()


def test_header_declares_the_four_entry_points():
    d = _declared()
    for name in ("omni_router_logits", "omni_product_topk", "omni_schedule_tasks",
                 "omni_atomic_forward"):
        assert name in d


def test_every_declared_symbol_is_exported(lib):
    raw = ctypes.CDLL(B.LIB_PATH)
    for name in _declared():
        assert hasattr(raw, name), name
    assert set(_declared()) == set(B.EXPORTS)


def test_abi_version_and_status_strings(lib):
    assert lib.omni_abi_version() == 14
    for code in range(5):
        assert lib.omni_status_string(code)
    assert lib.omni_status_string(99) == b"unknown status"


FAKE = ctypes.c_void_p(1 << 20)       # aligned, never dereferenced (checks fail first)
MIS = ctypes.c_void_p((1 << 20) + 2)  # misaligned


def test_router_argument_checks(lib):
    f = lib.omni_router_logits
    ok_args = dict(dt=B.OMNI_BF16, L=4, d=64, Nr=8, Nc=8)

    def call(dt=1, L=4, d=64, Nr=8, Nc=8, x=FAKE, wr=FAKE, wc=FAKE, rl=FAKE, cl=FAKE, ws=None,
             n=0):
        return f(dt, L, d, Nr, Nc, x, wr, wc, None, None, rl, cl, ws, n, None)
    assert ok_args
    assert call(dt=7) == B.OMNI_ERR_INVALID_ARG
    assert call(L=-1) == B.OMNI_ERR_INVALID_ARG
    assert call(Nr=0) == B.OMNI_ERR_INVALID_ARG
    assert call(x=None) == B.OMNI_ERR_INVALID_ARG
    assert call(rl=None) == B.OMNI_ERR_INVALID_ARG
    assert call(x=MIS) == B.OMNI_ERR_INVALID_ARG
    assert call(d=60) == B.OMNI_ERR_UNSUPPORTED          # bf16 needs d % 8 == 0
    assert call(dt=0, d=66) == B.OMNI_ERR_UNSUPPORTED    # f32 needs d % 4 == 0
    assert call(L=1 << 30, d=64) == B.OMNI_ERR_UNSUPPORTED
    assert call(L=0) == B.OMNI_OK                        # empty batch: nothing enqueued
    # few tokens: the contraction over d is split and the partials need a workspace
    nws = lib.omni_router_logits_workspace(1, 256, 2048, 1024, 1024)
    assert nws == 8 * 256 * 2048 * 4                     # 8 chunks of 256 features
    assert lib.omni_router_logits_workspace(1, 8192, 2048, 1024, 1024) == 0   # enough tiles
    assert lib.omni_router_logits_workspace(0, 256, 2048, 1024, 1024) == 0    # float32 path
    assert call(L=256, d=2048, Nr=1024, Nc=1024) == B.OMNI_ERR_WORKSPACE
    assert call(L=256, d=2048, Nr=1024, Nc=1024, ws=FAKE, n=nws - 1) == B.OMNI_ERR_WORKSPACE
    assert call(L=256, d=2048, Nr=1024, Nc=1024, ws=ctypes.c_void_p((1 << 20) + 16),
                n=nws) == B.OMNI_ERR_WORKSPACE


def test_product_topk_argument_checks(lib):
    f = lib.omni_product_topk

    def call(L=4, Nr=16, Nc=16, kp=4, K=4, ws=None, nws=0):
        return f(L, Nr, Nc, kp, K, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, None, ws, nws,
                 None)
    assert call(kp=0) == B.OMNI_ERR_INVALID_ARG
    assert call(kp=17) == B.OMNI_ERR_INVALID_ARG         # k' > Nr
    assert call(kp=4, K=17) == B.OMNI_ERR_INVALID_ARG    # K > k'^2
    assert call(K=0) == B.OMNI_ERR_INVALID_ARG
    assert call(Nr=1 << 16, Nc=1 << 16, kp=4) == B.OMNI_ERR_INVALID_ARG  # N >= 2^31
    assert call(Nr=128, Nc=128, kp=65, K=8) == B.OMNI_ERR_UNSUPPORTED
    assert call(Nr=128, Nc=128, kp=64, K=65) == B.OMNI_ERR_UNSUPPORTED
    assert call(Nr=4096, Nc=16, kp=4, K=4) == B.OMNI_ERR_UNSUPPORTED
    assert call(L=0) == B.OMNI_OK
    nws = lib.omni_product_topk_workspace(8192, 1024, 1024, 64, 64)
    assert nws >= 8192 * 4 + 2 * 8192 * 64 * 4
    assert call(ws=None, nws=nws) == B.OMNI_ERR_WORKSPACE
    assert call(ws=FAKE, nws=1) == B.OMNI_ERR_WORKSPACE
    assert call(ws=ctypes.c_void_p((1 << 20) + 8), nws=1 << 20) == B.OMNI_ERR_WORKSPACE


def test_schedule_argument_checks(lib):
    L, K, N, Bg = 64, 8, 1024, 16
    assert lib.omni_schedule_max_groups(L, K, N, Bg, 0) == 32
    assert lib.omni_schedule_max_groups(8192, 64, 1 << 20, 256, 0) == 2048
    assert lib.omni_schedule_max_groups(256, 64, 1 << 20, 64, 0) == 256
    # id windows: every window of the id space is a group
    assert lib.omni_schedule_max_groups(L, K, N, Bg, 1) == 64
    assert lib.omni_schedule_max_groups(256, 64, 1 << 20, 64, 1) == 16384
    assert lib.omni_schedule_max_groups(L, K, N, Bg, 2) == 0
    assert lib.omni_schedule_workspace(L, K, N, Bg, 2) == 0
    nws = lib.omni_schedule_workspace(L, K, N, Bg, 0)
    assert nws > 0
    st = B.ScheduleStruct(*([1 << 20] * 7))
    f = lib.omni_schedule_tasks

    def call(L=L, K=K, N=N, Bg=Bg, ws=FAKE, n=nws, s=st, grouping=0):
        return f(L, K, N, Bg, grouping, FAKE, FAKE, ctypes.byref(s) if s is not None else None,
                 ws, n, None)
    assert call(grouping=2) == B.OMNI_ERR_INVALID_ARG
    assert call(grouping=-1) == B.OMNI_ERR_INVALID_ARG
    assert call(K=0) == B.OMNI_ERR_INVALID_ARG
    assert call(Bg=0) == B.OMNI_ERR_INVALID_ARG
    assert call(N=0) == B.OMNI_ERR_INVALID_ARG
    assert call(L=1 << 28, K=64) == B.OMNI_ERR_INVALID_ARG   # L*K >= 2^31
    assert call(s=None) == B.OMNI_ERR_INVALID_ARG
    assert call(n=nws - 1) == B.OMNI_ERR_WORKSPACE
    assert call(ws=None) == B.OMNI_ERR_WORKSPACE
    assert call(ws=ctypes.c_void_p((1 << 20) + 16)) == B.OMNI_ERR_WORKSPACE  # not 256-aligned
    bad = B.ScheduleStruct(*([1 << 20] * 3 + [0] + [1 << 20] * 3))
    assert call(s=bad) == B.OMNI_ERR_INVALID_ARG


def test_atomic_forward_argument_checks(lib):
    st = B.ScheduleStruct(*([1 << 20] * 7))
    f = lib.omni_atomic_forward

    def call(dt=1, L=4, d=128, N=64, K=2, Bg=4, x=FAKE, w=FAKE, v=FAKE, y=FAKE, s=st, mode=0):
        return f(dt, L, d, N, K, Bg, x, w, v, ctypes.byref(s) if s is not None else None,
                 y, 0, mode, None, 0, None)
    assert call(dt=3) == B.OMNI_ERR_INVALID_ARG
    assert call(s=None) == B.OMNI_ERR_INVALID_ARG
    assert call(y=None) == B.OMNI_ERR_INVALID_ARG
    assert call(w=MIS) == B.OMNI_ERR_INVALID_ARG
    assert call(mode=4) == B.OMNI_ERR_INVALID_ARG
    assert call(mode=-1) == B.OMNI_ERR_INVALID_ARG
    # the grouped form: bf16 only, K <= 64, d a power of two up to 2048
    assert call(dt=0, mode=3) == B.OMNI_ERR_UNSUPPORTED
    assert call(d=4096, mode=3) == B.OMNI_ERR_UNSUPPORTED
    assert call(d=768, mode=3) == B.OMNI_ERR_UNSUPPORTED
    assert call(K=65, mode=3) == B.OMNI_ERR_UNSUPPORTED
    assert call(d=2048, mode=3) == B.OMNI_ERR_WORKSPACE
    # the expert- and token-centric forms: any d = 64 m up to 16384
    assert call(d=96) == B.OMNI_ERR_UNSUPPORTED
    assert call(d=16448) == B.OMNI_ERR_UNSUPPORTED
    assert call(d=32) == B.OMNI_ERR_UNSUPPORTED
    for d in (192, 320, 768, 3072, 4096, 16384):
        for mode in (0, 1, 2):
            assert call(d=d, mode=mode) == B.OMNI_ERR_WORKSPACE, (d, mode)
    assert call(dt=0, d=2048, mode=2) == B.OMNI_ERR_WORKSPACE
    assert call(L=0) == B.OMNI_OK
    assert call() == B.OMNI_ERR_WORKSPACE                  # L*K tasks need a workspace
    noidx = B.ScheduleStruct(*([1 << 20] * 6 + [0]))
    assert call(s=noidx) == B.OMNI_ERR_INVALID_ARG          # task_index is required
    # the flattened selection: both arrays or neither
    half = B.ScheduleStruct(*([1 << 20] * 8 + [0]))
    assert call(s=half) == B.OMNI_ERR_INVALID_ARG
    both = B.ScheduleStruct(*([1 << 20] * 9))
    assert call(s=both) == B.OMNI_ERR_WORKSPACE
    ws = lib.omni_atomic_forward_workspace
    # per form: 8 bytes per task; the grouped form adds a task count per
    # expert id (4 bytes each), 16 level lists of 512 ids (32 KiB) and the
    # gathered W_H and V_H^T (1 KiB each per column of d)
    for mode in (1, 2):
        assert 8 * 8192 * 64 <= ws(1, 8192, 2048, 1 << 20, 64, 256, mode) < 8 * 8192 * 64 + 4096
    g = ws(1, 8192, 2048, 1 << 20, 64, 256, 3)
    assert g >= 8 * 8192 * 64 + 4 * (1 << 20) + 32768 + 2 * 1024 * 2048
    assert g < 8 * 8192 * 64 + 4 * (1 << 20) + 32768 + 2 * 1024 * 2048 + 8192
    # auto sizes for the form it runs; an invalid mode or dtype asks for nothing
    auto_form = lib.omni_atomic_forward_mode(1, 8192, 2048, 1 << 20, 64, 256)
    assert ws(1, 8192, 2048, 1 << 20, 64, 256, 0) == ws(1, 8192, 2048, 1 << 20, 64, 256,
                                                         auto_form)
    assert ws(1, 8192, 2048, 1 << 20, 64, 256, 4) == 0
    assert ws(2, 8192, 2048, 1 << 20, 64, 256, 1) == 0


def test_atomic_forward_auto_mode(lib):
    mode = lib.omni_atomic_forward_mode
    # the measured crossovers: token-centric from L = 8192 tokens of d >= 1024,
    # and below 4096 tokens (each token split over several waves)
    assert mode(1, 8192, 2048, 1 << 20, 64, 256) == 2      # large
    assert mode(1, 16384, 2048, 1 << 18, 64, 128) == 2     # mid
    assert mode(1, 4096, 1024, 1 << 14, 32, 64) == 1       # small
    assert mode(1, 256, 2048, 1 << 20, 64, 64) == 2        # decode
    assert mode(0, 64, 128, 1024, 8, 16) == 2              # tiny float32
    assert mode(0, 64, 2048, 1024, 8, 16) == 1             # float32 row over 4 KiB
    assert mode(1, 8192, 4096, 1 << 20, 64, 256) == 1      # row over 4 KiB
    assert mode(0, 8192, 2048, 1 << 20, 64, 256) == 1      # float32 row over 4 KiB
    assert mode(1, 8192, 768, 1 << 20, 64, 256) == 1       # d not a power of two (chunked)
    assert mode(3, 8192, 2048, 1 << 20, 64, 256) == 0      # bad dtype
    assert mode(1, 8192, 2048, 1 << 20, 0, 256) == 0       # bad K


def test_routed_backward_argument_checks(lib):
    f = lib.omni_routed_backward
    nws = lib.omni_routed_backward_workspace(1, 4, 128, 8, 8, 4)
    assert nws > 0
    assert lib.omni_routed_backward_workspace(1, 4, 128, 8, 8, 65) == 0

    def call(dt=1, L=4, d=128, Nr=8, Nc=8, K=4, x=FAKE, dy=FAKE, dw=FAKE, ws=FAKE, n=nws,
             dwr=FAKE):
        P = [x, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, dy, FAKE, dwr, FAKE, None, None, FAKE,
             FAKE, dw, FAKE, None]
        return f(dt, L, d, Nr, Nc, K, *P, ws, n, None)
    assert call(dt=2) == B.OMNI_ERR_INVALID_ARG
    assert call(K=0) == B.OMNI_ERR_INVALID_ARG
    assert call(x=None) == B.OMNI_ERR_INVALID_ARG
    assert call(dw=None) == B.OMNI_ERR_INVALID_ARG
    assert call(dwr=MIS) == B.OMNI_ERR_INVALID_ARG
    assert call(K=65) == B.OMNI_ERR_UNSUPPORTED
    assert call(d=4096) == B.OMNI_ERR_UNSUPPORTED           # bf16 rows over 4 KiB
    assert call(dt=0, d=2048) == B.OMNI_ERR_UNSUPPORTED     # float32 rows over 4 KiB
    assert call(d=96) == B.OMNI_ERR_UNSUPPORTED
    assert call(n=nws - 1) == B.OMNI_ERR_WORKSPACE
    assert call(ws=ctypes.c_void_p((1 << 20) + 16)) == B.OMNI_ERR_WORKSPACE
    # no tokens: still zero router gradients to write, through the workspace
    assert call(L=0, x=None, dy=None, ws=None, n=0) == B.OMNI_ERR_WORKSPACE


def test_shared_mlp_argument_checks(lib):
    f = lib.omni_shared_mlp
    nws = lib.omni_shared_mlp_workspace(1, 4, 128, 256)
    assert nws == 4 * 256 * 2                 # the hidden activation; no split over d_ff = 256
    assert lib.omni_shared_mlp_workspace(0, 4, 128, 256) == 4 * 256 * 4
    assert lib.omni_shared_mlp_workspace(1, 4, 128, 0) == 0
    assert lib.omni_shared_mlp_workspace(2, 4, 128, 256) == 0
    # few tokens, long hidden width: the down product is split, partials after the hidden
    big = lib.omni_shared_mlp_workspace(1, 256, 2048, 5632)
    assert big == 256 * 5632 * 2 + 8 * 256 * 2048 * 4

    def call(dt=1, L=4, d=128, d_ff=256, x=FAKE, wg=FAKE, wu=FAKE, wd=FAKE, y=FAKE, ws=FAKE,
             n=nws):
        return f(dt, L, d, d_ff, x, wg, wu, wd, y, 0, ws, n, None)
    assert call(dt=2) == B.OMNI_ERR_INVALID_ARG
    assert call(d=0) == B.OMNI_ERR_INVALID_ARG
    assert call(d_ff=0) == B.OMNI_ERR_INVALID_ARG
    assert call(L=-1) == B.OMNI_ERR_INVALID_ARG
    assert call(x=None) == B.OMNI_ERR_INVALID_ARG
    assert call(wd=None) == B.OMNI_ERR_INVALID_ARG
    assert call(wu=MIS) == B.OMNI_ERR_INVALID_ARG
    assert call(d=132) == B.OMNI_ERR_UNSUPPORTED            # bf16 needs multiples of 8
    assert call(d_ff=252) == B.OMNI_ERR_UNSUPPORTED
    assert call(dt=0, d=130, n=4096) == B.OMNI_ERR_UNSUPPORTED  # float32: multiples of 4
    assert call(n=nws - 1) == B.OMNI_ERR_WORKSPACE
    assert call(ws=ctypes.c_void_p((1 << 20) + 16)) == B.OMNI_ERR_WORKSPACE
    # an empty batch needs no x or y and enqueues nothing
    assert call(L=0, x=None, y=None, n=lib.omni_shared_mlp_workspace(1, 0, 128, 256)) == B.OMNI_OK
    assert call(L=0, x=None, y=None, ws=None, n=0) == B.OMNI_OK


def test_atomic_forward_glu_argument_checks(lib):
    st = B.ScheduleStruct(*([1 << 20] * 7))
    f = lib.omni_atomic_forward_glu
    nws = lib.omni_atomic_forward_workspace(1, 4, 128, 64, 2, 4, 2)

    def call(dt=1, L=4, d=128, N=64, K=2, Bg=4, x=FAKE, u=FAKE, y=FAKE, s=st, ws=FAKE, n=nws):
        return f(dt, L, d, N, K, Bg, x, FAKE, u, FAKE, ctypes.byref(s) if s is not None else None,
                 y, 0, ws, n, None)
    assert call(dt=2) == B.OMNI_ERR_INVALID_ARG
    assert call(u=None) == B.OMNI_ERR_INVALID_ARG
    assert call(s=None) == B.OMNI_ERR_INVALID_ARG
    assert call(s=B.ScheduleStruct(*([1 << 20] * 7 + [0, 1 << 20]))) == B.OMNI_ERR_INVALID_ARG
    assert call(x=None) == B.OMNI_ERR_INVALID_ARG
    assert call(u=MIS) == B.OMNI_ERR_INVALID_ARG
    assert call(d=96) == B.OMNI_ERR_UNSUPPORTED
    assert call(d=16448) == B.OMNI_ERR_UNSUPPORTED
    # any d = 64 m up to 16384 (rows over 4 KiB or m not a power of two:
    # chunked); no workspace, so the call stops before any launch
    assert call(d=4096, ws=None, n=0) == B.OMNI_ERR_WORKSPACE
    assert call(d=768, ws=None, n=0) == B.OMNI_ERR_WORKSPACE
    assert call(dt=0, d=2048, ws=None, n=0) == B.OMNI_ERR_WORKSPACE
    assert call(n=nws - 1) == B.OMNI_ERR_WORKSPACE
    assert call(L=0, x=None, y=None) == B.OMNI_OK


def test_flat_router_argument_checks(lib):
    f = lib.omni_flat_router_topk
    nws = lib.omni_flat_router_workspace(1, 4, 1000)
    assert nws >= 4 * 1000 * 4 and nws % 256 == 0
    assert lib.omni_flat_router_workspace(2, 4, 1000) == 0

    def call(dt=1, L=4, d=128, N=1000, K=8, x=FAKE, wf=FAKE, idx=FAKE, ws=FAKE, n=nws):
        return f(dt, L, d, N, K, x, wf, None, idx, FAKE, FAKE, None, ws, n, None)
    assert call(dt=2) == B.OMNI_ERR_INVALID_ARG
    assert call(K=0) == B.OMNI_ERR_INVALID_ARG
    assert call(K=1001) == B.OMNI_ERR_INVALID_ARG             # K > N
    assert call(wf=None) == B.OMNI_ERR_INVALID_ARG
    assert call(idx=None) == B.OMNI_ERR_INVALID_ARG
    assert call(wf=MIS) == B.OMNI_ERR_INVALID_ARG
    assert call(K=65) == B.OMNI_ERR_UNSUPPORTED
    assert call(d=132) == B.OMNI_ERR_UNSUPPORTED
    assert call(n=nws - 1) == B.OMNI_ERR_WORKSPACE
    assert call(L=0, x=None, idx=None, n=lib.omni_flat_router_workspace(1, 0, 1000)) == B.OMNI_OK
    assert call(L=0, x=None, idx=None, ws=None, n=0) == B.OMNI_OK


def test_binding_refuses_a_schedule_of_another_shape():
    # the executor indexes x, W and V with the schedule's token and expert ids
    import types
    sched = types.SimpleNamespace(L=4, N=100, task_index=object())
    B._same_shape_schedule(sched, 4, 100)
    with pytest.raises(ValueError):
        B._same_shape_schedule(sched, 5, 100)
    with pytest.raises(ValueError):
        B._same_shape_schedule(sched, 4, 99)
    with pytest.raises(ValueError):
        B._same_shape_schedule(types.SimpleNamespace(L=4, N=100, task_index=None), 4, 100)
