"""omni_product_topk_static, the product top-K with its workspace in the
library's fixed per-GPU device array, against omni_product_topk with a
caller workspace: bit-identical outputs on two calls in a row (the second on
fewer tokens, so it runs over what the first left in the array), with and
without the per-axis lists, through the C ABI.  Sizes beyond the array are
refused on the host before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import cartesian_routed_atomic_amd.binding as B
from synth import tie_case

SCRATCH = 8 << 20


def _a(n):
    return (n + 255) // 256 * 256


def _need(L, kp, lists_r, lists_c):
    return _a(4 * L) + _a(8 * L) + (_a(4 * L * kp) if lists_r else 0) + \
        (_a(4 * L * kp) if lists_c else 0)


def test_sizes_beyond_the_array_are_refused_on_the_host():
    lib = B.lib()
    f = lib.omni_product_topk_static
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: the size check comes first

    def call(L, with_lists):
        sel = None if with_lists else fake
        return f(L, 1024, 1024, 64, 64, fake, fake, fake, fake, fake, None, None, sel, sel, None)
    # the largest batches that fit, per the header: 16,008 tokens with both lists,
    # 699,040 without; one more token is refused
    assert _need(16008, 64, True, True) <= SCRATCH < _need(16009, 64, True, True)
    assert _need(699040, 64, False, False) <= SCRATCH < _need(699041, 64, False, False)
    assert call(16009, True) == B.OMNI_ERR_WORKSPACE
    assert call(699041, False) == B.OMNI_ERR_WORKSPACE
    assert call(0, True) == B.OMNI_OK
    assert f(4, 8, 8, 9, 4, fake, fake, fake, fake, fake, None, None, None, None,
             None) == B.OMNI_ERR_INVALID_ARG  # k' > grid lines, as omni_product_topk


def _run_both(za, zb, kp, K, lists):
    lib = B.lib()
    L, Nr = za.shape
    Nc = zb.shape[1]
    dev = "cuda"
    zr, zc = torch.from_numpy(za).to(dev), torch.from_numpy(zb).to(dev)
    outs = []
    for static in (False, True):
        o = {"idx": torch.full((L, K), -7, dtype=torch.int32, device=dev),
             "score": torch.full((L, K), np.nan, device=dev),
             "gate": torch.full((L, K), np.nan, device=dev),
             "a": torch.full((L, Nr), np.nan, device=dev),
             "b": torch.full((L, Nc), np.nan, device=dev)}
        if lists:
            o["R"] = torch.full((L, kp), -7, dtype=torch.int32, device=dev)
            o["C"] = torch.full((L, kp), -7, dtype=torch.int32, device=dev)
        p = {k: ctypes.c_void_p(t.data_ptr()) for k, t in o.items()}
        R, C = (p["R"], p["C"]) if lists else (None, None)
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        if static:
            rc = lib.omni_product_topk_static(L, Nr, Nc, kp, K, ctypes.c_void_p(zr.data_ptr()),
                                              ctypes.c_void_p(zc.data_ptr()), p["idx"],
                                              p["score"], p["gate"], p["a"], p["b"], R, C, st)
        else:
            nws = lib.omni_product_topk_workspace(L, Nr, Nc, kp, K)
            ws = torch.empty(nws, dtype=torch.uint8, device=dev)
            rc = lib.omni_product_topk(L, Nr, Nc, kp, K, ctypes.c_void_p(zr.data_ptr()),
                                       ctypes.c_void_p(zc.data_ptr()), p["idx"], p["score"],
                                       p["gate"], p["a"], p["b"], R, C,
                                       ctypes.c_void_p(ws.data_ptr()), nws, st)
        assert rc == B.OMNI_OK
        torch.cuda.synchronize()
        outs.append({k: t.cpu().numpy() for k, t in o.items()})
    ref, got = outs
    for k in ref:
        np.testing.assert_array_equal(got[k].view(np.uint32) if got[k].dtype == np.float32
                                      else got[k],
                                      ref[k].view(np.uint32) if ref[k].dtype == np.float32
                                      else ref[k], err_msg=k)


@pytest.mark.gpu
@pytest.mark.parametrize("lists", [False, True])
def test_static_workspace_matches_the_caller_workspace(lists):
    # first call: 3000 tokens of a tie-heavy 256 x 192 grid (many tokens take
    # the exact fix-up); second call: 700 tokens of another grid, so it runs
    # over what the first left in the array
    rng = np.random.default_rng(5)
    za, zb = tie_case(3000, 256, 192, 0.25)
    _run_both(za, zb, 48, 40, lists)
    za2 = rng.standard_normal((700, 1024)).astype(np.float32)
    zb2 = rng.standard_normal((700, 1024)).astype(np.float32)
    _run_both(za2, zb2, 64, 64, lists)
