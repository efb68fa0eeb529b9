"""sda_sparse_decode_attn_noalloc: the whole op with the library's static scratch as its workspace, for
callers that cannot allocate. Its results must equal those of sda_sparse_decode_attn with a caller
workspace, bit for bit, on consecutive calls whose second input is smaller (the scratch keeps the first
call's contents), and meet the oracle's bar."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import sliding_window_decode_amd as sda
import workloads as wl
from gpu_util import DeviceWorkload, compare


def test_noalloc_rejects_plans_beyond_the_scratch():
    """No device access: a split plan whose partials exceed SDA_SCRATCH_BYTES is refused on the host."""
    plan = sda.make_plan(128, 128, 576, 2048, 0)
    need = sda.noalloc_workspace_bytes(128, 128, 512, plan)
    assert need > sda.SCRATCH_BYTES
    plan.whole_tokens = 1
    assert sda.noalloc_workspace_bytes(128, 128, 512, plan) == 0
    plan.whole_tokens = 0
    cache = sda.sda_cache(1 << 30, 2048, 64, sda.V32_656, 64 * 656, None)
    lst = sda.sda_list(1 << 31, 2048, 2048, 1, None)
    rc = sda.lib().sda_sparse_decode_attn_noalloc(1 << 32, 128 * 576, 576, 128, 128, 576, 512, ctypes.byref(cache),
                                                  ctypes.byref(lst), None, None, None, ctypes.c_float(0.04),
                                                  ctypes.byref(plan), None, None, 1 << 33, 128 * 512, 512, 1 << 34,
                                                  128, None)
    assert rc == sda.SDA_ERR_WORKSPACE


def _pair(w, plan):
    dw = DeviceWorkload(w)
    out_ref, lse_ref, _ = dw.run(plan=plan)
    out = torch.full_like(out_ref, 3.0)
    lse = torch.full_like(lse_ref, 3.0)
    # meta and num_splits NULL: the scheduler runs into the scratch as well
    sda.sparse_decode_attn_noalloc(dw.q, dw.cache, dw.lst, dw.xcache, dw.xlst, dw.sink, w.scale, plan, None, None,
                                   out, lse)
    torch.cuda.synchronize()
    return out, lse, out_ref, lse_ref


@pytest.mark.gpu
def test_noalloc_equals_the_workspace_entry_point_on_consecutive_calls():
    cases = [  # (seed, T, H, width, xwidth): the second call is smaller than the first
        (11, 40, 32, 128, 512),
        (12, 9, 16, 96, 200),
    ]
    for seed, T, H, W, X in cases:
        w = wl.small_workload(seed, wl.FP8_528, wl.FP8_528, T=T, H=H, width=W, xwidth=X, num_slots=4096, sink=True,
                              p_invalid=0.05, lens_lo=1)
        plan = sda.make_plan(w.T, w.H, w.d_qk, W, X)
        assert not plan.whole_tokens
        need = sda.noalloc_workspace_bytes(w.T, w.H, 512, plan)
        assert 0 < need <= sda.SCRATCH_BYTES
        print(f"[noalloc] T={T} H={H} {plan} scratch {need} B", flush=True)
        out, lse, out_ref, lse_ref = _pair(w, plan)
        assert torch.equal(out, out_ref) and torch.equal(lse, lse_ref), f"T={T}: differs from the workspace call"
        o_ref, l_ref, o_abs = oracle.attention(w, nthreads=8, with_abs=True)
        compare(out, lse, o_ref, l_ref, o_abs, what=f"noalloc T={T}")


@pytest.mark.gpu
def test_noalloc_whole_token_plan_needs_no_scratch():
    w = wl.make_workload("c5_topk_v32", seed=2, T=3)
    plan = sda.make_plan(w.T, w.H, w.d_qk, w.lst.width, 0)
    plan.whole_tokens = 1
    assert sda.noalloc_workspace_bytes(w.T, w.H, 512, plan) == 0
    out, lse, out_ref, lse_ref = _pair(w, plan)
    assert torch.equal(out, out_ref) and torch.equal(lse, lse_ref)
