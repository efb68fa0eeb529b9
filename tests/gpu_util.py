"""Helpers for GPU tests: move a synthetic workload to the device, run the HIP path through the
C ABI, and compare with the oracle at the stated tolerances."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import sliding_window_decode_amd as sda

# Tolerances: bf16 output vs the round-to-nearest-even bf16 of the fp64 oracle, and fp32 LSE.
OUT_MAX_ABS = 1e-2
OUT_REL_L2 = 5e-3
LSE_MAX_ABS = 1e-3


def dev_cache(c, device="cuda"):
    return sda.Cache(torch.from_numpy(c.data).to(device), c.num_pages, c.page_size, c.page_stride, c.fmt,
                     None if c.slot_scale is None else torch.from_numpy(c.slot_scale).to(device))


def dev_list(L, device="cuda"):
    return sda.SlotList(torch.from_numpy(np.ascontiguousarray(L.idx)).to(device), L.width,
                        None if L.lens is None else torch.from_numpy(L.lens).to(device),
                        getattr(L, "queries_per_len", 1))


def dev_q(w, device="cuda"):
    return torch.from_numpy(w.q.view(np.int16)).to(device).view(torch.bfloat16)


class DeviceWorkload:
    def __init__(self, w, device="cuda"):
        self.w = w
        self.q = dev_q(w, device)
        self.cache = dev_cache(w.cache, device)
        self.lst = dev_list(w.lst, device)
        self.xcache = dev_cache(w.xcache, device) if w.xcache is not None else None
        self.xlst = dev_list(w.xlst, device) if w.xlst is not None else None
        self.sink = torch.from_numpy(w.sink).to(device) if w.sink is not None else None

    def run(self, plan=None, sink="default", q=None, out=None, lse=None):
        w = self.w
        dec = sda.Decoder(w.T, w.H, w.d_qk, w.lst.width, w.xlst.width if w.xlst is not None else 0,
                          device=self.q.device, plan=plan)
        snk = self.sink if isinstance(sink, str) else sink
        o, l = dec(self.q if q is None else q, self.cache, self.lst, self.xcache, self.xlst, snk, w.scale,
                   out=out, lse=lse)
        torch.cuda.synchronize()
        return o, l, dec


def compare(out_gpu, lse_gpu, o_ref, l_ref, tokens=None, what="", count_flips=True):
    """Assert the tolerances; returns a dict of the error figures.

    out: every element within 1e-2 of the round-to-nearest-even bf16 of the fp64 oracle, except that an
    element may sit one bf16 ulp away where that ulp itself exceeds 1e-2 (|x| >= 2): a rounding-boundary
    flip, which an fp32 computation produces whenever the exact value lies within its rounding error of
    a bf16 midpoint. Flips are counted and must stay below 1 in 10^4 elements (count_flips=False lifts
    that count for the single-term P mode, whose 2^-9 weight rounding flips more of them). rel-L2 <=
    5e-3 over all elements. lse: within 1e-3 absolute, infinities exact."""
    got = out_gpu.float().cpu().numpy().astype(np.float64)
    lg = lse_gpu.float().cpu().numpy().astype(np.float64)
    if tokens is not None:
        got, lg = got[tokens], lg[tokens]
    ref = oracle.bf16_rne(o_ref)
    diff = np.abs(got - ref)
    max_abs = float(diff.max()) if diff.size else 0.0
    nrm = float(np.linalg.norm(ref))
    rel_l2 = float(np.linalg.norm(got - ref) / nrm) if nrm > 0 else float(np.linalg.norm(got))
    inf_ref = ~np.isfinite(l_ref)
    assert np.array_equal(inf_ref, ~np.isfinite(lg)), f"{what}: LSE infinities differ"
    assert np.array_equal(l_ref[inf_ref], lg[inf_ref]), f"{what}: LSE infinity signs differ"
    lse_err = float(np.abs(lg[~inf_ref] - l_ref[~inf_ref]).max()) if (~inf_ref).any() else 0.0
    over = diff > OUT_MAX_ABS
    ulp = np.ldexp(1.0, np.frexp(np.abs(ref))[1] - 8)  # bf16 spacing at |ref|
    info = dict(max_abs=max_abs, rel_l2=rel_l2, lse_max_abs=lse_err, ulp_flips=int(over.sum()), n=int(diff.size))
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert np.all(diff[over] <= ulp[over]), f"{what}: error beyond 1e-2 and beyond one bf16 ulp {info}"
    if count_flips:
        assert info["ulp_flips"] <= max(1, diff.size // 10000), f"{what}: too many rounding flips {info}"
    assert rel_l2 <= OUT_REL_L2, f"{what}: out rel-L2 {rel_l2:.3e} {info}"
    assert lse_err <= LSE_MAX_ABS, f"{what}: lse max-abs {lse_err:.3e} {info}"
    return info
