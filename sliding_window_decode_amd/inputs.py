"""Device-resident copies of the synthetic workloads (workloads.py) for the benchmark and the GPU tests:
the host arrays are copied into torch device tensors and wrapped in the binding's Cache / SlotList
descriptors. Nothing here computes any part of the method."""
from __future__ import annotations

import numpy as np

from . import Cache, Decoder, SlotList, auto_plan


def dev_cache(c, device="cuda"):
    import torch
    return Cache(torch.from_numpy(c.data).to(device), c.num_pages, c.page_size, c.page_stride, c.fmt,
                 None if c.slot_scale is None else torch.from_numpy(c.slot_scale).to(device))


def dev_list(L, device="cuda"):
    import torch
    return SlotList(torch.from_numpy(np.ascontiguousarray(L.idx)).to(device), L.width,
                    None if L.lens is None else torch.from_numpy(L.lens).to(device),
                    getattr(L, "queries_per_len", 1))


def dev_q(w, device="cuda"):
    import torch
    return torch.from_numpy(w.q.view(np.int16)).to(device).view(torch.bfloat16)


def plan_for(w, num_cus: int = 256):
    """The library's plan (sda_choose_plan) for workload w, from its host-side lengths."""
    X = w.xlst.width if w.xlst is not None else 0
    return auto_plan(w.T, w.H, w.d_qk, w.lst.width, X, w.lst.lens, w.xlst.lens if w.xlst is not None else None,
                     [w.cache.fmt, w.xcache.fmt if w.xcache is not None else None], getattr(w, "rope", None) is not None,
                     max(1, getattr(w.lst, "queries_per_len", 1)), num_cus)


class DeviceWorkload:
    """Workload w's inputs in device memory, with helpers that run the plain and the V4.1 call."""

    def __init__(self, w, device="cuda"):
        import torch
        self.w = w
        self.q = dev_q(w, device)
        self.cache = dev_cache(w.cache, device)
        self.lst = dev_list(w.lst, device)
        self.xcache = dev_cache(w.xcache, device) if w.xcache is not None else None
        self.xlst = dev_list(w.xlst, device) if w.xlst is not None else None
        self.sink = torch.from_numpy(w.sink).to(device) if w.sink is not None else None
        rope = getattr(w, "rope", None)
        self.positions = torch.from_numpy(rope.positions).to(device) if rope is not None else None
        self.cos_sin = torch.from_numpy(rope.cos_sin).to(device) if rope is not None else None

    def decoder(self, plan=None):
        w = self.w
        return Decoder(w.T, w.H, w.d_qk, w.lst.width, w.xlst.width if w.xlst is not None else 0,
                       device=self.q.device, plan=plan)

    def run(self, plan=None, sink="default", q=None, out=None, lse=None):
        """The plain call (scheduler, decode, combine as the plan says); returns (out, lse, decoder)."""
        import torch
        w = self.w
        dec = self.decoder(plan)
        snk = self.sink if isinstance(sink, str) else sink
        o, l = dec(self.q if q is None else q, self.cache, self.lst, self.xcache, self.xlst, snk, w.scale,
                   out=out, lse=lse)
        torch.cuda.synchronize()
        return o, l, dec

    def run_v41(self, plan=None):
        """The V4.1 call: returns (codes, scale bytes, lse, decoder)."""
        import torch
        w = self.w
        dec = self.decoder(plan)
        c, s, l = dec.v41(self.q, self.cache, self.lst, self.xcache, self.xlst, self.sink, w.scale, self.positions,
                          self.cos_sin)
        torch.cuda.synchronize()
        return c, s, l, dec
