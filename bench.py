"""Benchmark of the decode-attention hot path on one MI355X.

A step is the whole op on one batch of synthetic, seeded inputs already resident in HBM: the library's plan
(sda_choose_plan from the host-side lengths), then the scheduler, the decode kernel and the LSE combine for a
split plan, or the decode kernel alone for a whole-token plan. The headline (default) workload is the top-k
configuration: 128 decode tokens x 128 heads, d_qk 576 / d_v 512, 656-byte V3.2 records in a 131072-slot
paged cache, 2048 slots per token, sink on. It is timed on cold buffers: enough independent copies of q,
the cache, the slot lists and the outputs are rotated that their total exceeds twice the 256 MB MALL, so
every call reads from HBM. The timed region is exactly --steps back-to-back steps between two
synchronizations, bracketed by HIP events on the launch stream; with the whole-token plan the library picks
for it a step is one launch of the decode kernel, so the region also gives that kernel's mean duration for
the roofline (split plans: the decode kernel is timed the same way over its own back-to-back launches).

Prints one JSON line: query-tokens/s (value), the roofline position of the decode kernel and of the whole
step, per-configuration results for the five benchmark configurations (hot and cold; the top-k one on both
its whole-token plan and its split-KV + combine plan), and the CPU oracle's throughput on a bounded sample
of the headline workload (all available host cores, and one thread).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
KERNEL_SRCS = [os.path.join(ROOT, "sliding_window_decode_amd", "csrc", f)
               for f in ("sda_decode_ring.hip", "sda_decode_wide.hip", "sda_decode_staged.hip", "sda_items.h", "sda_sched.hip", "sda_device.h",
                         "sda_internal.h", "sda_v41.hip")]
CALIB_BYTES = 256 << 20        # the plain copy that calibrates the HBM byte counters
COLD_BYTES = 600e6             # rotated buffer sets exceed twice the MALL
RAMP_S = 0.3                   # untimed steps before the headline's warmup, for the clocks to settle
HEADLINE = "c5_topk_v32"
BENCH_CONFIGS = ("c1_tiny_swa", "c2_swa_h128", "c3_swa_fp8extra", "c4_swa_nvfp4extra", "c5_topk_v32")
BOX_CPU_SHARE = 16             # host CPUs a one-GPU machine allots to a job


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_work(w):
    """Bytes and FLOPs the method needs: Q, the valid rows' records (+ the fp32 slot scale), the list
    entries read (positions below the length), out and lse (V4.1: fp8 out with its scale bytes, plus each
    token's position and cos/sin row). Masked rows, padding and split partials are not counted."""
    rows = 0
    if getattr(w, "rope", None) is not None:
        byts = w.T * w.H * w.d_qk * 2 + w.T * w.H * (w.d_v + w.d_v // 32) + w.T * w.H * 4 + w.T * (8 + 64 * 4)
    else:
        byts = w.T * w.H * w.d_qk * 2 + w.T * w.H * w.d_v * 2 + w.T * w.H * 4
    for cache, L in w.lists():
        qpl = max(1, getattr(L, "queries_per_len", 1))
        n = np.clip(L.lens[np.arange(w.T) // qpl], 0, L.width) if L.lens is not None else np.full(w.T, L.width)
        for t in range(w.T):
            sids = L.idx[t, :n[t]]
            valid = int(((sids >= 0) & (sids < cache.num_slots)).sum())
            rows += valid
            byts += valid * (cache.record_bytes + (4 if cache.fmt == wl.FP8_SLOTSCALE else 0)) + int(n[t]) * 4
    flops = rows * 2 * w.H * (w.d_qk + w.d_v)
    return byts, flops, rows


def kernel_sha() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(workload: str, sha: str):
    """HBM bytes per decode launch from the committed rocprofv3 counter summary, if it was taken on
    the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_decode_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_sha") != sha:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _pmc_rows(path_dir):
    """(kernel name, counter name, value) rows of every rocprofv3 counter-collection CSV under a dir."""
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(path_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                rows.append((r.get("Kernel_Name", ""), r.get("Counter_Name", ""), float(r.get("Counter_Value", "nan"))))
    return rows


def summarize_pmc(fetch_dir: str, write_dir: str, workload: str, command: str):
    """Turns the two counter passes (FETCH_SIZE, WRITE_SIZE; KiB per dispatch) over a bench run with
    --copy-calib into profiles/traffic_decode_<workload>.txt: the decode kernel's mean counters per
    launch, each divided by what the same counter reads per byte of the calibration copy."""
    w = wl.make_workload(workload, seed=0)
    alg_bytes, _, _ = algorithmic_work(w)
    out = {}
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _pmc_rows(d) if r[1] == name]
        dec = [v for k, _, v in rows if "decode" in k and "kernel" in k]
        cal = [v for k, _, v in rows if "elementwise" in k.lower() and "mul" in k.lower()]
        if not dec or not cal:
            raise SystemExit(f"no decode or calibration dispatches with {name} under {d}")
        dec_names = sorted({k for k, _, _ in rows if "decode" in k and "kernel" in k})
        out[name] = (sum(dec) / len(dec), sum(cal) / len(cal), len(dec), dec_names)
    f_kib, f_cal, n_f, names = out["FETCH_SIZE"]
    w_kib, w_cal, n_w, _ = out["WRITE_SIZE"]
    f_factor = f_cal * 1024.0 / CALIB_BYTES
    w_factor = w_cal * 1024.0 / CALIB_BYTES
    hbm = f_kib * 1024.0 / f_factor + w_kib * 1024.0 / w_factor
    path = os.path.join(ROOT, "profiles", f"traffic_decode_{workload}.txt")
    with open(path, "w") as fh:
        fh.write(f"# L2 <-> fabric traffic of the decode kernel, {workload}: rocprofv3 --pmc, one pass per counter\n")
        fh.write(f"# command: {command}\n")
        fh.write("# the calibration is an elementwise copy (x * 1) of 256 MiB in the same process\n")
        fh.write(f"kernel = {' / '.join(n.split('(')[0] for n in names)}\n")
        fh.write(f"kernel_sha = {kernel_sha()}\n")
        fh.write(f"decode_dispatches = {n_f} / {n_w}\n")
        fh.write(f"fetch_kib_per_launch = {f_kib:.1f}\n")
        fh.write(f"write_kib_per_launch = {w_kib:.1f}\n")
        fh.write(f"copy_fetch_factor = {f_factor:.4f}\n")
        fh.write(f"copy_write_factor = {w_factor:.4f}\n")
        fh.write(f"hbm_bytes_per_launch = {hbm:.0f}\n")
        fh.write(f"alg_bytes_per_launch = {alg_bytes}\n")
        fh.write(f"traffic_over_alg = {hbm / alg_bytes:.3f}\n")
    print(open(path).read())


def host_cores() -> int:
    """Host CPUs this process may use (its affinity set; a one-GPU machine allots BOX_CPU_SHARE of them)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, BOX_CPU_SHARE))


def _oracle_rate(w, tokens: int, threads: int, seconds: float):
    import oracle
    sl = slice(0, tokens)
    t0 = time.perf_counter()
    oracle.attention(w, tokens=sl, nthreads=threads)
    done, el = 1, time.perf_counter() - t0
    while el < seconds:
        oracle.attention(w, tokens=sl, nthreads=threads)
        done += 1
        el = time.perf_counter() - t0
    return done * tokens / el, done, el


def cpu_baseline(w):
    """The fp64 oracle as it stands on a bounded sample of workload w's tokens: on every available host core,
    then on one thread (about 10 s and 5 s of CPU work)."""
    threads = host_cores()
    n_all = min(w.T, max(1, 2 * threads))
    v_all, d_all, e_all = _oracle_rate(w, n_all, threads, 10.0)
    n_one = 1
    v_one, d_one, e_one = _oracle_rate(w, n_one, 1, 5.0)
    return {"value": round(v_all, 2), "unit": "query-tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"tokens 0..{n_all - 1} of {w.T} of the workload, {d_all} passes, fp64, {e_all:.1f} s on "
                      f"{threads} threads",
            "single_thread": {"value": round(v_one, 3), "unit": "query-tokens/s", "cores": 1,
                              "sample": f"token 0, {d_one} passes, {e_one:.1f} s"}}


def roofline(byts, flops, t):
    """Position of a duration t (s) against both roofs; the bound is the roof the algorithmic work hits first."""
    hbm = byts / t / 1e9
    tfl = flops / t / 1e12
    bound = "hbm" if byts / (HBM_PEAK_GBS * 1e9) >= flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) else "mfma"
    if bound == "hbm":
        r = {"bound": "hbm", "achieved": round(hbm, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(hbm / HBM_PEAK_GBS, 4)}
    else:
        r = {"bound": "mfma", "achieved": round(tfl, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
             "frac": round(tfl / MFMA_BF16_PEAK_TFLOPS, 4)}
    r["hbm_frac"] = round(hbm / HBM_PEAK_GBS, 4)
    r["mfma_frac"] = round(tfl / MFMA_BF16_PEAK_TFLOPS, 4)
    return r


class Runner:
    """Device inputs and launch plumbing of one workload under one plan. The step is the whole op: for a
    whole-token plan one launch of the decode kernel, for a split plan the scheduler, the decode kernel and the
    combine (the launches sda_sparse_decode_attn makes). Arguments are marshalled once per buffer set, so
    the host enqueues a step in a few microseconds."""

    def __init__(self, w, dw, plan):
        import torch

        import sliding_window_decode_amd as sda
        self.sda, self.torch = sda, torch
        self.w, self.dw, self.plan = w, dw, plan
        self.dec = dw.decoder(plan)
        self.v41 = getattr(w, "rope", None) is not None
        dev = dw.q.device
        self.out = torch.empty((w.T, w.H, 512), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((w.T, w.H), dtype=torch.float32, device=dev)
        if self.v41:
            self.out8 = torch.empty((w.T, w.H, 512), dtype=torch.uint8, device=dev)
            self.osc = torch.empty((w.T, w.H, 16), dtype=torch.uint8, device=dev)
        S = w.T + plan.num_parts
        off = sda.workspace_lse_offset(w.T, w.H, 512, plan)
        ws = self.dec.workspace
        self.o_acc = ws[:S * w.H * 512 * 4].view(torch.float32).view(S, w.H, 512)
        self.lse_acc = ws[off:off + S * w.H * 4].view(torch.float32).view(S, w.H)
        self.set_buffers([(dw.q, dw.cache, dw.lst, dw.xcache, dw.xlst, self.out, self.lse)])

    def set_buffers(self, sets):
        self.sets = sets
        self.calls = [self._prepare(st) for st in sets]

    def _prepare(self, st):
        """(the step's launches, the decode-kernel launch alone) for one buffer set."""
        sda, w, plan, dec, dw = self.sda, self.w, self.plan, self.dec, self.dw
        q, c, L, xc, xL, out, lse = st
        meta, ns = dec.sched_arrays
        sched = [] if plan.whole_tokens else [sda.prepare_get_sched_meta(w.T, L, xL, plan, meta, ns)]
        if self.v41:  # Q RoPE, decode, combine with the inverse RoPE and the MXFP8 cast (one call)
            def v41_call():
                sda.sparse_decode_attn_v41(q, c, L, xc, xL, dw.sink, w.scale, plan, meta, ns, dec.workspace,
                                           dw.positions, dw.cos_sin, self.out8, self.osc, lse)
            decode = sda.prepare_decode_splits(q, c, L, xc, xL, dw.sink, w.scale, plan, meta, ns, dec.workspace,
                                               None, None)
            return sched + [v41_call], decode
        if plan.whole_tokens:  # one launch: the decode kernel writes every token whole
            call = sda.prepare_sparse_decode_attn(q, c, L, xc, xL, dw.sink, w.scale, plan, None, None, dec.workspace,
                                                  out, lse)
            return [call], call
        decode = sda.prepare_decode_splits(q, c, L, xc, xL, dw.sink, w.scale, plan, meta, ns, dec.workspace, out,
                                           lse)
        combine = sda.prepare_combine_splits(self.o_acc, self.lse_acc, ns, dw.sink, out, lse)
        return sched + [decode, combine], decode

    def make_cold_sets(self):
        """Independent copies of q, the caches, the slot lists and the outputs, rotated by the steps so that
        their total exceeds twice the MALL and each call reads from HBM."""
        sda, torch, dw = self.sda, self.torch, self.dw

        def cache_copy(c):
            if c is None:
                return None
            return sda.Cache(c.data.clone(), c.num_pages, c.page_size, c.page_stride, c.format,
                             None if c.slot_scale is None else c.slot_scale.clone())

        def list_copy(L):
            if L is None:
                return None
            return sda.SlotList(L.idx.clone(), L.width, None if L.lens is None else L.lens.clone(), L.queries_per_len)

        per_set = (dw.q.numel() * 2 + self.out.numel() * 2 + dw.cache.data.numel() + dw.lst.idx.numel() * 4 +
                   (dw.xcache.data.numel() + dw.xlst.idx.numel() * 4 if dw.xcache is not None else 0))
        nsets = min(64, max(2, int(math.ceil(COLD_BYTES / per_set))))
        self.set_buffers([(dw.q.clone(), cache_copy(dw.cache), list_copy(dw.lst), cache_copy(dw.xcache),
                           list_copy(dw.xlst), torch.empty_like(self.out), torch.empty_like(self.lse))
                          for _ in range(nsets)])
        return nsets, per_set

    def ramp(self, seconds):
        """Untimed steps for about `seconds` of wall time before anything is timed, so that the GPU's clocks and
        power state have settled (the first tens of milliseconds after an idle period run measurably slower)."""
        torch = self.torch
        n = len(self.calls)
        t0 = time.perf_counter()
        i = 0
        while time.perf_counter() - t0 < seconds:
            for _ in range(32):
                for f in self.calls[i % n][0]:
                    f()
                i += 1
            torch.cuda.synchronize()
        return i

    def time(self, steps, warmup):
        """(mean step, mean decode-kernel duration, host enqueue time per step), all in ms. The step is timed
        over exactly `steps` back-to-back steps between two synchronizations, with HIP events on the launch
        stream bracketing them; the decode kernel is the step itself for a whole-token plan (one launch), and
        otherwise timed the same way over `steps` back-to-back decode-kernel launches."""
        torch = self.torch
        n = len(self.calls)
        for i in range(warmup):
            for f in self.calls[i % n][0]:
                f()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        h0 = time.perf_counter()
        e0.record()
        for i in range(steps):
            for f in self.calls[i % n][0]:
                f()
        e1.record()
        h1 = time.perf_counter()
        torch.cuda.synchronize()
        step = e0.elapsed_time(e1) / steps
        host = (h1 - h0) * 1e3 / steps
        if self.plan.whole_tokens and not self.v41:
            return step, step, host
        for i in range(min(warmup, 5)):
            self.calls[i % n][1]()
        torch.cuda.synchronize()
        e0.record()
        for i in range(steps):
            self.calls[i % n][1]()
        e1.record()
        torch.cuda.synchronize()
        return step, e0.elapsed_time(e1) / steps, host


def plan_dict(plan):
    return {"num_parts": plan.num_parts, "heads_per_group": plan.heads_per_group,
            "fixed_overhead": plan.fixed_overhead, "precision": plan.precision,
            "whole_tokens": bool(plan.whole_tokens)}


def measure(w, dw, plan, steps, warmup, cold=True, ramp=0.05):
    """Hot and (optionally) cold timings of one workload under one plan, with rooflines of the whole step
    and of the decode kernel."""
    byts, flops, rows = algorithmic_work(w)
    r = Runner(w, dw, plan)
    if ramp > 0:
        r.ramp(ramp)
    st_h, k_h, ho_h = r.time(steps, warmup)
    res = {"plan": plan_dict(plan), "alg_bytes": byts, "alg_flops": flops, "valid_rows": rows,
           "hot": {"step_us": round(st_h * 1e3, 2), "kernel_us": round(k_h * 1e3, 2),
                   "host_enqueue_us": round(ho_h * 1e3, 2), "query_tokens_per_s": round(w.T / (st_h / 1e3), 1),
                   "roofline_step": roofline(byts, flops, st_h / 1e3),
                   "roofline_kernel": roofline(byts, flops, k_h / 1e3)}}
    if cold:
        nsets, per_set = r.make_cold_sets()
        st_c, k_c, ho_c = r.time(steps, max(warmup, nsets))
        res["cold"] = {"step_us": round(st_c * 1e3, 2), "kernel_us": round(k_c * 1e3, 2),
                       "host_enqueue_us": round(ho_c * 1e3, 2), "query_tokens_per_s": round(w.T / (st_c / 1e3), 1),
                       "tflops": round(flops / (st_c / 1e3) / 1e12, 2), "gbps": round(byts / (st_c / 1e3) / 1e9, 1),
                       "roofline_step": roofline(byts, flops, st_c / 1e3),
                       "roofline_kernel": roofline(byts, flops, k_c / 1e3),
                       "buffer_sets": nsets, "set_mb": round(per_set / 1e6, 1)}
        r.set_buffers(r.sets[:1])
    return res, r


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE, choices=wl.CONFIGS, help="the headline workload")
    ap.add_argument("--configs", default=",".join(BENCH_CONFIGS),
                    help="comma-separated workloads reported per configuration ('none': headline only)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--precision", type=int, default=None, help="override the plan's PV precision (1, 2 or 3)")
    ap.add_argument("--parts", type=int, default=None)
    ap.add_argument("--heads-per-group", type=int, default=None)
    ap.add_argument("--fixed-overhead", type=int, default=None, help="override the plan's per-token tile overhead")
    ap.add_argument("--schedule", choices=["auto", "split", "whole"], default="auto",
                    help="auto: the library's choice (sda_choose_plan); split: scheduler + combine; whole: one "
                         "workgroup per token")
    ap.add_argument("--hot", action="store_true", help="headline on hot buffers (the same buffers every call)")
    ap.add_argument("--ramp", type=float, default=RAMP_S,
                    help="seconds of untimed steps before the headline's warmup (0 under a profiler)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a plain 256 MiB elementwise copy (calibrates the counter-based traffic)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic_decode_<workload>.txt from two rocprofv3 --pmc output dirs")
    ap.add_argument("--pmc-command", default="", help="the profiling command, recorded in the summary")
    args = ap.parse_args()

    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.workload, args.pmc_command)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import sliding_window_decode_amd as sda
    from sliding_window_decode_amd.inputs import DeviceWorkload, plan_for

    def headline_plan(w):
        plan = plan_for(w)
        if args.schedule == "split" or (args.schedule == "whole" and not plan.whole_tokens):
            X = w.xlst.width if w.xlst is not None else 0
            plan = sda.make_plan(w.T, w.H, w.d_qk, w.lst.width, X)
            plan.whole_tokens = 1 if args.schedule == "whole" else 0
        if args.precision is not None:
            plan.precision = args.precision
        if args.parts is not None:
            plan.num_parts = args.parts
        if args.heads_per_group is not None:
            plan.heads_per_group = args.heads_per_group
        if args.fixed_overhead is not None:
            plan.fixed_overhead = args.fixed_overhead
        return plan

    log(f"[bench] building {args.workload} seed {args.seed}")
    w = wl.make_workload(args.workload, seed=args.seed)
    dw = DeviceWorkload(w)
    plan = headline_plan(w)
    log(f"[bench] headline {args.workload}: plan {plan}; {args.steps} steps after {args.warmup} warmup")
    byts, flops, rows = algorithmic_work(w)
    r = Runner(w, dw, plan)
    if not args.hot:
        nsets, per_set = r.make_cold_sets()
        log(f"[bench] cold: {nsets} buffer sets of {per_set / 1e6:.1f} MB")
    ramp_steps = r.ramp(args.ramp) if args.ramp > 0 else 0
    log(f"[bench] clock ramp: {ramp_steps} untimed steps in {args.ramp:.2f} s")
    ms_step, ms_kern, ms_host = r.time(args.steps, max(args.warmup, len(r.sets)))
    log(f"[bench] step {ms_step * 1e3:.2f} us, decode kernel {ms_kern * 1e3:.2f} us, host enqueue "
        f"{ms_host * 1e3:.2f} us per step")
    t_step, t_kern = ms_step / 1e3, ms_kern / 1e3
    sha = kernel_sha()
    roof = roofline(byts, flops, t_kern)
    roof_k = {k: roof[k] for k in ("bound", "achieved", "peak", "unit", "frac")}
    roof_k["traffic"] = read_traffic(args.workload, sha)
    X = w.xlst.width if w.xlst is not None else 0
    result = {
        "metric": "decode-attn query-tokens/s, TFLOP/s and HBM GB/s vs roofline, per head count",
        "value": round(w.T / t_step, 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_ramp_steps": ramp_steps,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "buffers": "hot" if args.hot else "cold", "tokens": w.T, "heads": w.H,
                   "d_qk": w.d_qk, "d_v": w.d_v, "list_width": w.lst.width, "extra_width": X,
                   "format": wl.FORMAT_NAMES[w.cache.fmt],
                   "extra_format": wl.FORMAT_NAMES[w.xcache.fmt] if w.xcache is not None else None,
                   "sink": w.sink is not None, "valid_rows": rows,
                   "v41_rope_mxfp8_out": getattr(w, "rope", None) is not None, "plan": plan_dict(plan)},
        "tflops": round(flops / t_step / 1e12, 2),
        "gbps": round(byts / t_step / 1e9, 1),
        "decode_kernel_us": round(ms_kern * 1e3, 2),
        "host_enqueue_us": round(ms_host * 1e3, 2),
        "roofline": roof_k,
        "roofline_step": roofline(byts, flops, t_step),
        "alg_bytes": byts,
        "alg_flops": flops,
        "kernel_sha": sha,
    }
    del r

    configs = [c for c in args.configs.split(",") if c and c != "none"]
    per = {}
    for name in configs:
        log(f"[bench] config {name}")
        wc = w if (name == args.workload and args.seed == 0) else wl.make_workload(name, seed=0)
        dwc = dw if wc is w else DeviceWorkload(wc)
        pc = plan_for(wc)
        if args.precision is not None:
            pc.precision = args.precision
        res, _ = measure(wc, dwc, pc, args.steps, args.warmup, ramp=min(args.ramp, 0.05))
        entry = {"heads": wc.H, "tokens": wc.T, **res}
        if name == HEADLINE and pc.whole_tokens:
            # the plan the configuration names: split-KV sized to 256 CUs + combine
            sp = sda.make_plan(wc.T, wc.H, wc.d_qk, wc.lst.width, wc.xlst.width if wc.xlst is not None else 0)
            sp.precision = pc.precision
            entry["split_plan"], _ = measure(wc, dwc, sp, args.steps, args.warmup, ramp=min(args.ramp, 0.05))
        per[name] = entry
        log(f"[bench]   {name}: hot {res['hot']['step_us']} us, cold {res['cold']['step_us']} us")
        if dwc is not dw:
            del dwc
        torch.cuda.empty_cache()
    if per:
        result["configs"] = per

    if args.copy_calib:
        src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    if not args.no_cpu:
        log("[bench] CPU oracle baseline")
        result["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
