"""Benchmark of one decode-attention step on one MI355X.

A step is the whole hot path on one batch of synthetic, seeded inputs already resident in HBM:
the device scheduler (sda_get_sched_meta), the split-KV decode kernel and the LSE combine
(sda_sparse_decode_attn). Default workload: 64 decode tokens x 128 heads, d 512, a 4096-slot paged
fp8 cache with per-slot scales, window 128, lens U{96..128}.

Prints one JSON line with query-tokens/s (value), TFLOP/s and GB/s of algorithmic work, the
roofline position of the decode kernel (timed alone with HIP events on the same stream) and the
CPU oracle's throughput on a bounded sample of the same workload.
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
               for f in ("sda_decode_ring.hip", "sda_decode_staged.hip", "sda_items.h", "sda_sched.hip", "sda_device.h",
                         "sda_internal.h", "sda_v41.hip")]
CALIB_BYTES = 256 << 20        # the plain copy that calibrates the HBM byte counters


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


def cpu_baseline(w, max_seconds: float = 20.0):
    import oracle
    threads = max(1, min(os.cpu_count() or 1, 16))
    t0 = time.perf_counter()
    oracle.attention(w, nthreads=threads)
    one = time.perf_counter() - t0
    passes = max(1, int(10.0 / max(one, 1e-3)))
    t0 = time.perf_counter()
    done = 0
    while done < passes and time.perf_counter() - t0 < max_seconds:
        oracle.attention(w, nthreads=threads)
        done += 1
    el = time.perf_counter() - t0
    return {"value": done * w.T / el, "unit": "query-tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"the full workload ({w.T} tokens) {done} times, fp64, {el:.1f} s on {threads} threads"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c2_swa_h128", choices=wl.CONFIGS)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--precision", type=int, default=None, help="override the plan's PV precision (1 or 3)")
    ap.add_argument("--parts", type=int, default=None)
    ap.add_argument("--heads-per-group", type=int, default=None)
    ap.add_argument("--fixed-overhead", type=int, default=None, help="override the plan's per-token tile overhead")
    ap.add_argument("--schedule", choices=["auto", "split", "whole"], default="auto",
                    help="split: scheduler + combine; whole: one workgroup per token; auto: whole when its "
                         "makespan in tiles (host-side lengths) is close enough to the split plan's")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cold", action="store_true", help="also time with rotating buffer sets larger than the MALL")
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
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from gpu_util import DeviceWorkload, auto_plan_for

    log(f"[bench] building {args.workload} seed {args.seed}")
    w = wl.make_workload(args.workload, seed=args.seed)
    dw = DeviceWorkload(w)
    X = w.xlst.width if w.xlst is not None else 0
    # the caller's host-side lengths decide between the split schedule and one workgroup per token
    fmts = [w.cache.fmt, w.xcache.fmt if w.xcache is not None else None]
    if args.schedule == "auto":
        plan = auto_plan_for(w)
    else:
        plan = sda.make_plan(w.T, w.H, w.d_qk, w.lst.width, X)
        if args.schedule == "whole":
            plan.whole_tokens = 1
            plan.heads_per_group = sda.whole_token_heads_per_group(plan, w.T, w.H, w.d_qk, fmts)
    if args.precision is not None:
        plan.precision = args.precision
    if args.parts is not None:
        plan.num_parts = args.parts
    if args.heads_per_group is not None:
        plan.heads_per_group = args.heads_per_group
    if args.fixed_overhead is not None:
        plan.fixed_overhead = args.fixed_overhead
    dec = sda.Decoder(w.T, w.H, w.d_qk, w.lst.width, X, plan=plan)
    out = torch.empty((w.T, w.H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.T, w.H), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    v41 = w.rope is not None
    if v41:
        out8 = torch.empty((w.T, w.H, 512), dtype=torch.uint8, device="cuda")
        osc = torch.empty((w.T, w.H, 16), dtype=torch.uint8, device="cuda")

    meta, num_splits = dec.sched_arrays  # None for a whole-token plan

    def step():
        dec.schedule(dw.lst, dw.xlst)  # nothing for a whole-token plan
        if v41:  # Q RoPE, decode, combine with the inverse RoPE and MXFP8 cast
            sda.sparse_decode_attn_v41(dw.q, dw.cache, dw.lst, dw.xcache, dw.xlst, dw.sink, w.scale, dec.plan,
                                       meta, num_splits, dec.workspace, dw.positions, dw.cos_sin, out8, osc, lse)
        else:
            sda.sparse_decode_attn(dw.q, dw.cache, dw.lst, dw.xcache, dw.xlst, dw.sink, w.scale, dec.plan,
                                   meta, num_splits, dec.workspace, out, lse)

    log(f"[bench] plan {plan}; warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    log(f"[bench] step {ms_step * 1e3:.2f} us")

    # the decode kernel alone, back to back on the same stream, launched as in the step (V4.1: every token
    # leaves as a partial; the rotation of q changes values, not work)
    def decode_only():
        sda.decode_splits(dw.q, dw.cache, dw.lst, dw.xcache, dw.xlst, dw.sink, w.scale, dec.plan, meta,
                          num_splits, dec.workspace, None if v41 else out, None if v41 else lse)

    for _ in range(max(5, args.warmup // 2)):
        decode_only()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        decode_only()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_decode = e0.elapsed_time(e1) / args.steps
    log(f"[bench] decode kernel {ms_decode * 1e3:.2f} us")

    byts, flops, rows = algorithmic_work(w)
    t_step = ms_step / 1e3
    t_dec = ms_decode / 1e3
    gbs_dec = byts / t_dec / 1e9
    tfl_dec = flops / t_dec / 1e12
    hbm_frac = gbs_dec / HBM_PEAK_GBS
    mfma_frac = tfl_dec / MFMA_BF16_PEAK_TFLOPS
    bound = "hbm" if byts / (HBM_PEAK_GBS * 1e9) >= flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) else "mfma"
    sha = kernel_sha()
    traffic = read_traffic(args.workload, sha)
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": round(gbs_dec, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(hbm_frac, 4), "traffic": traffic}
    else:
        roof = {"bound": "mfma", "achieved": round(tfl_dec, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(mfma_frac, 4), "traffic": traffic}

    result = {
        "metric": "decode-attn query-tokens/s, TFLOP/s and HBM GB/s vs roofline, per head count",
        "value": round(w.T / t_step, 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "tokens": w.T, "heads": w.H, "d_qk": w.d_qk, "d_v": w.d_v,
                   "list_width": w.lst.width, "extra_width": X,
                   "format": wl.FORMAT_NAMES[w.cache.fmt],
                   "extra_format": wl.FORMAT_NAMES[w.xcache.fmt] if w.xcache is not None else None,
                   "sink": w.sink is not None, "valid_rows": rows, "v41_rope_mxfp8_out": v41,
                   "plan": {"num_parts": plan.num_parts, "heads_per_group": plan.heads_per_group,
                            "fixed_overhead": plan.fixed_overhead, "precision": plan.precision,
                            "whole_tokens": bool(plan.whole_tokens)}},
        "tflops": round(flops / t_step / 1e12, 2),
        "gbps": round(byts / t_step / 1e9, 1),
        "decode_kernel_us": round(ms_decode * 1e3, 2),
        "roofline": roof,
        "roofline_both": {"hbm_frac": round(hbm_frac, 4), "mfma_frac": round(mfma_frac, 4),
                          "alg_bytes": byts, "alg_flops": flops},
        "kernel_sha": sha,
    }

    if args.cold:
        # rotate independent copies of q, cache, lists and out so that the working set exceeds the MALL
        per_set = dw.q.numel() * 2 + out.numel() * 2 + dw.cache.data.numel() + (
            dw.xcache.data.numel() if dw.xcache is not None else 0)
        nsets = max(2, int(math.ceil(600e6 / per_set)))
        nsets = min(nsets, 64)
        log(f"[bench] cold: {nsets} buffer sets of {per_set / 1e6:.1f} MB")
        sets = []
        for _ in range(nsets):
            c = sda.Cache(dw.cache.data.clone(), dw.cache.num_pages, dw.cache.page_size, dw.cache.page_stride,
                          dw.cache.format, None if dw.cache.slot_scale is None else dw.cache.slot_scale.clone())
            xc = None
            if dw.xcache is not None:
                xc = sda.Cache(dw.xcache.data.clone(), dw.xcache.num_pages, dw.xcache.page_size,
                               dw.xcache.page_stride, dw.xcache.format, None)
            sets.append((dw.q.clone(), c, xc, torch.empty_like(out), torch.empty_like(lse)))
        for i in range(nsets):
            q_, c_, xc_, o_, l_ = sets[i]
            sda.sparse_decode_attn(q_, c_, dw.lst, xc_, dw.xlst, dw.sink, w.scale, dec.plan, meta,
                                   num_splits, dec.workspace, o_, l_)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(args.steps):
            q_, c_, xc_, o_, l_ = sets[i % nsets]
            dec.schedule(dw.lst, dw.xlst)
            sda.sparse_decode_attn(q_, c_, dw.lst, xc_, dw.xlst, dw.sink, w.scale, dec.plan, meta,
                                   num_splits, dec.workspace, o_, l_)
        e1.record(stream)
        torch.cuda.synchronize()
        ms_cold = e0.elapsed_time(e1) / args.steps
        result["cold"] = {"ms_per_step": round(ms_cold, 5), "value": round(w.T / (ms_cold / 1e3), 1),
                          "buffer_sets": nsets}
        del sets

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
