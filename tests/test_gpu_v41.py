"""The V4.1 decode call (Q RoPE, decode, inverse RoPE and MXFP8 output) on an MI355X against the oracle.

Bar (gpu_util.compare_v41): every scale byte and every code is a correct cast of a value within the kernel's
fp32 error budget of the oracle's result (element by element, no count of differences allowed for); LSE
within 1e-3. Outputs that come out of the attention exactly (a single valid row) are bit-identical."""
import sys

import numpy as np
import pytest
import torch

import oracle
import sliding_window_decode_amd as sda
import workloads as wl
from gpu_util import DeviceWorkload, auto_plan_for, compare_v41

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _with_rope(w, seed, num_positions=4096, out_of_range=()):
    w.rope = wl.make_rope(np.random.default_rng([seed, 99]), w.T, num_positions=num_positions)
    for t, pos in out_of_range:
        w.rope.positions[t] = pos
    return w


@pytest.mark.parametrize("fmt,xfmt,H", [(wl.FP8_UE8M0, wl.FP8_UE8M0, 32), (wl.FP8_UE8M0, wl.NVFP4_288, 16),
                                        (wl.FP8_528, wl.FP8_528, 64), (wl.MODEL1_584, None, 128),
                                        (wl.FP8_SLOTSCALE, None, 16), (wl.FP8_UE8M0, None, 128),
                                        (wl.MODEL1_584, wl.FP8_UE8M0, 32)])
def test_v41_parity(fmt, xfmt, H):
    _log(f"[v41] fmt={fmt} xfmt={xfmt} H={H}")
    w = wl.small_workload(200 + fmt + H, fmt, xfmt, T=9, H=H, width=150, xwidth=330 if xfmt is not None else 0,
                          num_slots=2048, sink=True, p_invalid=0.05, lens_lo=0)
    _with_rope(w, fmt + H, out_of_range=[(1, -5), (2, 4096)])
    ref = oracle.attention_v41(w, nthreads=8)
    c, s, l, dec = DeviceWorkload(w).run_v41()
    info = compare_v41(c, s, l, ref, w.rope.positions, w.rope.cos_sin, what=f"v41 {fmt}/{xfmt} H={H}")
    _log(f"  {dec.plan} {info}")


@pytest.mark.parametrize("parts", [1, 7, 64])
def test_v41_any_split_same_bar(parts):
    import sliding_window_decode_amd as sda
    w = _with_rope(wl.small_workload(230 + parts, wl.FP8_UE8M0, wl.FP8_UE8M0, T=6, H=32, width=128, xwidth=512,
                                     num_slots=4096, sink=True, lens_lo=1), parts)
    ref = oracle.attention_v41(w, nthreads=8)
    c, s, l, _ = DeviceWorkload(w).run_v41(plan=sda.sda_plan(parts, 32, 2, 2))
    compare_v41(c, s, l, ref, w.rope.positions, w.rope.cos_sin, what=f"v41 {parts} parts")


@pytest.mark.parametrize("fmt", [wl.FP8_UE8M0, wl.MODEL1_584, wl.NVFP4_288])
def test_v41_single_row_is_bit_exact(fmt):
    """One valid row per token, no sink: the attention output is that row exactly (formats whose scales the
    kernels apply exactly: powers of two in the conversion, NVFP4 widened exactly), so the inverse RoPE and
    the cast see the same fp32 values as the oracle's and every code and scale byte matches."""
    rng = np.random.default_rng(240 + fmt)
    w = wl.small_workload(240 + fmt, fmt, None, T=6, H=16, width=70, num_slots=1024)
    w.lst.idx[:] = -1
    for t in range(w.T):
        w.lst.idx[t, int(rng.integers(0, 70))] = int(rng.integers(0, 1024))
    w.lst.lens[:] = 70
    _with_rope(w, fmt, out_of_range=[(0, -1)])
    ref = oracle.attention_v41(w, nthreads=8)
    c, s, l, _ = DeviceWorkload(w).run_v41()
    compare_v41(c, s, l, ref, w.rope.positions, w.rope.cos_sin, what=f"single row fmt {fmt}", exact=True)


def test_v41_empty_tokens_and_infinite_sink():
    w = _with_rope(wl.small_workload(250, wl.FP8_UE8M0, wl.FP8_UE8M0, T=4, H=16, width=64, xwidth=64, sink=True), 1)
    w.lst.lens[:2] = 0
    w.xlst.lens[:2] = 0
    w.sink[3] = np.inf
    ref = oracle.attention_v41(w, nthreads=8)
    c, s, l, _ = DeviceWorkload(w).run_v41()
    compare_v41(c, s, l, ref, w.rope.positions, w.rope.cos_sin, what="empty tokens")
    assert torch.all((c[:2] & 0x7F) == 0)  # zeros (a rotated zero may carry a minus sign)
    assert np.array_equal(s[:2].cpu().numpy(), ref[1][:2])


def test_v41_grouped_lengths_and_strided_outputs():
    """Requests of three queries sharing lengths; outputs written into larger, strided buffers."""
    import sliding_window_decode_amd as sda
    w = wl.small_workload(260, wl.FP8_UE8M0, wl.FP8_UE8M0, T=7, H=16, width=100, xwidth=200, num_slots=2048,
                          sink=True)
    rng = np.random.default_rng(260)
    for L in (w.lst, w.xlst):
        L.lens = rng.integers(0, L.width + 1, size=3).astype(np.int32)
        L.queries_per_len = 3
    _with_rope(w, 260)
    ref = oracle.attention_v41(w, nthreads=8)
    dw = DeviceWorkload(w)
    dec = sda.Decoder(w.T, w.H, 512, w.lst.width, w.xlst.width)
    big8 = torch.full((w.T, w.H, 640), 0x55, dtype=torch.uint8, device="cuda")
    bigs = torch.full((w.T, w.H, 32), 0x55, dtype=torch.uint8, device="cuda")
    c, s, l = dec.v41(dw.q, dw.cache, dw.lst, dw.xcache, dw.xlst, dw.sink, w.scale, dw.positions, dw.cos_sin,
                      out_fp8=big8[:, :, :512], out_scale=bigs[:, :, :16])
    torch.cuda.synchronize()
    compare_v41(c, s, l, ref, w.rope.positions, w.rope.cos_sin, what="grouped, strided")
    assert torch.all(big8[:, :, 512:] == 0x55) and torch.all(bigs[:, :, 16:] == 0x55)


@pytest.mark.parametrize("T", [5, 24])
def test_v41_workload_reduced_tokens(T):
    w = wl.make_workload("c8_v41_ue8m0", seed=1, T=T)
    ref = oracle.attention_v41(w, nthreads=8)
    c, s, l, dec = DeviceWorkload(w).run_v41()
    info = compare_v41(c, s, l, ref, w.rope.positions, w.rope.cos_sin, what=f"c8 T={T}")
    _log(f"  {dec.plan} {info}")


def test_v41_workload_full_size():
    """The full V4.1 workload in the benchmark's launch configuration; every token against the oracle."""
    w = wl.make_workload("c8_v41_ue8m0", seed=0)
    _log(f"[v41-full] T={w.T}")
    c, s, l, dec = DeviceWorkload(w).run_v41(plan=auto_plan_for(w))
    ref = oracle.attention_v41(w, nthreads=8)
    info = compare_v41(c, s, l, ref, w.rope.positions, w.rope.cos_sin, what="c8 full size")
    _log(f"  {dec.plan} {info}")


def test_v41_whole_token_plan():
    """The V4.1 call on a whole-token plan (no scheduler; the epilogue merges each token's single partial)."""
    w = wl.make_workload("c8_v41_ue8m0", seed=4, T=12)
    ref = oracle.attention_v41(w, nthreads=8)
    plan = sda.make_plan(w.T, w.H, w.d_qk, w.lst.width, w.xlst.width)
    plan.whole_tokens = 1
    c, s, l, dec = DeviceWorkload(w).run_v41(plan=plan)
    assert dec.plan.whole_tokens
    info = compare_v41(c, s, l, ref, w.rope.positions, w.rope.cos_sin, what="c8 whole tokens")
    _log(f"  {dec.plan} {info}")
