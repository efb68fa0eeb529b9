"""Parity of the HIP path (through the C ABI) with the fp64 oracle on an MI355X.

Bar (tests/gpu_util.compare): every bf16 output element within max-abs 1e-2 of the RNE-bf16 oracle, or a
correct bf16 rounding of a value within the kernel's fp32 error budget of the oracle's (where that value
sits at a rounding midpoint and one ulp exceeds 1e-2); rel-L2 5e-3; LSE within 1e-3 absolute
(infinities exact). Sizes span several 64-row tiles and ragged tails; the configurations run at reduced
token counts with three seeds, and at full size, every token, in the benchmark's launch configuration."""
import copy
import sys

import numpy as np
import pytest
import torch

import oracle
import sliding_window_decode_amd as sda
import workloads as wl
from gpu_util import EPS_FP32, EPS_P1, DeviceWorkload, auto_plan_for, compare

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


SMALL_T = {"c1_tiny_swa": 4, "c2_swa_h128": 6, "c3_swa_fp8extra": 12, "c4_swa_nvfp4extra": 6, "c5_topk_v32": 3,
           "c6_swa_ue8m0": 12, "c7_swa_model1": 12, "c8_v41_ue8m0": 12}


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("name", wl.CONFIGS)
def test_config_parity_reduced_tokens(name, seed):
    _log(f"[parity] {name} seed={seed} T={SMALL_T[name]}")
    w = wl.make_workload(name, seed=seed, T=SMALL_T[name])
    o_ref, l_ref, o_abs = oracle.attention(w, nthreads=8, with_abs=True)
    dw = DeviceWorkload(w)
    out, lse, dec = dw.run()
    info = compare(out, lse, o_ref, l_ref, o_abs, what=f"{name}/{seed}")
    _log(f"  {dec.plan} {info}")


def _full_size_cases():
    cases = [(n, "auto") for n in wl.CONFIGS]
    # the top-k configuration also on the plan its description names: split-KV sized to 256 CUs + combine
    cases.append(("c5_topk_v32", "split"))
    return cases


@pytest.mark.parametrize("name,schedule", _full_size_cases())
def test_config_parity_full_size(name, schedule):
    """Full-size inputs, every token against the oracle: in the launch configuration bench.py times
    (sda_choose_plan from the host-side lengths), and for the top-k configuration also on the split plan."""
    w = wl.make_workload(name, seed=0)
    plan = auto_plan_for(w)
    if schedule == "split":
        plan = sda.make_plan(w.T, w.H, w.d_qk, w.lst.width, w.xlst.width if w.xlst is not None else 0)
    _log(f"[parity-full] {name} T={w.T} {plan}")
    dw = DeviceWorkload(w)
    out, lse, dec = dw.run(plan=plan)
    o_ref, l_ref, o_abs = oracle.attention(w, nthreads=8, with_abs=True)
    info = compare(out, lse, o_ref, l_ref, o_abs, what=f"{name} full size, {schedule} plan")
    _log(f"  {info}")


# ------------------------------------------------------------------ plans: results independent of the split

@pytest.mark.parametrize("parts,hb,F", [(1, 16, 2), (3, 16, 0), (17, 32, 5), (64, 16, 1), (1000, 32, 2)])
def test_any_plan_same_result(parts, hb, F):
    w = wl.small_workload(3, wl.FP8_528, wl.NVFP4_288, T=9, H=32, width=128, xwidth=300, num_slots=4096,
                          sink=True, p_invalid=0.05, lens_lo=1)
    o_ref, l_ref, o_abs = oracle.attention(w, nthreads=8, with_abs=True)
    dw = DeviceWorkload(w)
    out, lse, dec = dw.run(plan=sda.sda_plan(parts, hb, F, 3))
    compare(out, lse, o_ref, l_ref, o_abs, what=f"plan {parts}/{hb}/{F}")


# FP8_UE8M0 lists: both lists of the format run the ring kernel built for it; mixed with another
# format the call runs the staged kernel (which widens every format into a bf16 tile)
@pytest.mark.parametrize("fmt,xfmt", [(wl.FP8_UE8M0, wl.FP8_UE8M0), (wl.FP8_UE8M0, None), (wl.FP8_UE8M0, wl.FP8_528),
                                      (wl.FP8_528, wl.FP8_UE8M0), (wl.FP8_UE8M0, wl.NVFP4_288),
                                      (wl.FP8_SLOTSCALE, wl.FP8_UE8M0)])
@pytest.mark.parametrize("H,precision", [(16, 2), (32, 2), (32, 3), (128, 2), (16, 3)])
def test_ue8m0_lists(fmt, xfmt, H, precision):
    w = wl.small_workload(40 + 7 * fmt + (xfmt or 0) + H, fmt, xfmt, T=9, H=H, width=140,
                          xwidth=300 if xfmt is not None else 0, num_slots=2048, sink=True, p_invalid=0.05)
    o_ref, l_ref, o_abs = oracle.attention(w, nthreads=8, with_abs=True)
    plan = sda.make_plan(w.T, w.H, w.d_qk, w.lst.width, w.xlst.width if w.xlst is not None else 0)
    plan.precision = precision
    out, lse, dec = DeviceWorkload(w).run(plan=plan)
    compare(out, lse, o_ref, l_ref, o_abs, what=f"ue8m0 {fmt}/{xfmt} H={H} precision {precision}",
            eps=EPS_P1 if precision == 1 else EPS_FP32)


# MODEL1_584 lists (448 fp8 dims with a power-of-two scale per 64, 64 bf16 dims that are values too): the
# ring kernel when every list is one and a workgroup takes 32 or more heads (H >= 32 here), else the staged
# kernel (16 heads, or a list of any other 512-dim format)
@pytest.mark.parametrize("fmt,xfmt", [(wl.MODEL1_584, wl.MODEL1_584), (wl.MODEL1_584, None),
                                      (wl.MODEL1_584, wl.NVFP4_288), (wl.FP8_528, wl.MODEL1_584),
                                      (wl.FP8_UE8M0, wl.MODEL1_584), (wl.MODEL1_584, wl.FP8_SLOTSCALE)])
@pytest.mark.parametrize("H,precision", [(16, 2), (32, 3), (64, 2), (128, 2)])
def test_model1_lists(fmt, xfmt, H, precision):
    w = wl.small_workload(90 + 7 * fmt + (xfmt or 0) + H, fmt, xfmt, T=9, H=H, width=140,
                          xwidth=300 if xfmt is not None else 0, num_slots=2048, sink=True, p_invalid=0.05,
                          page_size=16)
    o_ref, l_ref, o_abs = oracle.attention(w, nthreads=8, with_abs=True)
    plan = sda.make_plan(w.T, w.H, w.d_qk, w.lst.width, w.xlst.width if w.xlst is not None else 0)
    plan.precision = precision
    out, lse, dec = DeviceWorkload(w).run(plan=plan)
    compare(out, lse, o_ref, l_ref, o_abs, what=f"model1 {fmt}/{xfmt} H={H} precision {precision}",
            eps=EPS_P1 if precision == 1 else EPS_FP32)


@pytest.mark.parametrize("H", [16, 32])
def test_model1_bf16_dims_are_values(H):
    """A single valid MODEL1 row: the output is the row itself, its bf16 dims 448..511 included, exactly;
    the pad byte changes nothing (16 heads: the staged kernel; 32: the ring kernel, whose gather reads the
    row's last 16 bytes from record byte 568)."""
    rng = np.random.default_rng(8)
    c = wl.make_cache(rng, wl.MODEL1_584, 64, page_size=16)
    q = wl.make_q(rng, 3, H, 512)
    idx = np.full((3, 40), -1, dtype=np.int32)
    idx[np.arange(3), [0, 17, 39]] = [5, 16, 63]
    lst = wl.SlotList(idx, 40, np.full(3, 40, dtype=np.int32))
    w = wl.Workload("model1 rows", 3, H, 512, 512, q, c, lst, None, None, None, 0.05)
    _, out, _ = _run_cmp(w, "model1 rows")
    pages = c.data.reshape(c.num_pages, c.page_stride)
    pages[:, 583::584][:, :16] = 0xFF
    _, out2, _ = _run_cmp(w, "model1 rows, pad set")
    assert torch.equal(out, out2)
    for t, s in enumerate([5, 16, 63]):
        ref = oracle.decode_slot(c, s)
        for h in (0, H - 1):
            assert np.array_equal(out[t, h].float().cpu().numpy(), oracle.bf16_rne(ref[:512]))


# 64-head workgroups (eight waves with 32 rows and 256 dims each) for every fp8 record layout; a call
# with an NVFP4 list runs 32-head workgroups under the same plan
@pytest.mark.parametrize("fmt,xfmt,H", [(wl.FP8_SLOTSCALE, None, 64), (wl.FP8_528, wl.FP8_528, 128),
                                        (wl.V32_656, None, 64), (wl.V32_656, None, 128),
                                        (wl.FP8_528, wl.NVFP4_288, 64), (wl.FP8_UE8M0, wl.FP8_UE8M0, 128),
                                        (wl.MODEL1_584, wl.MODEL1_584, 128), (wl.MODEL1_584, None, 64)])
@pytest.mark.parametrize("parts", [5, 40])
def test_64_head_workgroups(fmt, xfmt, H, parts):
    w = wl.small_workload(70 + fmt + parts, fmt, xfmt, T=7, H=H, width=150, xwidth=260 if xfmt is not None else 0,
                          num_slots=2048, sink=True, p_invalid=0.05, lens_lo=0)
    o_ref, l_ref, o_abs = oracle.attention(w, nthreads=8, with_abs=True)
    dw = DeviceWorkload(w)
    out, lse, dec = dw.run(plan=sda.sda_plan(parts, 64, 2, 2))
    compare(out, lse, o_ref, l_ref, o_abs, what=f"64-head plan, {parts} parts")


@pytest.mark.parametrize("H", [16, 32, 64, 128])
@pytest.mark.parametrize("fmt", [wl.FP8_SLOTSCALE, wl.FP8_528, wl.NVFP4_288, wl.V32_656, wl.FP8_UE8M0,
                                 wl.MODEL1_584])
def test_heads_and_formats(H, fmt):
    w = wl.small_workload(10 + H + fmt, fmt, None, T=3, H=H, width=200, num_slots=1024, sink=(H % 32 == 0),
                          p_invalid=0.1, lens_lo=0)
    o_ref, l_ref, o_abs = oracle.attention(w, nthreads=8, with_abs=True)
    out, lse, _ = DeviceWorkload(w).run()
    compare(out, lse, o_ref, l_ref, o_abs, what=f"H={H} fmt={fmt}")


@pytest.mark.parametrize("fmt,xfmt", [(wl.FP8_SLOTSCALE, wl.NVFP4_288), (wl.NVFP4_288, wl.FP8_SLOTSCALE),
                                      (wl.FP8_528, wl.FP8_SLOTSCALE), (wl.V32_656, wl.V32_656)])
def test_mixed_list_formats(fmt, xfmt):
    w = wl.small_workload(40 + fmt, fmt, xfmt, T=5, H=16, width=96, xwidth=160, num_slots=2048, sink=True)
    o_ref, l_ref, o_abs = oracle.attention(w, nthreads=8, with_abs=True)
    out, lse, _ = DeviceWorkload(w).run()
    compare(out, lse, o_ref, l_ref, o_abs, what=f"mixed {fmt}/{xfmt}")


# ------------------------------------------------------------------ edge cases

def _run_cmp(w, what, plan=None, sink="default"):
    o_ref, l_ref, o_abs = oracle.attention(w, nthreads=8, sink=sink, with_abs=True)
    dw = DeviceWorkload(w)
    snk = "default" if isinstance(sink, str) else (None if sink is None else torch.from_numpy(sink).cuda())
    out, lse, _ = dw.run(plan=plan, sink=snk)
    return compare(out, lse, o_ref, l_ref, o_abs, what=what), out, lse


@pytest.mark.parametrize("sink", [False, True])
def test_lens_zero(sink):
    w = wl.small_workload(50, wl.FP8_528, wl.FP8_528, T=4, H=16, width=64, xwidth=64, sink=sink)
    w.lst.lens[:] = 0
    w.xlst.lens[:] = 0
    _, out, lse = _run_cmp(w, "lens=0")
    assert torch.all(out == 0)


def test_all_slots_invalid():
    w = wl.small_workload(51, wl.NVFP4_288, None, T=3, H=32, width=130, sink=True)
    w.lst.idx[:] = -1
    w.lst.lens[:] = 130
    _run_cmp(w, "all -1")


@pytest.mark.parametrize("fmt", [wl.FP8_SLOTSCALE, wl.FP8_528, wl.NVFP4_288, wl.V32_656, wl.FP8_UE8M0,
                                 wl.MODEL1_584])
def test_single_valid_slot_returns_its_row(fmt):
    w = wl.small_workload(52 + fmt, fmt, None, T=4, H=32, width=100, num_slots=512)
    w.lst.idx[:] = -1
    for t in range(w.T):
        w.lst.idx[t, (37 * t) % 100] = 7 + 100 * t
        w.lst.lens[t] = 100
    _run_cmp(w, f"single slot fmt {fmt}")


def test_out_of_range_and_negative_slots():
    w = wl.small_workload(56, wl.FP8_528, wl.FP8_528, T=4, H=16, width=128, xwidth=128, num_slots=1024, sink=True)
    rng = np.random.default_rng(0)
    for L in (w.lst, w.xlst):
        m = rng.random(L.idx.shape) < 0.2
        L.idx[m] = rng.choice([1024, 1025, 1 << 30, -2, -1 << 31], size=int(m.sum())).astype(np.int32)
    _run_cmp(w, "out of range")


def test_lens_beyond_width_and_negative():
    w = wl.small_workload(57, wl.FP8_SLOTSCALE, wl.NVFP4_288, T=6, H=16, width=70, xwidth=130, sink=True)
    w.lst.lens[:] = [1000, -3, 70, 0, 69, 1 << 30]
    w.xlst.lens[:] = [-1, 130, 131, 65, 64, 1]
    _run_cmp(w, "lens clamp")


@pytest.mark.parametrize("fmt,xfmt,H", [(wl.FP8_528, wl.NVFP4_288, 16), (wl.FP8_SLOTSCALE, wl.NVFP4_288, 16),
                                        (wl.NVFP4_288, None, 32), (wl.FP8_UE8M0, wl.NVFP4_288, 16)])
def test_masked_rows_whatever_the_first_record_holds(fmt, xfmt, H):
    """Masked rows (slot -1, out of range, past the length) contribute nothing whatever bytes the cache's
    first record holds: here 0x7F 0xFF, the e2m1 pairs (-6, 6) and (-6, -6), which read as e4m3 block scales
    (or as a ue8m0 exponent) would be NaN. Slot 0 itself is left out of every list."""
    w = wl.small_workload(62, fmt, xfmt, T=6, H=H, width=100, xwidth=150 if xfmt is not None else 0, sink=True)
    for c, L in w.lists():
        c.data[0:2] = [0x7F, 0xFF]
        L.idx[L.idx == 0] = -1
        L.idx[:, ::5] = -1
    w.lst.lens[:] = [100, 37, 1, 99, 64, 0]
    if w.xlst is not None:
        w.xlst.lens[:] = [150, 65, 2, 149, 0, 127]
    _, out, _ = _run_cmp(w, "first record bytes")
    assert not torch.isnan(out.float()).any()


def test_page_stride_padding_and_small_pages():
    w = wl.small_workload(58, wl.FP8_528, wl.NVFP4_288, T=4, H=16, width=128, xwidth=128, num_slots=1024,
                          page_size=16, pad_bytes=272, sink=True)
    _run_cmp(w, "padded pages")


def test_row_stride_longer_than_width():
    w = wl.small_workload(59, wl.FP8_528, wl.FP8_528, T=4, H=16, width=90, xwidth=70, row_stride_extra=13)
    _run_cmp(w, "row stride")


def test_duplicate_slots():
    w = wl.small_workload(60, wl.FP8_528, None, T=3, H=16, width=64, num_slots=256)
    w.lst.idx[:, :] = -1
    w.lst.idx[:, 3] = 11
    w.lst.idx[:, 40] = 11
    w.lst.idx[:, 41] = 200
    w.lst.lens[:] = 64
    _run_cmp(w, "duplicates")


def test_sink_infinities():
    w = wl.small_workload(61, wl.FP8_528, None, T=3, H=16, width=64)
    _run_cmp(w, "sink -inf", sink=np.full(16, -np.inf, dtype=np.float32))
    _, out, lse = _run_cmp(w, "sink +inf", sink=np.full(16, np.inf, dtype=np.float32))
    assert torch.all(out == 0)


def test_rescale_path_with_rows_sorted_by_score():
    """Rows ordered by increasing score make the running max move up by more than the rescale
    threshold from tile to tile (moderate logits, the strict bar)."""
    w = wl.small_workload(64, wl.FP8_528, None, T=3, H=16, width=1024, num_slots=4096, sink=True, lens_lo=1024,
                          p_invalid=0.0)
    qf = torch.from_numpy(w.q.view(np.int16)).view(torch.bfloat16).float() * 1.5
    w.q = qf.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    q = qf.double().numpy()
    for t in range(w.T):
        k = np.array([oracle.decode_slot(w.cache, int(s)) for s in w.lst.idx[t]])
        z = k @ q[t, 0]
        w.lst.idx[t] = w.lst.idx[t][np.argsort(z)]
    _run_cmp(w, "sorted rows")


def test_extreme_logits():
    """Scores of magnitude ~30: fp32 score rounding (ulp(30) ~ 2e-6) can flip the bf16 rounding of an
    output element that sits on a rounding boundary; such flips (one ulp) are counted, not hidden."""
    w = wl.small_workload(62, wl.FP8_528, wl.FP8_528, T=3, H=16, width=256, xwidth=256, sink=True, lens_lo=200)
    w2 = copy.deepcopy(w)
    qf = torch.from_numpy(w.q.view(np.int16)).view(torch.bfloat16).float() * 8.0
    w2.q = qf.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    o_ref, l_ref, o_abs = oracle.attention(w2, nthreads=8, with_abs=True)
    out, lse, _ = DeviceWorkload(w2).run()
    info = compare(out, lse, o_ref, l_ref, o_abs, what="extreme logits")
    _log(f"  extreme logits: {info}")


def test_strided_q_and_out():
    w = wl.small_workload(63, wl.FP8_528, None, T=5, H=32, width=100, sink=True)
    o_ref, l_ref, o_abs = oracle.attention(w, nthreads=8, with_abs=True)
    dw = DeviceWorkload(w)
    qbig = torch.zeros((w.T, w.H + 3, 512 + 64), dtype=torch.bfloat16, device="cuda")
    qbig[:, :w.H, :512] = dw.q
    q = qbig[:, :w.H, :512]
    obig = torch.full((w.T, w.H + 1, 512 + 8), 7.0, dtype=torch.bfloat16, device="cuda")
    out = obig[:, :w.H, :512]
    lbig = torch.full((w.T, w.H + 5), 7.0, dtype=torch.float32, device="cuda")
    lse = lbig[:, :w.H]
    dw.run(q=q, out=out, lse=lse)
    compare(out, lse, o_ref, l_ref, o_abs, what="strided")
    assert torch.all(obig[:, w.H:, :] == 7.0) and torch.all(obig[:, :, 512:] == 7.0)
    assert torch.all(lbig[:, w.H:] == 7.0)


@pytest.mark.parametrize("name,T", [("c5_topk_v32", 2), ("c3_swa_fp8extra", 8), ("c4_swa_nvfp4extra", 4),
                                    ("c2_swa_h128", 4)])
@pytest.mark.parametrize("precision", [1, 2, 3])
def test_precision_modes(name, T, precision):
    """Every P precision (one, two (the default) or three bf16 terms) on every kernel path; the single
    term mode may flip more outputs of magnitude >= 2 by one bf16 ulp."""
    w = wl.make_workload(name, seed=4, T=T)
    o_ref, l_ref, o_abs = oracle.attention(w, nthreads=8, with_abs=True)
    X = w.xlst.width if w.xlst is not None else 0
    plan = sda.make_plan(w.T, w.H, w.d_qk, w.lst.width, X)
    plan.precision = precision
    out, lse, _ = DeviceWorkload(w).run(plan=plan)
    compare(out, lse, o_ref, l_ref, o_abs, what=f"{name} precision {precision}", eps=EPS_P1 if precision == 1 else EPS_FP32)


# ------------------------------------------------------------------ decode tables on the GPU

def test_every_e4m3_code_decodes_exactly():
    """Rows that hold every finite e4m3 code; a single valid slot returns its row exactly."""
    rng = np.random.default_rng(5)
    c = wl.make_cache(rng, wl.FP8_528, 64, page_size=64)
    codes = np.array([x for x in range(256) if x not in (0x7F, 0xFF)], dtype=np.uint8)
    for s in range(4):
        rec = c.data[s * 528:(s + 1) * 528]
        row = np.resize(codes, 512)
        rec[:512] = np.roll(row, 37 * s)
        rec[512:528] = np.array([1.0, 0.5, 2.0, 0.75], dtype=np.float32).view(np.uint8)
    q = wl.make_q(rng, 4, 16, 512)
    idx = np.full((4, 8), -1, dtype=np.int32)
    idx[:, 2] = np.arange(4)
    lst = wl.SlotList(idx, 8, np.full(4, 8, dtype=np.int32))
    w = wl.Workload("e4m3 table", 4, 16, 512, 512, q, c, lst, None, None, None, 0.05)
    _, out, _ = _run_cmp(w, "e4m3 table")
    for t in range(4):
        ref = oracle.decode_slot(c, t)
        assert np.array_equal(out[t, 0].float().cpu().numpy(), oracle.bf16_rne(ref[:512]))


def _ue8m0_sweep_workload(H, nan_slot=None, width=40):
    """16 FP8_UE8M0 records whose 16 scale bytes sweep 0..254 ((16 r + g) % 255 for record r, group g), codes of
    magnitude 1..1.875 (so every value c 2^(e - 127) is a bf16 number, 2^-127 scale included), and token t's
    list holding record t alone; q = 0, so each output row is its record exactly and every lse is 0.
    nan_slot: a 17th record with scale byte 255 in group 5, read alone by a 17th token. width: list width (the
    other entries -1)."""
    rng = np.random.default_rng(77)
    n = 17 if nan_slot else 16
    rec = np.zeros((64, 528), dtype=np.uint8)
    mags = rng.integers(0x38, 0x40, size=(n, 512)).astype(np.uint8)
    signs = (rng.integers(0, 2, size=(n, 512)) * 0x80).astype(np.uint8)
    rec[:n, :512] = mags | signs
    for r in range(16):
        rec[r, 512:528] = [(16 * r + g) % 255 for g in range(16)]
    if nan_slot:
        rec[16, 512:528] = 127
        rec[16, 512 + 5] = 255
    c = wl.Cache(wl.FP8_UE8M0, 1, 64, 64 * 528, rec.reshape(-1).copy())
    idx = np.full((n, width), -1, dtype=np.int32)
    idx[np.arange(n), (7 * np.arange(n) + width - 40) % width] = np.arange(n)
    lst = wl.SlotList(idx, width, np.full(n, width, dtype=np.int32))
    q = np.zeros((n, H, 512), dtype=np.uint16)
    return wl.Workload("ue8m0 byte sweep", n, H, 512, 512, q, c, lst, None, None, None, 0.05)


@pytest.mark.parametrize("H", [16, 32])
def test_every_ue8m0_scale_byte(H):
    """Every ue8m0 scale byte 0..254 (vLLM swapab_decode_attn, stage_inputs fp8 branch; OCP MX E8M0): a single
    valid row returns its record exactly, bit for bit with RNE-bf16 of the oracle, 2^-127 for byte 0 included
    (16 heads: the ring kernel built for the format; 32: the same at two head sets)."""
    w = _ue8m0_sweep_workload(H)
    o_ref, l_ref = oracle.attention(w)
    out, lse, dec = DeviceWorkload(w).run()
    got = out.float().cpu().numpy().astype(np.float64)
    ref = oracle.bf16_rne(o_ref)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} elements differ, first {[(tuple(b), got[tuple(b)], ref[tuple(b)]) for b in bad[:4]]}"
    assert np.array_equal(lse.cpu().numpy(), l_ref.astype(np.float32))
    # byte 0 of record 0 covers dims 0..31: its values are codes x 2^-127
    assert np.all(np.abs(ref[0, 0, :32]) < 2.0 ** -126) and np.all(ref[0, 0, :32] != 0)


@pytest.mark.parametrize("parts", [None, 68])
def test_ue8m0_byte_255_gives_nan_rows(parts):
    """Scale byte 255 is NaN in the MX encoding: the token that reads such a record gets NaN outputs and a NaN
    LSE, as the oracle does; the other tokens are untouched. parts = 68: lists of 256 entries (4 tiles) on 68
    parts, so each token is split in four, three partials without a valid row (LSE -inf) and one with the
    record, and the NaN partial is carried through the combine."""
    w = _ue8m0_sweep_workload(16, nan_slot=True, width=40 if parts is None else 256)
    o_ref, l_ref = oracle.attention(w)
    assert np.all(np.isnan(o_ref[16])) and np.all(np.isnan(l_ref[16]))
    out, lse, _ = DeviceWorkload(w).run(plan=None if parts is None else sda.sda_plan(parts, 16, 0, 3))
    got = out.float().cpu().numpy()
    assert np.all(np.isnan(got[16])) and np.all(np.isnan(lse[16].cpu().numpy()))
    assert np.array_equal(got[:16].astype(np.float64), oracle.bf16_rne(o_ref[:16]))


def test_every_e2m1_code_and_block_scale():
    rng = np.random.default_rng(6)
    c = wl.make_cache(rng, wl.NVFP4_288, 64, page_size=64)
    for s in range(4):
        rec = c.data[s * 288:(s + 1) * 288]
        rec[:256] = (np.arange(256) + 17 * s) % 256
        rec[256:288] = rng.choice([x for x in range(0x08, 0x78)], size=32)
    q = wl.make_q(rng, 4, 16, 512)
    idx = np.full((4, 8), -1, dtype=np.int32)
    idx[:, 5] = np.arange(4)
    lst = wl.SlotList(idx, 8, np.full(4, 8, dtype=np.int32))
    w = wl.Workload("e2m1 table", 4, 16, 512, 512, q, c, lst, None, None, None, 0.05)
    _, out, _ = _run_cmp(w, "e2m1 table")
    for t in range(4):
        ref = oracle.decode_slot(c, t)
        assert np.array_equal(out[t, 3].float().cpu().numpy(), oracle.bf16_rne(ref[:512]))


# ------------------------------------------------------------------ scheduler and combine through the ABI

@pytest.mark.parametrize("T,P,F", [(700, 1, 2), (700, 256, 2), (700, 513, 0), (700, 4096, 5), (1024, 768, 0),
                                   (1025, 768, 0), (1025, 97, 3), (3000, 256, 2), (3000, 5000, 1)])
def test_device_scheduler_matches_host(T, P, F):
    """The device scheduler against its host twin; T above 1024 takes the kernel's chunked pass (the
    lengths read per chunk of 1024 tokens, the scans carried across chunks)."""
    rng = np.random.default_rng(P + T)
    lens = rng.integers(-3, 140, size=T).astype(np.int32)
    xl = rng.integers(0, 2049, size=T).astype(np.int32)
    plan = sda.sda_plan(P, 16, F, 3)
    meta_h, ns_h = sda.get_sched_meta_host(T, lens, 128, xl, 2048, plan)
    lst = sda.SlotList(torch.zeros((T, 128), dtype=torch.int32, device="cuda"), 128, torch.from_numpy(lens).cuda())
    xlst = sda.SlotList(torch.zeros((T, 2048), dtype=torch.int32, device="cuda"), 2048, torch.from_numpy(xl).cuda())
    meta = torch.full((P, 8), -7, dtype=torch.int32, device="cuda")
    ns = torch.full((T + 1,), -7, dtype=torch.int32, device="cuda")
    sda.get_sched_meta(T, lst, xlst, plan, meta, ns)
    torch.cuda.synchronize()
    assert np.array_equal(meta.cpu().numpy(), meta_h)
    assert np.array_equal(ns.cpu().numpy(), ns_h)


def test_split_call_with_more_tokens_than_a_scheduler_chunk():
    """A split call of 1100 tokens (the scheduler's chunked pass) against the oracle, every token."""
    w = wl.small_workload(71, wl.FP8_528, wl.FP8_528, T=1100, H=16, width=64, xwidth=96, num_slots=4096,
                          sink=True)
    plan = auto_plan_for(w)
    plan.whole_tokens = 0
    plan.num_parts = 768
    plan.fixed_overhead = 1
    _run_cmp(w, "T = 1100 split", plan=plan)


def test_combine_splits_against_oracle_merge():
    w = wl.small_workload(70, wl.FP8_528, None, T=5, H=16, width=192, num_slots=2048, sink=True, lens_lo=100)
    H = w.H
    nparts = [2, 3, 2, 4, 5]
    o_parts, l_parts, refs = [], [], []
    rng = np.random.default_rng(0)
    for t in range(w.T):
        tw = copy.deepcopy(w)
        tw.T = 1
        tw.q = w.q[t:t + 1]
        tw.lst = wl.SlotList(w.lst.idx[t:t + 1].copy(), w.lst.width, w.lst.lens[t:t + 1].copy())
        owner = rng.integers(0, nparts[t], size=w.lst.width)
        for p in range(nparts[t]):
            pw = copy.deepcopy(tw)
            pw.lst.idx[0, owner != p] = -1
            o, l = oracle.attention(pw, sink=None)
            o_parts.append(o[0])
            l_parts.append(l[0])
        refs.append(oracle.attention(tw, with_abs=True))
    ns = np.concatenate([[0], np.cumsum(nparts)]).astype(np.int32)
    o_acc = torch.from_numpy(np.array(o_parts, dtype=np.float32)).cuda()
    l_acc = torch.from_numpy(np.array(l_parts, dtype=np.float32)).cuda()
    out = torch.zeros((w.T, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((w.T, H), dtype=torch.float32, device="cuda")
    sda.combine_splits(o_acc, l_acc, torch.from_numpy(ns).cuda(), torch.from_numpy(w.sink).cuda(), out, lse)
    torch.cuda.synchronize()
    o_ref = np.concatenate([r[0] for r in refs])
    l_ref = np.concatenate([r[1] for r in refs])
    o_abs = np.concatenate([r[2] for r in refs])
    compare(out, lse, o_ref, l_ref, o_abs, what="combine")


def test_repeat_runs_are_bitwise_identical():
    w = wl.make_workload("c4_swa_nvfp4extra", seed=2, T=40)
    dw = DeviceWorkload(w)
    o1, l1, _ = dw.run()
    o2, l2, _ = dw.run()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ------------------------------------------------------------------ requests of several queries

@pytest.mark.parametrize("fmt,xfmt,H,qpl", [(wl.FP8_528, wl.FP8_528, 64, 2), (wl.FP8_528, None, 128, 4),
                                            (wl.FP8_UE8M0, wl.FP8_UE8M0, 32, 3), (wl.FP8_528, wl.NVFP4_288, 16, 5),
                                            (wl.V32_656, None, 64, 2)])
def test_request_lengths_shared_by_queries(fmt, xfmt, H, qpl):
    """Lengths per request shared by its s_q queries (queries_per_len) give bit-identical results to the
    same lengths repeated per token, and match the oracle; the token count leaves a ragged last request."""
    T = 4 * qpl + 1
    _log(f"[requests] fmt={fmt} xfmt={xfmt} H={H} s_q={qpl} T={T}")
    kw = dict(T=T, H=H, width=128, num_slots=4096, sink=True, p_invalid=0.05, lens_lo=0)
    if xfmt is not None:
        kw["xwidth"] = 320
    w = wl.small_workload(80 + qpl, fmt, xfmt, **kw)
    rng = np.random.default_rng(qpl)
    nreq = -(-T // qpl)
    g = copy.deepcopy(w)
    for L in [g.lst] + ([g.xlst] if xfmt is not None else []):
        L.lens = rng.integers(0, L.width + 1, size=nreq).astype(np.int32)
        L.queries_per_len = qpl
    e = copy.deepcopy(w)
    r = np.arange(T) // qpl
    e.lst.lens = g.lst.lens[r].copy()
    if xfmt is not None:
        e.xlst.lens = g.xlst.lens[r].copy()
    _, out_g, lse_g = _run_cmp(g, f"grouped s_q={qpl}")
    out_e, lse_e, _ = DeviceWorkload(e).run()
    assert torch.equal(out_g, out_e) and torch.equal(lse_g, lse_e)


# ------------------------------------------------------------------ whole-token plans (no scheduler, no combine)

def _whole_plan(w):
    plan = sda.make_plan(w.T, w.H, w.d_qk, w.lst.width, w.xlst.width if w.xlst is not None else 0)
    plan.whole_tokens = 1
    return plan


@pytest.mark.parametrize("name", [n for n in wl.CONFIGS if n != "c8_v41_ue8m0"])
def test_whole_token_plan_parity(name):
    """One workgroup per (token, head group), no scheduler and no combine: the same bar against the oracle
    on every kernel (ring and staged, every record format), with empty tokens (C1) and uneven lengths
    (C3, C4)."""
    w = wl.make_workload(name, seed=3, T=SMALL_T[name])
    _log(f"[whole] {name} T={w.T}")
    o_ref, l_ref, o_abs = oracle.attention(w, nthreads=8, with_abs=True)
    out, lse, dec = DeviceWorkload(w).run(plan=_whole_plan(w))
    assert dec.plan.whole_tokens
    info = compare(out, lse, o_ref, l_ref, o_abs, what=f"{name} whole tokens")
    _log(f"  {dec.plan} {info}")


@pytest.mark.parametrize("name", ["c1_tiny_swa", "c2_swa_h128", "c3_swa_fp8extra", "c6_swa_ue8m0"])
def test_whole_token_plan_16_head_groups(name):
    """The head grouping the library picks for whole-token calls on the fp8 ring kernel (16 heads per
    workgroup): same bar against the oracle."""
    w = wl.make_workload(name, seed=4, T=SMALL_T[name])
    plan = _whole_plan(w)
    plan.heads_per_group = 16  # the grouping sda_choose_plan takes for such calls at full size
    _log(f"[whole hb16] {name} T={w.T}")
    o_ref, l_ref, o_abs = oracle.attention(w, nthreads=8, with_abs=True)
    out, lse, dec = DeviceWorkload(w).run(plan=plan)
    compare(out, lse, o_ref, l_ref, o_abs, what=f"{name} whole tokens, 16 heads per group")


@pytest.mark.parametrize("fmt,xfmt,width,xwidth,H,hb", [
    (wl.FP8_SLOTSCALE, wl.FP8_528, 40, 100, 32, 16),   # list 0 narrower than one tile
    (wl.FP8_528, wl.FP8_528, 200, 70, 32, 32),         # list 0 over four tiles, ragged
    (wl.MODEL1_584, wl.MODEL1_584, 100, 130, 32, 32),  # MODEL1 on the ring kernel
    (wl.V32_656, None, 150, 0, 64, 64),                # 576-dim records, 64-head groups
])
def test_whole_token_plan_first_tiles(fmt, xfmt, width, xwidth, H, hb):
    """The first tiles' slot ids of a whole-token workgroup are read before its lengths (and kept only where
    the first items are list 0's first tiles): narrow and wide main lists, empty main lists (the first
    items come from the extra list), a row stride past the width, and padded rows."""
    w = wl.small_workload(600 + width + fmt, fmt, xfmt, T=11, H=H, width=width, xwidth=xwidth, num_slots=2048,
                          sink=True, p_invalid=0.1, lens_lo=0, row_stride_extra=24)
    w.lst.lens[[0, 3, 7]] = 0
    w.lst.lens[[1, 5]] = width
    plan = _whole_plan(w)
    plan.heads_per_group = hb
    _log(f"[whole first tiles] fmt {fmt}/{xfmt} width {width}/{xwidth} H={H} hb={hb}")
    o_ref, l_ref, o_abs = oracle.attention(w, nthreads=8, with_abs=True)
    out, lse, dec = DeviceWorkload(w).run(plan=plan)
    compare(out, lse, o_ref, l_ref, o_abs, what=f"whole first tiles {fmt}/{xfmt} {width}/{xwidth}")


def test_whole_token_plan_equals_one_token_parts():
    """Where the split schedule gives every part exactly one whole token (64 tokens of two tiles each over 64
    parts at the 128-head SWA shape), the whole-token plan computes the same sums in the same order."""
    w = wl.make_workload("c2_swa_h128", seed=0)
    dw = DeviceWorkload(w)
    o1, l1, d1 = dw.run()
    assert not d1.plan.whole_tokens and d1.plan.num_parts == w.T
    o2, l2, _ = dw.run(plan=_whole_plan(w))
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_whole_token_plan_request_lengths_and_sinks():
    """Lengths per request (queries_per_len = 3, ragged last request, empty requests) and infinite sinks on a
    whole-token plan: bit-identical to the same lengths given per token, and within the bar of the oracle."""
    qpl, T, H = 3, 13, 32
    w = wl.small_workload(97, wl.FP8_528, wl.FP8_528, T=T, H=H, width=128, xwidth=320, num_slots=4096, sink=True,
                          p_invalid=0.05, lens_lo=0)
    rng = np.random.default_rng(5)
    nreq = -(-T // qpl)
    g = copy.deepcopy(w)
    for L in (g.lst, g.xlst):
        L.lens = rng.integers(0, L.width + 1, size=nreq).astype(np.int32)
        L.lens[1] = 0  # an empty request
        L.queries_per_len = qpl
    g.sink[3] = np.inf
    e = copy.deepcopy(g)
    r = np.arange(T) // qpl
    e.lst.lens = g.lst.lens[r].copy()
    e.xlst.lens = g.xlst.lens[r].copy()
    e.lst.queries_per_len = e.xlst.queries_per_len = 1
    o_ref, l_ref, o_abs = oracle.attention(g, nthreads=8, with_abs=True)
    out_g, lse_g, _ = DeviceWorkload(g).run(plan=_whole_plan(g))
    compare(out_g, lse_g, o_ref, l_ref, o_abs, what="whole tokens, request lengths")
    out_e, lse_e, _ = DeviceWorkload(e).run(plan=_whole_plan(e))
    assert torch.equal(out_g, out_e) and torch.equal(lse_g, lse_e)


def test_whole_token_plan_decode_only_entry_point():
    """sda_decode_splits on a whole-token plan (no meta, no num_splits) writes exactly what the whole op writes."""
    w = wl.make_workload("c5_topk_v32", seed=2, T=SMALL_T["c5_topk_v32"])
    dw = DeviceWorkload(w)
    plan = _whole_plan(w)
    o1, l1, dec = dw.run(plan=plan)
    o2 = torch.full_like(o1, 7.0)
    l2 = torch.full_like(l1, 7.0)
    sda.decode_splits(dw.q, dw.cache, dw.lst, None, None, dw.sink, w.scale, dec.plan, None, None, dec.workspace, o2, l2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
