"""Randomized parity: seeded random calls against the oracle, every token.

Each case draws a format mix (every record format, the 576-dim one with itself), a head count, a token
count, list widths, page size and page padding, the share of -1 slots, lengths below 0 and above the width,
a sink or none, and a plan (a whole-token plan or a split one with a random part count and per-token
overhead, any heads per workgroup that divides H, any precision). The first record of every cache is filled
with random bytes and slot 0 is left out of every list, so a load a kernel issues for a masked row cannot
leak those bytes into a result (they may read as NaN scales or codes). The bar is the parity bar of the
other GPU tests (gpu_util.compare)."""
import numpy as np
import pytest

import oracle
import sliding_window_decode_amd as sda
import workloads as wl
from gpu_util import EPS_FP32, EPS_P1, DeviceWorkload, compare

pytestmark = pytest.mark.gpu

FORMATS_512 = (wl.FP8_SLOTSCALE, wl.FP8_528, wl.NVFP4_288, wl.FP8_UE8M0, wl.MODEL1_584)


def _case(seed):
    rng = np.random.default_rng([seed, 7])
    if rng.random() < 0.2:
        fmt = wl.V32_656
        xfmt = wl.V32_656 if rng.random() < 0.5 else None
    else:
        fmt = int(rng.choice(FORMATS_512))
        xfmt = None if rng.random() < 0.3 else int(rng.choice(FORMATS_512))
    H = int(rng.choice([16, 32, 64, 128]))
    T = int(rng.integers(1, 40))
    width = int(rng.integers(1, 260))
    xwidth = int(rng.integers(1, 400)) if xfmt is not None else 0
    w = wl.small_workload(1000 + seed, fmt, xfmt, T=T, H=H, width=width, xwidth=xwidth, num_slots=2048,
                          page_size=int(rng.choice([16, 64])), pad_bytes=int(rng.choice([0, 16, 272])),
                          p_invalid=float(rng.choice([0.0, 0.1, 0.5])), sink=bool(rng.random() < 0.6))
    for c, L in w.lists():
        rec = int(sda.lib().sda_record_bytes(c.fmt))
        c.data[:rec] = rng.integers(0, 256, size=rec, dtype=np.uint8)
        L.idx[L.idx == 0] = -1
        L.lens[:] = rng.integers(-2, L.width + 3, size=L.lens.shape).astype(np.int32)
    hpg = int(rng.choice([h for h in (16, 32, 64) if H % h == 0]))
    precision = int(rng.choice([1, 2, 3]))
    if rng.random() < 0.4:
        plan = sda.sda_plan(1, hpg, 0, precision)
        plan.whole_tokens = 1
    else:
        plan = sda.sda_plan(int(rng.integers(1, 300)), hpg, int(rng.integers(0, 4)), precision)
    return w, plan


@pytest.mark.parametrize("seed", range(96))
def test_random_call_matches_the_oracle(seed):
    w, plan = _case(seed)
    what = f"seed {seed}: {w.name} {plan}"
    print(f"[random] {what}", flush=True)
    o_ref, l_ref, o_abs = oracle.attention(w, nthreads=8, with_abs=True)
    assert np.isfinite(o_ref).all(), what
    out, lse, _ = DeviceWorkload(w).run(plan=plan)
    compare(out, lse, o_ref, l_ref, o_abs, what=what, eps=EPS_P1 if plan.precision == 1 else EPS_FP32)
