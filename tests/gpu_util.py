"""Helpers for GPU tests: move a synthetic workload to the device, run the HIP path through the
C ABI, and compare with the oracle at the stated tolerances."""
from __future__ import annotations

import numpy as np
import torch

import sliding_window_decode_amd as sda

# Tolerances: bf16 output vs the round-to-nearest-even bf16 of the fp64 oracle, and fp32 LSE.
OUT_MAX_ABS = 1e-2
OUT_REL_L2 = 5e-3
LSE_MAX_ABS = 1e-3

# Error budget of the kernel's fp32 result before its rounding to bf16, relative to out_abs (the weighted
# mean of the rows' magnitudes under the softmax weights, oracle.attention(..., with_abs=True)). Relative
# errors d_i in the weights move the output by sum_i w_i (d_i - mean d) v_i, at most 2 max|d| out_abs.
# With two or three bf16 terms of P' a weight is within 2^-18 of its fp32 value; exp2 adds 2^-22; a
# score's fp32 sum (18 MFMA chunks, 4 scale folds and the scale: 23 roundings of partial sums below 2^4.5
# in log2 units here) is off by at most 2^-15 in log2 units, a relative 2^-15.5 in its weight; the P.V sums
# (at most 160 chunks of 16 rows) add 2^-16.7 of out_abs. Together below 2^-14: EPS_FP32. With one term
# each weight is rounded once to bf16 (2^-9), so 2 x 2^-9: EPS_P1.
EPS_FP32 = 2.0 ** -14
EPS_P1 = 2.0 ** -8


from sliding_window_decode_amd.inputs import DeviceWorkload, dev_cache, dev_list, dev_q, plan_for  # noqa: E402,F401


def auto_plan_for(w) -> "sda.sda_plan":
    """The plan bench.py times for workload w (sda_choose_plan from the host-side lengths)."""
    return plan_for(w)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()


def _e4m3_rne(y: np.ndarray) -> np.ndarray:
    """Decoded value of the round-to-nearest-even e4m3 code of y (|y| <= 448), via torch's cast."""
    t = torch.from_numpy(np.ascontiguousarray(y, dtype=np.float64)).float()
    return t.to(torch.float8_e4m3fn).to(torch.float64).numpy()


def _inverse_rope_f64(out: np.ndarray, oabs: np.ndarray, positions: np.ndarray, cos_sin: np.ndarray):
    """out [T, H, 512] with dims 448..511 rotated back per GPT-J pair in float64 (positions outside the table:
    unrotated), for locating the cast's decision points (the oracle takes the cast itself in fp32). Returns
    (x, m): the rotated values and the magnitudes their errors scale with: out_abs for an unrotated dim,
    |cos| out_abs_e + |sin| out_abs_o for a rotated one."""
    x = np.array(out, dtype=np.float64)
    m = np.array(oabs, dtype=np.float64)
    pos = np.asarray(positions, dtype=np.int64)
    ok = (pos >= 0) & (pos < cos_sin.shape[0])
    c = np.ones((len(pos), 32))
    sn = np.zeros((len(pos), 32))
    c[ok] = cos_sin[pos[ok], :32]
    sn[ok] = cos_sin[pos[ok], 32:64]
    c, sn = c[:, None, :], sn[:, None, :]
    e, o = out[..., 448::2], out[..., 449::2]
    ae, ao = oabs[..., 448::2], oabs[..., 449::2]
    x[..., 448::2] = e * c + sn * o
    x[..., 449::2] = o * c - sn * e
    m[..., 448::2] = np.abs(c) * ae + np.abs(sn) * ao
    m[..., 449::2] = np.abs(c) * ao + np.abs(sn) * ae
    return x, m


def compare_v41(codes_gpu, scales_gpu, lse_gpu, ref, positions, cos_sin, what="", exact=False, eps=EPS_FP32):
    """MXFP8 output against the oracle's cast of its own result, element by element.

    ref = oracle.attention_v41(...) (codes, scale bytes, lse, fp64 attention result, its out_abs). Both sides
    take the cast's decisions in fp32 from attention results that differ by the kernel's error (eps out_abs). Per 32-dim chunk
    with amax = max(max |x|, 1e-10) over the inverse-rotated oracle values x, the GPU's scale byte must be the
    ue8m0 rounding up of some value within eps of amax / 448; per element, with the GPU's own scale byte b, its
    code must decode to the e4m3 rounding of some value within eps of x 2^(127 - b). The window is checked to
    hold the oracle's own decisions. LSE within 1e-3. exact=True: codes and scales bit-identical."""
    codes_ref, scales_ref, l_ref, out_ref, oabs_ref = ref
    cg = codes_gpu.cpu().numpy() if hasattr(codes_gpu, "cpu") else codes_gpu
    sg = scales_gpu.cpu().numpy() if hasattr(scales_gpu, "cpu") else scales_gpu
    lg = lse_gpu.float().cpu().numpy().astype(np.float64)
    if exact:
        assert np.array_equal(sg, scales_ref), f"{what}: scale bytes differ"
        assert np.array_equal(cg, codes_ref), f"{what}: codes differ"
    assert np.all((cg & 0x7F) != 0x7F), f"{what}: NaN codes"
    # kernel error: eps times each element's magnitude m; the fp32 rotation adds at most 2^-21 of the chunk's
    # amax (two products of values within sqrt(2) amax, each rounded once, then their sum)
    x, m = _inverse_rope_f64(out_ref, oabs_ref, positions, cos_sin)
    T, H, _ = x.shape
    err = eps * m + 2.0 ** -21 * np.repeat(np.abs(x).reshape(T, H, 16, 32).max(-1), 32, axis=-1)
    amax_lo = np.maximum((np.abs(x) - err).reshape(T, H, 16, 32).max(-1), 1e-10)
    amax_hi = np.maximum((np.abs(x) + err).reshape(T, H, 16, 32).max(-1), 1e-10)
    b_lo = 127 + np.ceil(np.log2(amax_lo * (1 - 2.0 ** -22) / 448.0))
    b_hi = 127 + np.ceil(np.log2(amax_hi * (1 + 2.0 ** -22) / 448.0))
    assert np.all((scales_ref >= b_lo) & (scales_ref <= b_hi)), f"{what}: window misses the oracle's scale bytes"

    def code_window(byte):
        f = np.exp2(127.0 - np.repeat(byte.astype(np.float64), 32, axis=-1))
        y, ey = x * f, err * f
        return _e4m3_rne(np.clip(y - ey, -448, 448)), _e4m3_rne(np.clip(y + ey, -448, 448))

    rlo, rhi = code_window(scales_ref)
    dref = e4m3_decode(codes_ref)
    assert np.all((dref >= rlo) & (dref <= rhi)), f"{what}: window misses the oracle's codes"
    s_bad = (sg < b_lo) | (sg > b_hi)
    glo, ghi = code_window(sg)
    dg = e4m3_decode(cg)
    c_bad = (dg < glo) | (dg > ghi)
    info = dict(scale_diffs=int((sg != scales_ref).sum()), code_diffs=int((cg != codes_ref).sum()), n=int(cg.size),
                eps=eps)
    assert not s_bad.any(), f"{what}: {int(s_bad.sum())} scale bytes outside the rounding window {info}"
    assert not c_bad.any(), f"{what}: {int(c_bad.sum())} codes outside the rounding window {info}"
    inf_ref = ~np.isfinite(l_ref)
    assert np.array_equal(inf_ref, ~np.isfinite(lg)), f"{what}: LSE infinities differ"
    if (~inf_ref).any():
        lse_err = float(np.abs(lg[~inf_ref] - l_ref[~inf_ref]).max())
        info["lse_max_abs"] = lse_err
        assert lse_err <= LSE_MAX_ABS, f"{what}: lse max-abs {lse_err:.3e} {info}"
    return info


def eps_for(plan) -> float:
    """The error budget of compare() for a plan's precision mode."""
    return EPS_P1 if plan is not None and plan.precision == 1 else EPS_FP32


def error_stats(out_gpu, lse_gpu, o_ref, l_ref, o_abs, tokens=None, eps=EPS_FP32):
    """The error figures compare() asserts on, without asserting: max-abs and rel-L2 against the RNE-bf16 oracle,
    the LSE error, the elements beyond 1e-2 (midpoint roundings) and those of them outside the eps window."""
    got = out_gpu.float().cpu().numpy().astype(np.float64)
    lg = lse_gpu.float().cpu().numpy().astype(np.float64)
    if tokens is not None:
        got, lg = got[tokens], lg[tokens]
    import oracle  # test infrastructure: imported here, so that bench.py's timed path never loads it

    ref = oracle.bf16_rne(o_ref)
    diff = np.abs(got - ref)
    nrm = float(np.linalg.norm(ref))
    inf_ref = ~np.isfinite(l_ref)
    o_abs = np.asarray(o_abs, dtype=np.float64)
    assert o_abs.shape == o_ref.shape, f"out_abs shape {o_abs.shape} against {o_ref.shape}"
    over = diff > OUT_MAX_ABS
    # the bf16 values that round some y with |y - x| <= eps o_abs (rounding is monotonic: all between these two)
    lo = oracle.bf16_rne(o_ref - eps * o_abs)
    hi = oracle.bf16_rne(o_ref + eps * o_abs)
    bad = over & ~((got >= lo) & (got <= hi))
    st = dict(max_abs=float(diff.max()) if diff.size else 0.0,
              rel_l2=float(np.linalg.norm(got - ref) / nrm) if nrm > 0 else float(np.linalg.norm(got)),
              lse_max_abs=float(np.abs(lg[~inf_ref] - l_ref[~inf_ref]).max()) if (~inf_ref).any() else 0.0,
              midpoint_roundings=int(over.sum()), n=int(diff.size), eps=eps, n_bad=int(bad.sum()),
              finite=bool(np.all(np.isfinite(got))),
              lse_inf_match=bool(np.array_equal(inf_ref, ~np.isfinite(lg)) and np.array_equal(l_ref[inf_ref], lg[inf_ref])))
    if bad.any():
        i = np.flatnonzero(bad.ravel())[:4]
        st["first_bad"] = [(int(k), float(o_ref.ravel()[k]), float(o_abs.ravel()[k]), float(got.ravel()[k])) for k in i]
    return st


def compare(out_gpu, lse_gpu, o_ref, l_ref, o_abs, tokens=None, what="", eps=EPS_FP32):
    """Assert the tolerances element by element; returns a dict of the error figures.

    out: each element within 1e-2 of the round-to-nearest-even bf16 of the fp64 oracle value x, or else
    equal to the bf16 rounding of some value within eps o_abs of x (o_abs: the oracle's weighted mean of the
    rows' magnitudes): where x lies within the kernel's fp32 error budget of a bf16 rounding midpoint,
    either neighbour is a correct rounding of a result that precise, and where |x| >= 2 one bf16 ulp (2^-6
    and up) exceeds 1e-2 by itself. No count of such elements is allowed for; each is checked on its own.
    rel-L2 <= 5e-3 over all elements. lse: within 1e-3 absolute, infinities exact (with their signs)."""
    info = error_stats(out_gpu, lse_gpu, o_ref, l_ref, o_abs, tokens, eps)
    assert info["lse_inf_match"], f"{what}: LSE infinities differ {info}"
    assert info["finite"], f"{what}: non-finite output"
    assert info["n_bad"] == 0, f"{what}: elements beyond 1e-2 and outside the rounding window {info}"
    assert info["rel_l2"] <= OUT_REL_L2, f"{what}: out rel-L2 {info['rel_l2']:.3e} {info}"
    assert info["lse_max_abs"] <= LSE_MAX_ABS, f"{what}: lse max-abs {info['lse_max_abs']:.3e} {info}"
    return info
