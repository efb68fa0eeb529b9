"""Pins of the fp64 CPU oracle against things other than itself: library decoders,
the OCP e2m1 table, byte layouts stated on the pages, torch's SDPA, closed forms,
invariants and an independent brute-force loop. None of these needs a GPU."""
import copy
import math

import numpy as np
import pytest
import torch

import workloads as wl
from refdecode import bf16_torch, decode_rows, e2m1_table, e4m3_torch, layouts, q_f64, valid_rows

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ------------------------------------------------------------------ decoders

def test_e4m3_every_code_matches_torch(orc):
    L = orc.lib()
    ref = e4m3_torch(np.arange(256, dtype=np.uint8))
    got = np.array([L.orc_e4m3(c) for c in range(256)])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    assert got[0x7E] == layouts()["e4m3_max"]["value"]


def test_e2m1_every_code_matches_ocp_table(orc):
    L = orc.lib()
    got = np.array([L.orc_e2m1(c) for c in range(16)])
    tab = e2m1_table()
    assert np.array_equal(got, tab)
    assert np.array_equal(np.signbit(got), np.signbit(tab))


def test_bf16_matches_torch(orc):
    L = orc.lib()
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 1 << 16, size=4000).astype(np.uint16)
    ref = bf16_torch(bits)
    got = np.array([L.orc_bf16(int(b)) for b in bits])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_record_sizes_match_pages(orc):
    L = orc.lib()
    g = layouts()
    assert L.orc_record_bytes(wl.V32_656) == g["v32_656"]["bytes"] == sum(g["v32_656"]["parts"].values())
    assert L.orc_record_bytes(wl.FP8_528) == g["fp8_528"]["bytes"] == sum(g["fp8_528"]["parts"].values())
    assert L.orc_record_bytes(wl.NVFP4_288) == g["nvfp4_288"]["bytes"] == sum(g["nvfp4_288"]["parts"].values())
    assert L.orc_record_bytes(wl.FP8_SLOTSCALE) == g["fp8_slotscale_512"]["bytes"]
    assert L.orc_record_bytes(wl.FP8_UE8M0) == g["fp8_ue8m0_528"]["bytes"] == sum(g["fp8_ue8m0_528"]["parts"].values())
    assert L.orc_record_dims(wl.FP8_UE8M0) == 512
    assert L.orc_record_bytes(wl.MODEL1_584) == g["model1_584"]["bytes"] == sum(g["model1_584"]["parts"].values())
    assert L.orc_record_dims(wl.MODEL1_584) == 512
    assert g["model1_584"]["parts"]["ue8m0_scales"] * g["model1_584"]["scale_group_dims"] == g["model1_584"]["parts"]["e4m3_codes"]
    assert L.orc_record_dims(wl.V32_656) == 576 and L.orc_record_dims(wl.FP8_528) == 512
    for f in wl.RECORD_BYTES:
        assert L.orc_record_bytes(f) == wl.RECORD_BYTES[f]


@pytest.mark.parametrize("fmt", [wl.FP8_SLOTSCALE, wl.FP8_528, wl.NVFP4_288, wl.V32_656, wl.FP8_UE8M0,
                                 wl.MODEL1_584])
@pytest.mark.parametrize("pad", [0, 96])
def test_decode_slot_matches_library_decoding(orc, fmt, pad):
    rng = np.random.default_rng(fmt * 10 + pad)
    c = wl.make_cache(rng, fmt, 256, page_size=16, pad_bytes=pad)
    sids = rng.choice(256, size=40, replace=False)
    ref = decode_rows(c, sids)
    for i, s in enumerate(sids):
        got = orc.decode_slot(c, int(s))
        assert got is not None
        assert np.array_equal(got, ref[i]), (fmt, s)


def test_nvfp4_chunk_and_scale_mapping(orc):
    """Packed chunk c covers dims [32c, 32c+32) and uses scale bytes 2c, 2c+1 (vLLM page)."""
    c = wl.make_cache(np.random.default_rng(0), wl.NVFP4_288, 64, page_size=64)
    rec = c.data[:288]
    rec[:256] = 0x22                      # every element = e2m1 code 2 = 1.0
    rec[256:288] = np.arange(32, dtype=np.uint8) + 0x30   # distinct e4m3 scales
    k = orc.decode_slot(c, 0)
    sc = e4m3_torch(rec[256:288])
    for ch in range(16):
        dims = slice(32 * ch, 32 * ch + 32)
        assert np.array_equal(k[dims][:16], np.full(16, sc[2 * ch]))
        assert np.array_equal(k[dims][16:], np.full(16, sc[2 * ch + 1]))
    rec[0] = 0x67                         # low nibble (7 = 6.0) -> element 0, high (6 = 4.0) -> element 1
    k = orc.decode_slot(c, 0)
    assert k[0] == 6.0 * sc[0] and k[1] == 4.0 * sc[0]


def test_ue8m0_values(orc):
    """ue8m0 (OCP MX scale): 2^(byte - 127), 0xFF NaN."""
    L = orc.lib()
    assert L.orc_ue8m0(127) == 1.0 and L.orc_ue8m0(130) == 8.0 and L.orc_ue8m0(124) == 0.125
    assert L.orc_ue8m0(0) == 2.0 ** -127 and L.orc_ue8m0(254) == 2.0 ** 127
    assert np.isnan(L.orc_ue8m0(255))


def test_ue8m0_chunk_and_scale_mapping(orc):
    """Scale byte g covers dims [32g, 32g+32) (chunk c of 16 dims takes byte c // 2, vLLM page)."""
    c = wl.make_cache(np.random.default_rng(0), wl.FP8_UE8M0, 64, page_size=64)
    rec = c.data[:528]
    rec[:512] = 0x38                                      # e4m3 1.0 in every dim
    rec[512:528] = 119 + np.arange(16, dtype=np.uint8)    # scales 2^-8 .. 2^7
    k = orc.decode_slot(c, 0)
    assert np.array_equal(k, np.repeat(2.0 ** (np.arange(16) - 8), 32))
    rec[16:32] = 0x40                                     # chunk 1 (dims 16..31): e4m3 2.0, still scale byte 0
    rec[32:48] = 0xB8                                     # chunk 2 (dims 32..47): e4m3 -1.0, scale byte 1
    k = orc.decode_slot(c, 0)
    assert np.all(k[16:32] == 2.0 * 2.0 ** -8) and np.all(k[32:48] == -(2.0 ** -7))


def test_model1_parts_and_scale_mapping(orc):
    """MODEL1 record: dims 0..447 are e4m3 codes times scale byte d // 64 of the 7 after the bf16 part,
    dims 448..511 the bf16 values (no scale), the last byte plays no part."""
    c = wl.make_cache(np.random.default_rng(0), wl.MODEL1_584, 64, page_size=64)
    rec = c.data[:584]
    rec[:448] = 0x38                                      # e4m3 1.0 in every coded dim
    rec[576:583] = 124 + np.arange(7, dtype=np.uint8)     # scales 2^-3 .. 2^3
    rope = np.linspace(-3, 3, 64).astype(np.float32)
    rec[448:576] = wl.bf16_bits(rope).view(np.uint8)
    k = orc.decode_slot(c, 0)
    assert np.array_equal(k[:448], np.repeat(2.0 ** (np.arange(7) - 3), 64))
    assert np.array_equal(k[448:], wl.bf16_round(rope).astype(np.float64))
    rec[583] = 0xFF                                       # the pad byte
    rec[63:65] = 0xB8                                     # dims 63 (scale 0) and 64 (scale 1): e4m3 -1.0
    k2 = orc.decode_slot(c, 0)
    assert k2[63] == -(2.0 ** -3) and k2[64] == -(2.0 ** -2)
    k2[63:65] = k[63:65]
    assert np.array_equal(k2, k)


def test_ue8m0_equals_fp32_scales_when_a_group_shares_one(orc):
    """A record whose four scale bytes of each 128-dim group are equal decodes, and attends, exactly like
    the FP8_528 record with those powers of two as its fp32 group scales."""
    w = _w(21, fmt=wl.FP8_UE8M0)
    c = w.cache
    n = c.num_slots
    recs = c.data.reshape(c.num_pages, c.page_stride)[:, : c.page_size * 528].reshape(n, 528)
    recs[:, 512:528] = np.repeat(recs[:, 512:528:4], 4, axis=1)    # one exponent per 128 dims
    w2 = copy.deepcopy(w)
    c2 = w2.cache
    c2.fmt = wl.FP8_528
    r2 = c2.data.reshape(c2.num_pages, c2.page_stride)[:, : c2.page_size * 528].reshape(n, 528)
    r2[:, 512:528] = np.exp2(recs[:, 512:528:4].astype(np.float64) - 127).astype(np.float32).view(np.uint8).reshape(n, 16)
    for s in (0, 5, n - 1):
        assert np.array_equal(orc.decode_slot(c, s), orc.decode_slot(c2, s))
    o1, l1 = orc.attention(w)
    o2, l2 = orc.attention(w2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_slot_range_masking(orc):
    c = wl.make_cache(np.random.default_rng(1), wl.FP8_528, 128, page_size=32)
    assert orc.decode_slot(c, -1) is None
    assert orc.decode_slot(c, 128) is None
    assert orc.decode_slot(c, 1 << 30) is None
    assert orc.decode_slot(c, 127) is not None
    assert orc.decode_slot(c, 0) is not None


def test_bf16_rne_against_torch(orc):
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(orc.bf16_rne(x.astype(np.float64)), ref)
    # exact ties: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 -> even (1.0)
    assert orc.bf16_rne(np.array([1 + 2.0 ** -8]))[0] == 1.0
    assert orc.bf16_rne(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6
    # a float64 value just above the tie must round up (a float32 detour would lose it)
    assert orc.bf16_rne(np.array([1 + 2.0 ** -8 + 2.0 ** -40]))[0] == 1 + 2.0 ** -7


# ------------------------------------------------------------------ attention: textbook reduction

def _sdpa_reference(w, t):
    """torch SDPA (float64, CPU) over the full width with a -inf mask for masked entries."""
    L = w.lst
    n = int(np.clip(L.lens[t], 0, L.width))
    sids = L.idx[t, :L.width]
    keep = np.array([(j < n) and (0 <= s < w.cache.num_slots) for j, s in enumerate(sids)])
    safe = np.where(keep, sids, 0)
    K = torch.from_numpy(decode_rows(w.cache, safe))                       # [W, d]
    q = torch.from_numpy(q_f64(w)[t])                                       # [H, d]
    mask = torch.zeros(1, L.width, dtype=torch.float64)
    mask[0, torch.from_numpy(~keep)] = float("-inf")
    out = torch.nn.functional.scaled_dot_product_attention(
        q[:, None, :], K[None].expand(w.H, -1, -1), K[None, :, :w.d_v].expand(w.H, -1, -1),
        attn_mask=mask.expand(w.H, 1, -1), scale=w.scale)[:, 0, :]
    scores = (q @ K.T) * w.scale + mask
    lse = torch.logsumexp(scores, dim=-1)
    return out.numpy(), lse.numpy(), keep.sum()


def test_matches_torch_sdpa_fp8_slotscale(orc):
    w = wl.make_workload("c1_tiny_swa", seed=11)
    w.lst.lens[:] = [128, 77, 3, 40]
    out, lse = orc.attention(w)
    for t in range(w.T):
        o_ref, l_ref, nvalid = _sdpa_reference(w, t)
        assert nvalid > 0
        np.testing.assert_allclose(out[t], o_ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[t], l_ref, rtol=0, atol=1e-12)


def test_bruteforce_tiny(orc):
    """Independent pure-Python loop (math.fsum, decoding through refdecode) on a tiny mixed case."""
    w = wl.small_workload(7, wl.FP8_528, wl.NVFP4_288, T=3, H=2, width=6, xwidth=5, num_slots=64,
                          page_size=8, pad_bytes=32, p_invalid=0.3, sink=True)
    out, lse = orc.attention(w)
    q = q_f64(w)
    for t in range(w.T):
        rows = [decode_rows(c, [s])[0] for c, s in valid_rows(w, t)]
        for h in range(w.H):
            zs = [w.scale * math.fsum(q[t, h, d] * r[d] for d in range(w.d_qk)) for r in rows]
            sk = float(w.sink[h])
            M = max(zs + [sk])
            ws = [math.exp(z - M) for z in zs]
            den = math.fsum(ws + [math.exp(sk - M)])
            ref = [math.fsum(wi * r[d] for wi, r in zip(ws, rows)) / den for d in range(w.d_v)]
            np.testing.assert_allclose(out[t, h], ref, rtol=0, atol=1e-12)
            assert abs(lse[t, h] - (M + math.log(den))) < 1e-12


# ------------------------------------------------------------------ invariants

def _w(seed=0, fmt=wl.FP8_528, xfmt=None, sink=False, **kw):
    args = dict(T=4, H=4, width=24, xwidth=16, num_slots=256, page_size=16, p_invalid=0.2, lens_lo=3)
    args.update(kw)
    return wl.small_workload(seed, fmt, xfmt, sink=sink, **args)


def test_permuting_the_list_changes_nothing(orc):
    w = _w(1, xfmt=wl.FP8_528)
    out, lse = orc.attention(w)
    rng = np.random.default_rng(2)
    w2 = copy.deepcopy(w)
    for L in (w2.lst, w2.xlst):
        for t in range(w.T):
            n = int(np.clip(L.lens[t], 0, L.width))
            L.idx[t, :n] = L.idx[t, :n][rng.permutation(n)]
    out2, lse2 = orc.attention(w2)
    np.testing.assert_allclose(out2, out, atol=1e-13, rtol=0)
    np.testing.assert_allclose(lse2, lse, atol=1e-13, rtol=0)


def _compact(w):
    """Rewrite every list so that masked entries are removed and lens counts only valid rows."""
    w2 = copy.deepcopy(w)
    for cache, L in w2.lists():
        for t in range(w.T):
            n = int(np.clip(L.lens[t], 0, L.width))
            keep = [int(s) for s in L.idx[t, :n] if 0 <= s < cache.num_slots]
            L.idx[t, :] = -1
            L.idx[t, :len(keep)] = keep
            L.lens[t] = len(keep)
    return w2


def test_masked_entries_equal_removal(orc):
    w = _w(3, xfmt=wl.FP8_528, sink=True)
    w.lst.idx[0, 0] = w.cache.num_slots          # out of range -> masked
    w.lst.idx[1, 1] = -7                         # any negative -> masked
    out, lse = orc.attention(w)
    out2, lse2 = orc.attention(_compact(w))
    np.testing.assert_allclose(out2, out, atol=1e-13, rtol=0)
    np.testing.assert_allclose(lse2, lse, atol=1e-13, rtol=0)


def test_entries_beyond_lens_are_ignored_and_lens_clamp(orc):
    w = _w(4)
    out, lse = orc.attention(w)
    w2 = copy.deepcopy(w)
    rng = np.random.default_rng(9)
    for t in range(w.T):
        n = int(w.lst.lens[t])
        w2.lst.idx[t, n:] = rng.integers(0, w.cache.num_slots, size=w.lst.width - n)
    out2, lse2 = orc.attention(w2)
    np.testing.assert_array_equal(out2, out)
    np.testing.assert_array_equal(lse2, lse)
    w3 = copy.deepcopy(w)
    w3.lst.lens[:] = 10 ** 6
    w4 = copy.deepcopy(w)
    w4.lst.lens = None
    np.testing.assert_array_equal(orc.attention(w3)[0], orc.attention(w4)[0])
    w5 = copy.deepcopy(w)
    w5.lst.lens[:] = -5
    o5, l5 = orc.attention(w5)
    assert np.all(o5 == 0) and np.all(l5 == -np.inf)


@pytest.mark.parametrize("qpl", [2, 3])
def test_request_lengths_shared_by_its_queries(orc, qpl):
    """Lengths per request [b] with q [b][s_q] (FlashMLA sparse_decode.h, topk_length): query t of the
    flattened tokens uses entry t // s_q; positions past it are ignored for every query of the request."""
    w = _w(31, xfmt=wl.FP8_528, sink=True, T=7)
    nreq = -(-w.T // qpl)
    rng = np.random.default_rng(31)
    g = copy.deepcopy(w)
    g.lst.lens = rng.integers(0, w.lst.width + 1, size=nreq).astype(np.int32)
    g.xlst.lens = rng.integers(0, w.xlst.width + 1, size=nreq).astype(np.int32)
    g.lst.queries_per_len = g.xlst.queries_per_len = qpl
    e = copy.deepcopy(w)
    r = np.arange(w.T) // qpl
    e.lst.lens, e.xlst.lens = g.lst.lens[r].copy(), g.xlst.lens[r].copy()
    og, lg = orc.attention(g)
    oe, le = orc.attention(e)
    np.testing.assert_array_equal(og, oe)
    np.testing.assert_array_equal(lg, le)
    for t in range(w.T):
        n = int(g.lst.lens[t // qpl])
        g.lst.idx[t, n:] = rng.integers(0, w.cache.num_slots, size=w.lst.width - n)
    np.testing.assert_array_equal(orc.attention(g)[0], og)
    g.lst.lens = g.lst.lens[:nreq - 1]
    with pytest.raises(ValueError):
        orc.attention(g)


def test_lens_zero_gives_zero_output_and_sink_lse(orc):
    w = _w(5, sink=True)
    w.lst.lens[:] = 0
    out, lse = orc.attention(w)
    assert np.all(out == 0)
    np.testing.assert_array_equal(lse, np.broadcast_to(w.sink.astype(np.float64), lse.shape))
    out, lse = orc.attention(w, sink=None)
    assert np.all(out == 0) and np.all(lse == -np.inf)


@pytest.mark.parametrize("fmt", [wl.FP8_SLOTSCALE, wl.FP8_528, wl.NVFP4_288, wl.V32_656, wl.FP8_UE8M0,
                                 wl.MODEL1_584])
def test_single_valid_slot_returns_its_row(orc, fmt):
    w = _w(6, fmt=fmt, width=8)
    w.lst.idx[:, :] = -1
    sids = [3, 100, 255, 17]
    for t in range(w.T):
        w.lst.idx[t, t % 8] = sids[t]
        w.lst.lens[t] = 8
    out, lse = orc.attention(w)
    q = q_f64(w)
    for t in range(w.T):
        k = decode_rows(w.cache, [sids[t]])[0]
        for h in range(w.H):
            np.testing.assert_array_equal(out[t, h], k[:w.d_v])
            z = w.scale * float(np.dot(q[t, h], k))
            assert abs(lse[t, h] - z) < 1e-12


def test_zero_query_averages_rows(orc):
    w = _w(7, xfmt=wl.FP8_528)
    w.q[:] = 0
    out, lse = orc.attention(w)
    for t in range(w.T):
        rows = np.concatenate([decode_rows(c, [s]) for c, s in valid_rows(w, t)])
        np.testing.assert_allclose(out[t], np.broadcast_to(rows[:, :w.d_v].mean(0), out[t].shape), atol=1e-12)
        np.testing.assert_allclose(lse[t], np.log(len(rows)), atol=1e-13)


def test_two_rows_logistic_weights(orc):
    w = _w(8, width=4)
    w.lst.idx[:, :] = -1
    w.lst.idx[:, 0] = 11
    w.lst.idx[:, 2] = 200
    w.lst.lens[:] = 4
    out, lse = orc.attention(w)
    k = decode_rows(w.cache, [11, 200])
    q = q_f64(w)
    for t in range(w.T):
        for h in range(w.H):
            z1, z2 = (w.scale * (k @ q[t, h]))
            a = 1.0 / (1.0 + math.exp(z2 - z1))
            np.testing.assert_allclose(out[t, h], a * k[0, :512] + (1 - a) * k[1, :512], atol=1e-12)
            assert abs(lse[t, h] - np.logaddexp(z1, z2)) < 1e-12


def test_duplicate_slot_adds_ln2(orc):
    w = _w(9, width=6)
    w.lst.idx[:, :] = -1
    w.lst.idx[:, 1] = 42
    w.lst.lens[:] = 6
    out1, lse1 = orc.attention(w)
    w.lst.idx[:, 4] = 42
    out2, lse2 = orc.attention(w)
    np.testing.assert_allclose(out2, out1, atol=1e-13)
    np.testing.assert_allclose(lse2, lse1 + math.log(2.0), atol=1e-13)


def test_sink_closed_form(orc):
    w = _w(10, xfmt=wl.NVFP4_288, sink=True)
    out_s, lse_s = orc.attention(w)
    out, lse = orc.attention(w, sink=None)
    s = w.sink.astype(np.float64)[None, :]
    ref_lse = np.logaddexp(lse, s)
    frac = np.exp(lse - ref_lse)
    np.testing.assert_allclose(lse_s, ref_lse, atol=1e-13)
    np.testing.assert_allclose(out_s, out * frac[:, :, None], atol=1e-13)


# ------------------------------------------------------------------ out_abs (the tolerance scale)

def test_out_abs_bounds_and_closed_forms(orc):
    """orc_attn_abs: the weighted mean of |v| under the output's own weights. It bounds |out| (triangle
    inequality), returns |row| for a single valid row, matches a math.fsum brute force, and with two rows
    is the logistic mix of their magnitudes."""
    w = _w(30, xfmt=wl.NVFP4_288, sink=True)
    out, lse, oabs = orc.attention(w, with_abs=True)
    out2, lse2 = orc.attention(w)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)
    assert np.all(oabs >= np.abs(out) - 1e-15 * np.abs(out)) and np.all(oabs >= 0)
    # brute force of token 1 with the sink
    q = q_f64(w)
    rows = np.concatenate([decode_rows(c, [s]) for c, s in valid_rows(w, 1)])
    for h in range(w.H):
        z = [w.scale * float(np.dot(q[1, h], r)) for r in rows]
        sk = float(w.sink[h])
        M = max(z + [sk])
        ws = [math.exp(zi - M) for zi in z]
        den = math.fsum(ws + [math.exp(sk - M)])
        ref = [math.fsum(wi * abs(r[d]) for wi, r in zip(ws, rows)) / den for d in range(w.d_v)]
        np.testing.assert_allclose(oabs[1, h], ref, rtol=0, atol=1e-12)
    # a single valid row: its magnitudes
    w = _w(31, width=8)
    w.lst.idx[:, :] = -1
    w.lst.idx[:, 2] = 77
    w.lst.lens[:] = 8
    _, _, oabs = orc.attention(w, with_abs=True)
    k = decode_rows(w.cache, [77])[0]
    for t in range(w.T):
        np.testing.assert_allclose(oabs[t], np.broadcast_to(np.abs(k[:512]), oabs[t].shape), rtol=1e-15)
    # two rows: a |k0| + (1 - a) |k1|
    w = _w(32, width=4)
    w.lst.idx[:, :] = -1
    w.lst.idx[:, 0] = 5
    w.lst.idx[:, 3] = 150
    w.lst.lens[:] = 4
    _, _, oabs = orc.attention(w, with_abs=True)
    k = decode_rows(w.cache, [5, 150])
    q = q_f64(w)
    for t in range(w.T):
        for h in range(w.H):
            z1, z2 = (w.scale * (k @ q[t, h]))
            a = 1.0 / (1.0 + math.exp(z2 - z1))
            np.testing.assert_allclose(oabs[t, h], a * np.abs(k[0, :512]) + (1 - a) * np.abs(k[1, :512]), atol=1e-12)
    # empty tokens: zeros
    w = _w(33, sink=True)
    w.lst.lens[:] = 0
    _, _, oabs = orc.attention(w, with_abs=True)
    assert np.all(oabs == 0)


def test_sink_infinities(orc):
    w = _w(11)
    out, lse = orc.attention(w, sink=None)
    o2, l2 = orc.attention(w, sink=np.full(w.H, -np.inf, dtype=np.float32))
    np.testing.assert_array_equal(o2, out)
    np.testing.assert_array_equal(l2, lse)
    o3, l3 = orc.attention(w, sink=np.full(w.H, np.inf, dtype=np.float32))
    assert np.all(o3 == 0) and np.all(l3 == np.inf)


def test_query_scale_invariance(orc):
    w = _w(12, fmt=wl.V32_656)
    out, lse = orc.attention(w)
    w2 = copy.deepcopy(w)
    w2.q = wl.bf16_bits(bf16_torch(w.q.reshape(-1)).reshape(w.q.shape).astype(np.float32) * 4.0)
    out2, lse2 = orc.attention(w2, scale=w.scale / 4.0)
    np.testing.assert_allclose(out2, out, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, atol=1e-13)


def test_main_plus_extra_equals_one_concatenated_list(orc):
    w = _w(13, fmt=wl.FP8_528, xfmt=wl.FP8_528, sink=True)
    w.xcache = w.cache                                   # same cache for both lists
    w.xlst.idx = np.where(w.xlst.idx >= 0, w.xlst.idx % w.cache.num_slots, -1).astype(np.int32)
    out, lse = orc.attention(w)
    W = w.lst.width + w.xlst.width
    idx = np.full((w.T, W), -1, dtype=np.int32)
    lens = np.zeros(w.T, dtype=np.int32)
    for t in range(w.T):
        a = w.lst.idx[t, :w.lst.lens[t]]
        b = w.xlst.idx[t, :w.xlst.lens[t]]
        idx[t, :len(a) + len(b)] = np.concatenate([a, b])
        lens[t] = len(a) + len(b)
    w1 = copy.deepcopy(w)
    w1.lst = wl.SlotList(idx, W, lens)
    w1.xcache = w1.xlst = None
    out1, lse1 = orc.attention(w1)
    np.testing.assert_allclose(out1, out, atol=1e-13)
    np.testing.assert_allclose(lse1, lse, atol=1e-13)


def test_page_stride_padding_is_transparent(orc):
    a = _w(14, fmt=wl.NVFP4_288, pad_bytes=0)
    b = _w(14, fmt=wl.NVFP4_288, pad_bytes=160)
    np.testing.assert_array_equal(orc.attention(a)[0], orc.attention(b)[0])


def test_threads_do_not_change_results(orc):
    w = _w(15, xfmt=wl.FP8_528, sink=True, T=9)
    o1, l1 = orc.attention(w, nthreads=1)
    o4, l4 = orc.attention(w, nthreads=4)
    np.testing.assert_array_equal(o1, o4)
    np.testing.assert_array_equal(l1, l4)


# ------------------------------------------------------------------ merge of split partials

@pytest.mark.parametrize("nparts", [2, 3, 5])
def test_merge_of_any_partition_equals_unsplit(orc, nparts):
    w = _w(20 + nparts, xfmt=wl.FP8_528, sink=True, T=3)
    out, lse = orc.attention(w)
    rng = np.random.default_rng(nparts)
    for t in range(w.T):
        tw = copy.deepcopy(w)
        tw.T = 1
        tw.q = w.q[t:t + 1]
        tw.lst = wl.SlotList(w.lst.idx[t:t + 1].copy(), w.lst.width, w.lst.lens[t:t + 1].copy())
        tw.xlst = wl.SlotList(w.xlst.idx[t:t + 1].copy(), w.xlst.width, w.xlst.lens[t:t + 1].copy())
        # assign every list position to a random part (some parts may end up empty)
        owner_m = rng.integers(0, nparts, size=w.lst.width)
        owner_x = rng.integers(0, nparts, size=w.xlst.width)
        o_parts, l_parts = [], []
        for p in range(nparts):
            pw = copy.deepcopy(tw)
            pw.lst.idx[0, owner_m != p] = -1
            pw.xlst.idx[0, owner_x != p] = -1
            o, l = orc.attention(pw, sink=None)
            o_parts.append(o[0])
            l_parts.append(l[0])
        mo, ml = orc.merge(np.array(o_parts), np.array(l_parts), w.sink)
        np.testing.assert_allclose(mo, out[t], atol=1e-12, rtol=0)
        np.testing.assert_allclose(ml, lse[t], atol=1e-12, rtol=0)


def test_merge_with_all_parts_empty(orc):
    H = 3
    o = np.zeros((2, H, 8))
    l = np.full((2, H), -np.inf)
    out, lse = orc.merge(o, l, None)
    assert np.all(out == 0) and np.all(lse == -np.inf)
    s = np.array([0.5, -1.0, 2.0], dtype=np.float32)
    out, lse = orc.merge(o, l, s)
    assert np.all(out == 0)
    np.testing.assert_array_equal(lse, s.astype(np.float64))


def test_oracle_rejects_inconsistent_arguments(orc):
    w = _w(30, fmt=wl.FP8_528, xfmt=wl.FP8_528)
    w.d_qk = 576
    with pytest.raises(ValueError):
        orc.attention(w)


# ------------------------------------------------------------------ V4.1 prologue and epilogue

def test_bf16_encoder_matches_torch(orc):
    L = orc.lib()
    rng = np.random.default_rng(40)
    x = np.concatenate([rng.standard_normal(3000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 3000),
                        # exact ties between two bf16 values (odd and even lower neighbours)
                        (np.arange(1, 200, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
                        np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38], dtype=np.float32)]).astype(np.float32)
    got = np.array([L.orc_bf16_rne(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(got, wl.bf16_bits(x))


def test_e4m3_encoder_matches_torch(orc):
    L = orc.lib()
    vals = e4m3_torch(np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8))
    vals = np.unique(vals)
    mids = (vals[1:] + vals[:-1]) / 2                    # ties: round to the even code
    rng = np.random.default_rng(41)
    x = np.concatenate([vals, mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf),
                        rng.uniform(-460, 460, 4000), rng.standard_normal(2000) * 1e-3]).astype(np.float32)
    got = np.array([L.orc_e4m3_encode(float(v)) for v in x], dtype=np.uint8)
    ref = wl.e4m3_codes(x)
    assert np.array_equal(got, ref)
    # beyond the largest value the cast saturates (the page's MXFP8 scale keeps |x| <= 448 up to rounding)
    for v in (448.5, 463.0, 1e6, np.inf):
        assert L.orc_e4m3_encode(v) == 0x7E and L.orc_e4m3_encode(-v) == 0xFE
    assert L.orc_e4m3_encode(float("nan")) == 0x7F


def _rotate(x, cos, sin, sign=1.0):
    """GPT-J pairs (2i, 2i+1) of x[..., 448:512] as complex numbers times exp(sign * i * angle), in float64."""
    z = x[..., 448:512:2] + 1j * x[..., 449:512:2]
    z = z * (cos + 1j * sign * sin)
    y = x.copy()
    y[..., 448:512:2] = z.real
    y[..., 449:512:2] = z.imag
    return y


def test_rope_q_is_the_rotation_of_gptj_pairs(orc):
    rng = np.random.default_rng(42)
    T, H = 6, 4
    q = wl.make_q(rng, T, H, 512)
    rope = wl.make_rope(rng, T, num_positions=512)
    rope.positions[0] = 0                                   # angle 0: identity
    rope.positions[1] = 512                                 # outside the table: identity
    rope.positions[2] = -1
    got = bf16_torch(orc.rope_q(q, rope.positions, rope.cos_sin))
    qf = bf16_torch(q)
    assert np.array_equal(got[:3], qf[:3])
    assert np.array_equal(got[:, :, :448], qf[:, :, :448])
    cs = rope.cos_sin[rope.positions[3:]].astype(np.float64)
    ref = _rotate(qf[3:], cs[:, None, :32], cs[:, None, 32:])
    ref_b = bf16_torch(wl.bf16_bits(ref.astype(np.float32)))
    # fp32 products and fma against the float64 rotation: equal after the bf16 rounding except where the
    # exact value sits within fp32 rounding of a bf16 midpoint (then one bf16 step)
    d = np.abs(got[3:] - ref_b)
    ulp = np.abs(ref_b) * 2.0 ** -7 + 1e-30
    assert np.all(d <= ulp)
    assert (d > 0).mean() < 1e-3


def test_mxfp8_scale_and_codes_closed_forms(orc):
    T, H = 1, 1
    pos = np.array([-1], dtype=np.int64)                    # identity rotation
    cs = np.zeros((1, 64), dtype=np.float32)
    out = np.zeros((T, H, 512))
    out[0, 0, 0:32] = 1.0                                   # amax 1: smallest 2^e >= 1/448 is 2^-8 -> byte 119
    out[0, 0, 32:64] = 448.0 * 2.0 ** -5                    # amax 448 * 2^k: scale exactly 2^k
    out[0, 0, 64] = 448.0 * 2.0 ** -5                       # ... and one step above it: scale 2^(k+1)
    out[0, 0, 65] = np.nextafter(np.float32(448.0 * 2.0 ** -5), np.float32(1e9))
    out[0, 0, 96:128] = np.linspace(-3, 3, 32)
    codes, sc = orc.mxfp8_out(out, pos, cs)
    assert sc[0, 0, 0] == 119 and np.all(codes[0, 0, 0:32] == 0x78)        # 1 * 2^8 = 256 = 0x78
    assert sc[0, 0, 1] == 127 - 5 and np.all(codes[0, 0, 32:64] == 0x7E)  # 448
    assert sc[0, 0, 2] == 127 - 4 and codes[0, 0, 64] == 0x76              # 224
    # all-zero chunks: amax is taken as 1e-10, codes 0
    assert np.all(codes[0, 0, 128:] == 0) and sc[0, 0, 5] == sc[0, 0, 15]
    e = sc[0, 0, 3].astype(np.float64) - 127
    assert 3.0 / 448 <= 2.0 ** e < 2 * 3.0 / 448
    np.testing.assert_allclose(e4m3_torch(codes[0, 0, 96:128]) * 2.0 ** e, out[0, 0, 96:128], rtol=2 ** -4)


def test_mxfp8_out_undoes_the_rotation_and_bounds_the_error(orc):
    """Results whose rope dims are u rotated by the position's angle come back as u (inverse RoPE), and every
    decoded value is within half an e4m3 step of the unrounded one; the scale is the smallest power of two
    that keeps the chunk within 448."""
    rng = np.random.default_rng(43)
    T, H = 5, 3
    rope = wl.make_rope(rng, T, num_positions=1000)
    u = rng.standard_normal((T, H, 512)) * 2.0 ** rng.integers(-6, 6, size=(T, H, 16)).repeat(32, axis=2)
    cs = rope.cos_sin[rope.positions].astype(np.float64)
    out = _rotate(u, cs[:, None, :32], cs[:, None, 32:])
    codes, sc = orc.mxfp8_out(out, rope.positions, rope.cos_sin)
    scale = 2.0 ** (sc.astype(np.float64) - 127)
    dec = e4m3_torch(codes.reshape(-1)).reshape(codes.shape) * scale.repeat(32, axis=2)
    amax = np.abs(u).reshape(T, H, 16, 32).max(axis=3)
    assert np.all(amax <= 448 * scale * (1 + 1e-6)) and np.all(amax > 224 * scale * (1 - 1e-6))
    # half a step of the value's binade (subnormal step below 2^-6), plus fp32 rounding of the rotation
    x = u / scale.repeat(32, axis=2)
    step = np.where(np.abs(x) < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(x), 1e-300))) - 3))
    err = np.abs(dec - u) / scale.repeat(32, axis=2)
    assert np.all(err <= step / 2 + np.abs(x) * 1e-6 + 1e-12)


def test_v41_with_identity_rotation_is_the_plain_decode_cast(orc):
    w = _w(44, fmt=wl.FP8_UE8M0, xfmt=wl.FP8_UE8M0, sink=True, T=5)
    w.rope = wl.make_rope(np.random.default_rng(1), w.T, num_positions=64)
    w.rope.positions[:] = 64                                   # outside the table
    codes, sc, lse, out, _ = orc.attention_v41(w)
    o, l = orc.attention(w)
    assert np.array_equal(out, o) and np.array_equal(lse, l)
    c2, s2 = orc.mxfp8_out(o, w.rope.positions, w.rope.cos_sin)
    assert np.array_equal(codes, c2) and np.array_equal(sc, s2)
    w.rope.positions[:] = 7
    codes3, _, lse3, _, _ = orc.attention_v41(w)
    assert not np.array_equal(lse3, l)                         # the rotation reaches the scores
