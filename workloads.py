"""Seeded synthetic inputs for paged, quantized, shared-KV decode attention.

This module only draws random numbers and lays bytes out in the cache record
formats. It holds none of the attention arithmetic and no decoder: both the
CPU oracle (``oracle/``) and the HIP library consume exactly the arrays made
here.

Record formats (bytes of one slot; ``page_stride`` bytes between pages):

* ``FP8_SLOTSCALE`` (512 B): 512 e4m3 codes; the dequant scale is a separate
  fp32 array indexed by slot id (native_swa_decode.py page: the batched
  gather + dequant pre-step multiplies the e4m3 row by ``inv_scale[slot]``).
* ``FP8_528`` (528 B): 512 e4m3 codes, then 4 little-endian fp32 scales, one
  per 128 dims.
* ``NVFP4_288`` (288 B): 256 bytes of packed e2m1 (low nibble = even
  element), then 32 e4m3 block scales, one per 16 dims (vLLM swapab_decode_attn
  page, ``stage_inputs``: NVFP4 chunk/scale mapping).
* ``V32_656`` (656 B): 512 e4m3 codes, 4 fp32 scales (per 128 dims), then 64
  bf16 values for dims 512..575 (FlashMLA sparse_decode.h page: the V3.2
  bytes-per-token sum 512 + 64*2 + 4*4).
* ``FP8_UE8M0`` (528 B): 512 e4m3 codes, then 16 ue8m0 scale bytes, byte g the
  power-of-two scale 2^(g - 127) of dims 32g..32g+31 (vLLM swapab_decode_attn
  page, stage_inputs: fp8 chunk c of 16 dims takes scale byte c // 2).
* ``MODEL1_584`` (584 B, d_qk = d_v = 512): 448 e4m3 codes (dims 0..447), 64 bf16
  values (dims 448..511), 7 ue8m0 scale bytes (byte g scales dims 64g..64g+63),
  one zero pad byte (FlashMLA sparse_decode.h page: the MODEL1 bytes-per-token
  sum 448 + 64*2 + 448/64 + 1; the parts in the order of that sum).

Quantization of the synthetic N(0,1) data: e4m3 by torch's float8_e4m3fn cast
after clipping to +-448 (round-to-nearest-even with saturation); FP8_UE8M0 rows
first get a random magnitude 2^U{-4..4} per 32-dim block, then each block the
scale exponent ceil(log2(amax / 448)) (the MXFP8 rule of the vLLM page's output
cast) and codes e4m3(x / scale); MODEL1_584 rows the same per 64-dim block of
dims 0..447, dims 448..511 bf16(N(0,1)); NVFP4 by the
usual recipe, block scale = e4m3(amax/6) and codes = round-to-nearest-even of
x/scale on the e2m1 grid, saturating at 6 (torch has no float->e2m1 cast, so
the grid rounding is written out here).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

FP8_SLOTSCALE, FP8_528, NVFP4_288, V32_656, FP8_UE8M0, MODEL1_584 = 0, 1, 2, 3, 4, 5
FORMAT_NAMES = {FP8_SLOTSCALE: "fp8_slotscale", FP8_528: "fp8_528", NVFP4_288: "nvfp4_288", V32_656: "v32_656",
                FP8_UE8M0: "fp8_ue8m0", MODEL1_584: "model1_584"}
RECORD_BYTES = {FP8_SLOTSCALE: 512, FP8_528: 528, NVFP4_288: 288, V32_656: 656, FP8_UE8M0: 528, MODEL1_584: 584}
D_QK = {FP8_SLOTSCALE: 512, FP8_528: 512, NVFP4_288: 512, V32_656: 576, FP8_UE8M0: 512, MODEL1_584: 512}


@dataclasses.dataclass
class Cache:
    fmt: int
    num_pages: int
    page_size: int
    page_stride: int            # bytes between consecutive pages
    data: np.ndarray            # uint8, num_pages * page_stride bytes
    slot_scale: Optional[np.ndarray] = None   # float32 [num_pages * page_size] (FP8_SLOTSCALE only)

    @property
    def num_slots(self) -> int:
        return self.num_pages * self.page_size

    @property
    def record_bytes(self) -> int:
        return RECORD_BYTES[self.fmt]


@dataclasses.dataclass
class SlotList:
    idx: np.ndarray             # int32 [T, row_stride]; only the first `width` columns are read
    width: int
    lens: Optional[np.ndarray]  # int32 [ceil(T / queries_per_len)] or None (= width)
    queries_per_len: int = 1    # consecutive tokens (the queries of one request) sharing a length entry


@dataclasses.dataclass
class Workload:
    name: str
    T: int
    H: int
    d_qk: int
    d_v: int
    q: np.ndarray               # uint16 bf16 bit patterns [T, H, d_qk]
    cache: Cache
    lst: SlotList
    xcache: Optional[Cache]
    xlst: Optional[SlotList]
    sink: Optional[np.ndarray]  # float32 [H] or None
    scale: float                # fp32 value
    rope: Optional["Rope"] = None   # V4.1 decode: Q RoPE, inverse RoPE and MXFP8 output

    def lists(self):
        out = [(self.cache, self.lst)]
        if self.xcache is not None:
            out.append((self.xcache, self.xlst))
        return out


@dataclasses.dataclass
class Rope:
    positions: np.ndarray       # int64 [T]: each token's position
    cos_sin: np.ndarray         # float32 [num_positions, 64]: row p = cos(p th_i) for i < 32, then sin(p th_i)


def make_rope(rng: np.random.Generator, T: int, num_positions: int = 8192, base: float = 10000.0) -> Rope:
    """Positions U{0..num_positions-1} and the usual RoPE table over 32 pairs, th_i = base^(-i/32), computed in
    float64 and stored as float32."""
    pos = rng.integers(0, num_positions, size=T).astype(np.int64)
    th = base ** (-np.arange(32, dtype=np.float64) / 32.0)
    ang = np.arange(num_positions, dtype=np.float64)[:, None] * th[None, :]
    cs = np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)
    return Rope(pos, cs)


# ----------------------------------------------------------------------------- quantizers

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (RNE, torch cast); return the uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 value (RNE), returned as float32."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.to(torch.float32).numpy()


def e4m3_codes(x: np.ndarray) -> np.ndarray:
    """float32 -> e4m3fn byte codes (RNE, saturating at +-448)."""
    x = np.clip(np.asarray(x, dtype=np.float32), -448.0, 448.0)
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _mx_blocks(rng: np.random.Generator, x: np.ndarray, block: int):
    """[n, d] float32 -> (codes [n, d] uint8, scale bytes [n, d / block] uint8): per block a random magnitude
    2^U{-4..4}, then the block's scale byte 127 + ceil(log2(amax / 448)) (clamped to 1..254) and codes
    e4m3(x / scale)."""
    n, d = x.shape
    nb = d // block
    blocks = x.reshape(n, nb, block) * np.exp2(rng.integers(-4, 5, size=(n, nb, 1))).astype(np.float32)
    amax = np.abs(blocks).max(axis=2)
    with np.errstate(divide="ignore"):
        ex = np.where(amax > 0, np.ceil(np.log2(amax / 448.0)), -127.0)
    ex = np.clip(ex, -126, 127).astype(np.int32)
    codes = e4m3_codes((blocks / np.exp2(ex)[:, :, None].astype(np.float32)).reshape(n, d))
    return codes, (ex + 127).astype(np.uint8)


def ue8m0_records(rng: np.random.Generator, x: np.ndarray) -> np.ndarray:
    """[n, 512] float32 -> [n, 528] FP8_UE8M0 records (one scale byte per 32 dims)."""
    codes, sb = _mx_blocks(rng, x, 32)
    return np.concatenate([codes, sb], axis=1)


def model1_records(rng: np.random.Generator, x: np.ndarray) -> np.ndarray:
    """[n, 512] float32 -> [n, 584] MODEL1_584 records: dims 0..447 as e4m3 with one scale byte per 64
    dims, dims 448..511 replaced by bf16(N(0,1)), one zero pad byte."""
    n = x.shape[0]
    codes, sb = _mx_blocks(rng, x[:, :448], 64)
    rope = bf16_bits(rng.standard_normal((n, 64), dtype=np.float32)).view(np.uint8).reshape(n, 128)
    return np.concatenate([codes, rope, sb, np.zeros((n, 1), dtype=np.uint8)], axis=1)


def e4m3_values(codes: np.ndarray) -> np.ndarray:
    """e4m3fn codes -> float32 via torch's cast (used only to build NVFP4 block scales)."""
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).to(torch.float32).numpy()


_E2M1_MID = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)


def e2m1_codes(y: np.ndarray) -> np.ndarray:
    """float32 -> 4-bit e2m1 codes, round to nearest with ties to the even code, saturating at 6."""
    a = np.abs(y).astype(np.float32)
    c = np.searchsorted(_E2M1_MID, a, side="left").astype(np.uint8)
    cm = np.minimum(c, 6)
    tie = (c < 7) & (a == _E2M1_MID[cm])
    c = np.where(tie & (c % 2 == 1), c + 1, c).astype(np.uint8)
    sign = ((y < 0) & (c != 0)).astype(np.uint8) << 3
    return (c | sign).astype(np.uint8)


def nvfp4_records(x: np.ndarray) -> np.ndarray:
    """x float32 [n, 512] -> uint8 [n, 288]: packed e2m1 (low nibble first) + 32 e4m3 block scales."""
    n = x.shape[0]
    blocks = x.reshape(n, 32, 16)
    amax = np.abs(blocks).max(axis=2)
    sc_codes = e4m3_codes(amax / 6.0)                    # [n, 32]
    sc_vals = e4m3_values(sc_codes)
    safe = np.where(sc_vals > 0, sc_vals, 1.0).astype(np.float32)
    y = blocks / safe[:, :, None]
    y = np.where(sc_vals[:, :, None] > 0, y, 0.0)
    nib = e2m1_codes(y.reshape(n, 512))
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return np.concatenate([packed, sc_codes.astype(np.uint8)], axis=1)


# ----------------------------------------------------------------------------- cache / list builders

def make_cache(rng: np.random.Generator, fmt: int, num_slots: int, page_size: int = 64,
               pad_bytes: int = 0, chunk: int = 16384) -> Cache:
    """A paged cache of `num_slots` records of N(0,1) data quantized in `fmt`.

    Per-slot / per-128-dim fp32 scales are U[0.5, 2]; bf16 rope dims are bf16(N(0,1)).
    `pad_bytes` extra bytes separate consecutive pages (page_stride > page_size * record).
    """
    assert num_slots % page_size == 0
    rec = RECORD_BYTES[fmt]
    num_pages = num_slots // page_size
    stride = page_size * rec + pad_bytes
    data = np.zeros(num_pages * stride, dtype=np.uint8)
    pages = data.reshape(num_pages, stride)[:, : page_size * rec].reshape(num_slots, rec) if pad_bytes == 0 else None
    recs = np.empty((num_slots, rec), dtype=np.uint8)
    for s0 in range(0, num_slots, chunk):
        n = min(chunk, num_slots - s0)
        x = rng.standard_normal((n, 512), dtype=np.float32)
        if fmt == NVFP4_288:
            recs[s0:s0 + n] = nvfp4_records(x)
            continue
        if fmt == FP8_UE8M0:
            recs[s0:s0 + n] = ue8m0_records(rng, x)
            continue
        if fmt == MODEL1_584:
            recs[s0:s0 + n] = model1_records(rng, x)
            continue
        recs[s0:s0 + n, :512] = e4m3_codes(x)
        if fmt in (FP8_528, V32_656):
            sc = rng.uniform(0.5, 2.0, size=(n, 4)).astype(np.float32)
            recs[s0:s0 + n, 512:528] = sc.view(np.uint8).reshape(n, 16)
        if fmt == V32_656:
            rope = bf16_bits(rng.standard_normal((n, 64), dtype=np.float32))
            recs[s0:s0 + n, 528:656] = rope.view(np.uint8).reshape(n, 128)
    if pages is not None:
        pages[:] = recs
    else:
        view = data.reshape(num_pages, stride)
        view[:, : page_size * rec] = recs.reshape(num_pages, page_size * rec)
        # padding bytes get a recognisable non-zero filler so that reading them shows up
        view[:, page_size * rec:] = 0x7F
    slot_scale = None
    if fmt == FP8_SLOTSCALE:
        slot_scale = rng.uniform(0.5, 2.0, size=num_slots).astype(np.float32)
    return Cache(fmt, num_pages, page_size, stride, data, slot_scale)


def make_list(rng: np.random.Generator, T: int, width: int, num_slots: int, lens_lo: int, lens_hi: int,
              p_invalid: float = 0.0, row_stride: Optional[int] = None) -> SlotList:
    """Per token `width` distinct random slots; each entry -1 w.p. p_invalid; lens ~ U{lo..hi}."""
    rs = width if row_stride is None else row_stride
    idx = np.full((T, rs), -1, dtype=np.int32)
    for t in range(T):
        idx[t, :width] = rng.choice(num_slots, size=width, replace=False).astype(np.int32)
    if p_invalid > 0:
        drop = rng.random((T, width)) < p_invalid
        idx[:, :width][drop] = -1
    lens = rng.integers(lens_lo, lens_hi + 1, size=T).astype(np.int32)
    return SlotList(idx, width, lens)


def make_q(rng: np.random.Generator, T: int, H: int, d_qk: int) -> np.ndarray:
    return bf16_bits(rng.standard_normal((T, H, d_qk), dtype=np.float32))


def make_sink(rng: np.random.Generator, H: int) -> np.ndarray:
    return bf16_round(rng.standard_normal(H, dtype=np.float32)).astype(np.float32)


# ----------------------------------------------------------------------------- the five configurations

CONFIGS = ("c1_tiny_swa", "c2_swa_h128", "c3_swa_fp8extra", "c4_swa_nvfp4extra", "c5_topk_v32", "c6_swa_ue8m0",
           "c7_swa_model1", "c8_v41_ue8m0")


def make_workload(name: str, seed: int = 0, T: Optional[int] = None, **kw) -> Workload:
    """Build one of the five decode configurations (or a smaller-T variant of it).

    c1_tiny_swa      4 tokens, 16 heads, d 512; 4096-slot FP8_SLOTSCALE cache (64 pages x 64);
                     128 distinct slots per token, 10% set to -1; lens U{0..128}; no sink.
    c2_swa_h128      64 tokens, 128 heads; same cache shape; 128 distinct slots; lens U{96..128}.
    c3_swa_fp8extra  256 tokens, 32 heads; SWA width 128 over a 32768-slot FP8_528 cache;
                     extra width 512 over a 65536-slot FP8_528 cache; lens U{1..W} per list; sink.
    c4_swa_nvfp4extra 512 tokens, 16 heads; SWA width 128 over a 65536-slot FP8_528 cache;
                     extra width 2048 over a 262144-slot NVFP4_288 cache; lens U{1..W}; sink.
    c5_topk_v32      128 tokens, 128 heads, d_qk 576; top-k width 2048 over a 131072-slot
                     V32_656 cache; lens = 2048; sink; scale 1/sqrt(576).
    c6_swa_ue8m0     c3's shape with both caches in FP8_UE8M0 (the fp8 record with one power-of-two
                     scale per 32 dims); a measurement workload for that format, not one of the five.
    c7_swa_model1    c3's shape with both caches in MODEL1_584 (448 fp8 dims with a power-of-two scale
                     per 64 dims, 64 bf16 dims); a measurement workload for that format.
    c8_v41_ue8m0     c6 (same draws) as the full V4.1 decode call: positions U{0..8191} and a RoPE table,
                     Q RoPE on dims 448..511, inverse RoPE and MXFP8 output.
    All pages hold 64 slots.
    """
    rng = np.random.default_rng(seed)
    pad = kw.get("pad_bytes", 0)
    if name == "c1_tiny_swa":
        T = 4 if T is None else T
        H, W = 16, 128
        q = make_q(rng, T, H, 512)
        cache = make_cache(rng, FP8_SLOTSCALE, 4096, 64, pad)
        lst = make_list(rng, T, W, 4096, 0, W, p_invalid=0.1)
        return Workload(name, T, H, 512, 512, q, cache, lst, None, None, None, float(np.float32(1 / math.sqrt(512))))
    if name == "c2_swa_h128":
        T = 64 if T is None else T
        H, W = 128, 128
        q = make_q(rng, T, H, 512)
        cache = make_cache(rng, FP8_SLOTSCALE, 4096, 64, pad)
        lst = make_list(rng, T, W, 4096, 96, W)
        return Workload(name, T, H, 512, 512, q, cache, lst, None, None, None, float(np.float32(1 / math.sqrt(512))))
    if name == "c3_swa_fp8extra":
        T = 256 if T is None else T
        H = 32
        q = make_q(rng, T, H, 512)
        cache = make_cache(rng, FP8_528, 32768, 64, pad)
        xcache = make_cache(rng, FP8_528, 65536, 64, pad)
        lst = make_list(rng, T, 128, 32768, 1, 128)
        xlst = make_list(rng, T, 512, 65536, 1, 512)
        sink = make_sink(rng, H)
        return Workload(name, T, H, 512, 512, q, cache, lst, xcache, xlst, sink, float(np.float32(1 / math.sqrt(512))))
    if name == "c4_swa_nvfp4extra":
        T = 512 if T is None else T
        H = 16
        q = make_q(rng, T, H, 512)
        cache = make_cache(rng, FP8_528, 65536, 64, pad)
        xcache = make_cache(rng, NVFP4_288, 262144, 64, pad)
        lst = make_list(rng, T, 128, 65536, 1, 128)
        xlst = make_list(rng, T, 2048, 262144, 1, 2048)
        sink = make_sink(rng, H)
        return Workload(name, T, H, 512, 512, q, cache, lst, xcache, xlst, sink, float(np.float32(1 / math.sqrt(512))))
    if name == "c5_topk_v32":
        T = 128 if T is None else T
        H, W = 128, 2048
        q = make_q(rng, T, H, 576)
        cache = make_cache(rng, V32_656, 131072, 64, pad)
        lst = make_list(rng, T, W, 131072, W, W)
        sink = make_sink(rng, H)
        return Workload(name, T, H, 576, 512, q, cache, lst, None, None, sink, float(np.float32(1 / math.sqrt(576))))
    if name == "c6_swa_ue8m0":
        T = 256 if T is None else T
        H = 32
        q = make_q(rng, T, H, 512)
        cache = make_cache(rng, FP8_UE8M0, 32768, 64, pad)
        xcache = make_cache(rng, FP8_UE8M0, 65536, 64, pad)
        lst = make_list(rng, T, 128, 32768, 1, 128)
        xlst = make_list(rng, T, 512, 65536, 1, 512)
        sink = make_sink(rng, H)
        return Workload(name, T, H, 512, 512, q, cache, lst, xcache, xlst, sink, float(np.float32(1 / math.sqrt(512))))
    if name == "c8_v41_ue8m0":
        w = make_workload("c6_swa_ue8m0", seed=seed, T=T, **kw)
        w.name = name
        w.rope = make_rope(np.random.default_rng([seed, 8]), w.T)
        return w
    if name == "c7_swa_model1":
        T = 256 if T is None else T
        H = 32
        q = make_q(rng, T, H, 512)
        cache = make_cache(rng, MODEL1_584, 32768, 64, pad)
        xcache = make_cache(rng, MODEL1_584, 65536, 64, pad)
        lst = make_list(rng, T, 128, 32768, 1, 128)
        xlst = make_list(rng, T, 512, 65536, 1, 512)
        sink = make_sink(rng, H)
        return Workload(name, T, H, 512, 512, q, cache, lst, xcache, xlst, sink, float(np.float32(1 / math.sqrt(512))))
    raise ValueError(f"unknown workload {name!r}")


def small_workload(seed: int, fmt: int, xfmt: Optional[int], T: int, H: int, width: int, xwidth: int = 0,
                   num_slots: int = 1024, page_size: int = 64, pad_bytes: int = 0, p_invalid: float = 0.1,
                   sink: bool = False, lens_lo: int = 0, row_stride_extra: int = 0,
                   xnum_slots: Optional[int] = None) -> Workload:
    """A small random workload of any format mix, for parity and edge-case tests."""
    rng = np.random.default_rng(seed)
    d_qk = D_QK[fmt]
    q = make_q(rng, T, H, d_qk)
    cache = make_cache(rng, fmt, num_slots, page_size, pad_bytes)
    lst = make_list(rng, T, width, num_slots, lens_lo, width, p_invalid, width + row_stride_extra)
    xcache = xlst = None
    if xfmt is not None:
        assert D_QK[xfmt] == d_qk
        xn = num_slots if xnum_slots is None else xnum_slots
        xcache = make_cache(rng, xfmt, xn, page_size, pad_bytes)
        xlst = make_list(rng, T, xwidth, xn, lens_lo, xwidth, p_invalid, xwidth + row_stride_extra)
    snk = make_sink(rng, H) if sink else None
    return Workload(f"small_f{fmt}_x{xfmt}_T{T}_H{H}", T, H, d_qk, 512, q, cache, lst, xcache, xlst, snk,
                    float(np.float32(1 / math.sqrt(d_qk))))
