"""ctypes loader for the fp64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: tests, the smoke check and the benchmark's CPU
baseline use it; the library under test never imports it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into liboracle.so (no fast-math: IEEE double throughout)."""
    if force or not os.path.exists(LIB_PATH):
        src = os.path.join(_HERE, "oracle.c")
        tmp = LIB_PATH + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-Wall", "-o", tmp, src, "-lm"],
                       check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


class OrcCache(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("num_pages", ctypes.c_int64), ("page_size", ctypes.c_int32),
                ("page_stride", ctypes.c_int64), ("format", ctypes.c_int32), ("slot_scale", ctypes.c_void_p)]


class OrcList(ctypes.Structure):
    _fields_ = [("idx", ctypes.c_void_p), ("row_stride", ctypes.c_int64), ("width", ctypes.c_int32),
                ("lens", ctypes.c_void_p)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(LIB_PATH)
        L.orc_e4m3.restype = ctypes.c_double
        L.orc_e4m3.argtypes = [ctypes.c_int]
        L.orc_e2m1.restype = ctypes.c_double
        L.orc_e2m1.argtypes = [ctypes.c_int]
        L.orc_ue8m0.restype = ctypes.c_double
        L.orc_ue8m0.argtypes = [ctypes.c_int]
        L.orc_bf16.restype = ctypes.c_double
        L.orc_bf16.argtypes = [ctypes.c_int]
        L.orc_record_bytes.argtypes = [ctypes.c_int]
        L.orc_record_dims.argtypes = [ctypes.c_int]
        L.orc_decode_slot.argtypes = [ctypes.POINTER(OrcCache), ctypes.c_int64, ctypes.c_void_p]
        L.orc_attn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                               ctypes.c_int, ctypes.c_int, ctypes.POINTER(OrcCache), ctypes.POINTER(OrcList),
                               ctypes.POINTER(OrcCache), ctypes.POINTER(OrcList), ctypes.c_void_p, ctypes.c_float,
                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        L.orc_attn_abs.argtypes = L.orc_attn.argtypes[:-1] + [ctypes.c_void_p, ctypes.c_int]
        L.orc_merge.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.orc_bf16_rne.argtypes = [ctypes.c_float]
        L.orc_e4m3_encode.argtypes = [ctypes.c_float]
        L.orc_rope_q.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
        L.orc_mxfp8_out.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _cache_struct(c, keep):
    data = np.ascontiguousarray(c.data)
    ss = None if c.slot_scale is None else np.ascontiguousarray(c.slot_scale, dtype=np.float32)
    keep += [data, ss]
    return OrcCache(data.ctypes.data, c.num_pages, c.page_size, c.page_stride, c.fmt, _ptr(ss))


def token_lens(L, T: int) -> Optional[np.ndarray]:
    """Per-token lengths of list L over T tokens: token t takes entry t // queries_per_len (the queries
    of one request share its length: FlashMLA sparse_decode.h, topk_length [b] for indices [b][s_q])."""
    if L.lens is None:
        return None
    qpl = max(1, int(getattr(L, "queries_per_len", 1)))
    lens = np.asarray(L.lens, dtype=np.int32)
    if len(lens) < -(-T // qpl):
        raise ValueError("lengths hold fewer entries than the tokens need")
    return lens[np.arange(T) // qpl]


def _list_struct(L, keep, T, t0=0, t1=None):
    idx = np.ascontiguousarray(L.idx[t0:t1], dtype=np.int32)
    lt = token_lens(L, T)
    lens = None if lt is None else np.ascontiguousarray(lt[t0:t1], dtype=np.int32)
    keep += [idx, lens]
    return OrcList(idx.ctypes.data, idx.shape[1], L.width, _ptr(lens))


def decode_slot(cache, sid: int) -> Optional[np.ndarray]:
    keep = []
    cs = _cache_struct(cache, keep)
    dims = lib().orc_record_dims(cache.fmt)
    k = np.zeros(dims, dtype=np.float64)
    ok = lib().orc_decode_slot(ctypes.byref(cs), int(sid), k.ctypes.data)
    return k if ok else None


def attention(w, tokens: Optional[slice] = None, nthreads: int = 1, sink="default", scale: Optional[float] = None,
              with_abs: bool = False):
    """Oracle out [T, H, d_v] (float64) and lse [T, H] for workload `w` (or a slice of its tokens); with_abs adds
    out_abs [T, H, d_v], the weighted mean of the rows' magnitudes (orc_attn_abs)."""
    t0, t1 = (0, w.T) if tokens is None else (tokens.start or 0, tokens.stop if tokens.stop is not None else w.T)
    T = t1 - t0
    keep = []
    q = np.ascontiguousarray(w.q[t0:t1], dtype=np.uint16)
    keep.append(q)
    cs = _cache_struct(w.cache, keep)
    ls = _list_struct(w.lst, keep, w.T, t0, t1)
    xcs = xls = None
    if w.xcache is not None:
        xcs = _cache_struct(w.xcache, keep)
        xls = _list_struct(w.xlst, keep, w.T, t0, t1)
    snk = w.sink if isinstance(sink, str) else sink
    snk = None if snk is None else np.ascontiguousarray(snk, dtype=np.float32)
    keep.append(snk)
    out = np.zeros((T, w.H, w.d_v), dtype=np.float64)
    lse = np.zeros((T, w.H), dtype=np.float64)
    oabs = np.zeros((T, w.H, w.d_v), dtype=np.float64) if with_abs else None
    rc = lib().orc_attn_abs(q.ctypes.data, q.shape[1] * q.shape[2], q.shape[2], T, w.H, w.d_qk, w.d_v,
                            ctypes.byref(cs), ctypes.byref(ls),
                            ctypes.byref(xcs) if xcs is not None else None,
                            ctypes.byref(xls) if xls is not None else None,
                            _ptr(snk), ctypes.c_float(w.scale if scale is None else scale),
                            out.ctypes.data, lse.ctypes.data, _ptr(oabs), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return (out, lse, oabs) if with_abs else (out, lse)


def rope_q(q: np.ndarray, positions: np.ndarray, cos_sin: np.ndarray) -> np.ndarray:
    """q bf16 bits [T, H, 512] with dims 448..511 rotated by the positions' angles (bf16 bits, same shape)."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    T, H, d = q.shape
    assert d == 512
    pos = np.ascontiguousarray(positions, dtype=np.int64)
    cs = np.ascontiguousarray(cos_sin, dtype=np.float32)
    out = np.empty_like(q)
    lib().orc_rope_q(q.ctypes.data, H * d, d, T, H, pos.ctypes.data, cs.ctypes.data, cs.shape[1], cs.shape[0],
                     out.ctypes.data)
    return out


def mxfp8_out(out: np.ndarray, positions: np.ndarray, cos_sin: np.ndarray):
    """Inverse RoPE and MXFP8 cast of attention results out [T, H, 512] (float64): (codes uint8 [T, H, 512],
    scale bytes uint8 [T, H, 16])."""
    o = np.ascontiguousarray(out, dtype=np.float64)
    T, H, d = o.shape
    assert d == 512
    pos = np.ascontiguousarray(positions, dtype=np.int64)
    cs = np.ascontiguousarray(cos_sin, dtype=np.float32)
    codes = np.empty((T, H, 512), dtype=np.uint8)
    scales = np.empty((T, H, 16), dtype=np.uint8)
    lib().orc_mxfp8_out(o.ctypes.data, T, H, pos.ctypes.data, cs.ctypes.data, cs.shape[1], cs.shape[0],
                        codes.ctypes.data, scales.ctypes.data)
    return codes, scales


def attention_v41(w, tokens: Optional[slice] = None, nthreads: int = 1):
    """The V4.1 decode of workload `w` (which carries `rope`): Q RoPE, attention, inverse RoPE and the MXFP8
    output cast. Returns (codes [T, H, 512], scale bytes [T, H, 16], lse [T, H], out [T, H, 512] float64 before
    the cast, out_abs [T, H, 512] of orc_attn_abs) for all tokens or a slice of them."""
    import copy
    assert w.rope is not None and w.d_qk == 512
    w2 = copy.copy(w)
    w2.q = rope_q(w.q, w.rope.positions, w.rope.cos_sin)
    out, lse, oabs = attention(w2, tokens=tokens, nthreads=nthreads, with_abs=True)
    pos = w.rope.positions if tokens is None else w.rope.positions[tokens]
    codes, scales = mxfp8_out(out, pos, w.rope.cos_sin)
    return codes, scales, lse, out, oabs


def merge(o_parts: np.ndarray, lse_parts: np.ndarray, sink: Optional[np.ndarray]):
    """LSE-merge n normalized partials: o_parts [n, H, d_v], lse_parts [n, H] -> (out [H, d_v], lse [H])."""
    n, H, dv = o_parts.shape
    o = np.ascontiguousarray(o_parts, dtype=np.float64)
    l = np.ascontiguousarray(lse_parts, dtype=np.float64)
    s = None if sink is None else np.ascontiguousarray(sink, dtype=np.float32)
    out = np.zeros((H, dv), dtype=np.float64)
    lse = np.zeros(H, dtype=np.float64)
    lib().orc_merge(n, H, dv, o.ctypes.data, l.ctypes.data, _ptr(s), out.ctypes.data, lse.ctypes.data)
    return out, lse


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 (ties to even) and return them as float64.

    Done exactly from the float64 bit pattern (float64 -> float32 -> bf16 would round twice)."""
    x = np.asarray(x, dtype=np.float64)
    bits = x.view(np.uint64)
    # bf16 keeps 1+7 significand bits; float64 has 52 stored bits: drop 45.
    drop = np.uint64(45)
    lsb = (bits >> drop) & np.uint64(1)
    rounded = (bits + (np.uint64((1 << 44) - 1) + lsb)) >> drop << drop
    out = rounded.view(np.float64).copy()
    out[~np.isfinite(x)] = x[~np.isfinite(x)]
    # values beyond the bf16 range saturate to inf like a hardware conversion would
    big = np.abs(out) > 3.3895313892515355e38
    out[big] = np.copysign(np.inf, x[big])
    # bf16 subnormals: below 2^-126 the spacing is 2^-133; round there explicitly
    tiny = (np.abs(x) < 2.0 ** -126) & (x != 0)
    if tiny.any():
        q = np.ldexp(np.round(np.ldexp(x[tiny], 133)), -133)
        out[tiny] = q
    return out
