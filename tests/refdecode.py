"""Independent record decoding for the oracle's pins.

This decodes cache records with library routines (torch's float8_e4m3fn and
bfloat16 views) and the OCP e2m1 value table stored under tests/golden, so that
the oracle's own bit-level decoders are checked against something other than
themselves.
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def e2m1_table() -> np.ndarray:
    vals = np.zeros(16)
    with open(os.path.join(GOLDEN, "e2m1_ocp_table.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            c, v = line.split()
            vals[int(c)] = float(v)
    return vals


def layouts() -> dict:
    with open(os.path.join(GOLDEN, "record_layouts.json")) as f:
        return json.load(f)


def e4m3_torch(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()


def bf16_torch(bits: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).to(
        torch.float64).numpy()


def record_bytes(cache, sid: int) -> np.ndarray:
    page, off = divmod(int(sid), cache.page_size)
    start = page * cache.page_stride + off * cache.record_bytes
    return cache.data[start:start + cache.record_bytes]


def decode_rows(cache, sids) -> np.ndarray:
    """[n, d_qk] float64 rows of the given (valid) slot ids."""
    L = layouts()
    tab = e2m1_table()
    out = []
    for sid in sids:
        r = record_bytes(cache, sid)
        if cache.fmt == 0:  # FP8_SLOTSCALE
            out.append(e4m3_torch(r[:512]) * float(cache.slot_scale[sid]))
        elif cache.fmt in (1, 3):  # FP8_528 / V32_656
            g = L["v32_656"]["scale_group_dims"]
            sc = r[512:528].copy().view(np.float32).astype(np.float64)
            row = e4m3_torch(r[:512]) * np.repeat(sc, g)
            if cache.fmt == 3:
                row = np.concatenate([row, bf16_torch(r[528:656].copy().view(np.uint16))])
            out.append(row)
        elif cache.fmt == 4:  # FP8_UE8M0
            g = L["fp8_ue8m0_528"]["scale_group_dims"]
            e = r[512:528].astype(np.float64)
            sc = np.where(e == 255, np.nan, np.exp2(e - 127.0))
            out.append(e4m3_torch(r[:512]) * np.repeat(sc, g))
        elif cache.fmt == 5:  # MODEL1_584: the parts at the offsets of the stated part order
            lay = L["model1_584"]
            off, o = {}, 0
            for name, n in lay["parts"].items():
                off[name] = o
                o += n
            g = lay["scale_group_dims"]
            a = off["e4m3_codes"]
            e = r[off["ue8m0_scales"]:off["ue8m0_scales"] + lay["parts"]["ue8m0_scales"]].astype(np.float64)
            sc = np.where(e == 255, np.nan, np.exp2(e - 127.0))
            nope = e4m3_torch(r[a:a + lay["parts"]["e4m3_codes"]]) * np.repeat(sc, g)
            b = off["bf16_rope"]
            rope = bf16_torch(r[b:b + lay["parts"]["bf16_rope"]].copy().view(np.uint16))
            out.append(np.concatenate([nope, rope]))
        elif cache.fmt == 2:  # NVFP4_288
            packed = r[:256]
            nib = np.empty(512, dtype=np.int64)
            nib[0::2] = packed & 15
            nib[1::2] = packed >> 4
            sc = e4m3_torch(r[256:288])
            out.append(tab[nib] * np.repeat(sc, 16))
        else:
            raise ValueError(cache.fmt)
    return np.array(out, dtype=np.float64).reshape(len(out), -1)


def valid_rows(w, t: int):
    """(cache, sid) pairs of token t's valid rows, main list first, in list order."""
    rows = []
    for cache, L in w.lists():
        qpl = max(1, getattr(L, "queries_per_len", 1))
        n = L.width if L.lens is None else int(np.clip(L.lens[t // qpl], 0, L.width))
        for j in range(n):
            sid = int(L.idx[t, j])
            if 0 <= sid < cache.num_slots:
                rows.append((cache, sid))
    return rows


def q_f64(w) -> np.ndarray:
    return bf16_torch(w.q.reshape(-1)).reshape(w.q.shape)
