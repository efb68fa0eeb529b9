"""The C ABI without a GPU: the library loads, exports what include/sda.h declares, rejects bad
arguments before touching the device, and its host scheduler partitions the work correctly."""
import ctypes
import os
import re

import numpy as np
import pytest

import sliding_window_decode_amd as sda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "sda.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(sda_[a-z_0-9]+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 10
    L = sda.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(sda.EXPORTED_SYMBOLS)


def test_status_strings():
    L = sda.lib()
    for st in (0, -1, -2, -3, -4):
        assert L.sda_status_string(st)
    assert L.sda_status_string(99) == b"unknown status"


def test_format_tables_match_generators():
    import workloads as wl
    L = sda.lib()
    for f, b in wl.RECORD_BYTES.items():
        assert L.sda_record_bytes(f) == b
        assert L.sda_format_dims(f) == wl.D_QK[f]
    assert L.sda_record_bytes(7) == -1


@pytest.mark.parametrize("T,H,dqk,W,X", [(4, 16, 512, 128, 0), (64, 128, 512, 128, 0), (256, 32, 512, 128, 512),
                                         (512, 16, 512, 128, 2048), (128, 128, 576, 2048, 0)])
def test_make_plan_and_workspace(T, H, dqk, W, X):
    plan = sda.make_plan(T, H, dqk, W, X)
    assert plan.num_parts >= 1 and H % plan.heads_per_group == 0 and plan.precision == 2
    ws = sda.workspace_bytes(T, H, 512, plan)
    assert ws >= (T + plan.num_parts) * H * 512 * 4 and ws % 256 == 0


def test_make_plan_rejects_unsupported():
    for args in [(4, 24, 512, 128, 0), (4, 16, 640, 128, 0), (0, 16, 512, 128, 0), (4, 16, 512, 0, 0)]:
        with pytest.raises(sda.SdaError):
            sda.make_plan(*args)


class _FakeTensor:
    """A stand-in exposing data_ptr/stride/shape; its address is never dereferenced because every call
    below fails validation on the host first."""

    def __init__(self, shape, ptr=1 << 20, strides=None, itemsize=2):
        self.shape = shape
        self._ptr = ptr
        self._strides = strides or tuple(int(np.prod(shape[i + 1:])) for i in range(len(shape)))
        self._itemsize = itemsize

    def data_ptr(self):
        return self._ptr

    def stride(self, i):
        return self._strides[i]

    def numel(self):
        return int(np.prod(self.shape))

    def element_size(self):
        return self._itemsize


def _call(q_shape=(4, 16, 512), fmt=sda.FP8_528, page_size=64, page_stride=None, width=128, H_out=16,
          extra=False, xfmt=None, plan=None, ws_bytes=None, q_ptr=1 << 20, slot_scale=False, meta=None, qpl=1):
    T, H, dqk = q_shape
    q = _FakeTensor(q_shape, ptr=q_ptr)
    rec = {0: 512, 1: 528, 2: 288, 3: 656}.get(fmt, 512)
    cache = sda.Cache(_FakeTensor((1,), 1 << 24), 16, page_size, page_stride or page_size * rec, fmt,
                      _FakeTensor((1,), 1 << 26) if slot_scale else None)
    lst = sda.SlotList(_FakeTensor((T, width), 1 << 27), width, None, qpl)
    xc = xl = None
    if extra:
        xrec = {0: 512, 1: 528, 2: 288, 3: 656}[xfmt]
        xc = sda.Cache(_FakeTensor((1,), 1 << 28), 16, 64, 64 * xrec, xfmt, None)
        xl = sda.SlotList(_FakeTensor((T, 64), 1 << 29), 64, None)
    if plan is None:
        plan = sda.sda_plan(8, 16, 2, 3)
    ws = _FakeTensor((ws_bytes if ws_bytes is not None else 1 << 30,), 1 << 30, itemsize=1)
    out = _FakeTensor((T, H_out, 512), 1 << 31)
    lse = _FakeTensor((T, H_out), 1 << 32, itemsize=4)
    ns = None if meta is None else _FakeTensor((T + 1,), 1 << 33)
    sda.sparse_decode_attn(q, cache, lst, xc, xl, None, 0.05, plan, meta, ns, ws, out, lse, stream=0)


@pytest.mark.parametrize("kw,status", [
    (dict(q_shape=(4, 24, 512)), sda.SDA_ERR_UNSUPPORTED),                 # H not supported
    (dict(q_shape=(4, 16, 576)), sda.SDA_ERR_UNSUPPORTED),                 # fp8_528 holds 512 dims
    (dict(q_shape=(4, 16, 640)), sda.SDA_ERR_UNSUPPORTED),                 # d_qk
    (dict(q_shape=(0, 16, 512)), sda.SDA_ERR_INVALID_ARG),                 # T
    (dict(page_size=48), sda.SDA_ERR_INVALID_ARG),                         # page size not a power of two
    (dict(page_stride=100), sda.SDA_ERR_INVALID_ARG),                      # page stride too small
    (dict(page_stride=64 * 528 + 8), sda.SDA_ERR_INVALID_ARG),             # page stride not a multiple of 16
    (dict(fmt=sda.FP8_SLOTSCALE), sda.SDA_ERR_INVALID_ARG),                # slot scale missing
    (dict(slot_scale=True), sda.SDA_ERR_INVALID_ARG),                      # slot scale given for fp8_528
    (dict(fmt=7), sda.SDA_ERR_UNSUPPORTED),                                # unknown format
    (dict(width=0), sda.SDA_ERR_INVALID_ARG),                              # width
    (dict(qpl=-2), sda.SDA_ERR_INVALID_ARG),                               # queries_per_len
    (dict(extra=True, xfmt=sda.V32_656), sda.SDA_ERR_UNSUPPORTED),         # extra cache d_qk mismatch
    (dict(plan=sda.sda_plan(0, 16, 2, 3)), sda.SDA_ERR_INVALID_ARG),       # num_parts
    (dict(plan=sda.sda_plan(8, 24, 2, 3)), sda.SDA_ERR_UNSUPPORTED),       # heads per group
    (dict(plan=sda.sda_plan(8, 16, 2, 4)), sda.SDA_ERR_INVALID_ARG),       # precision
    (dict(ws_bytes=1024), sda.SDA_ERR_WORKSPACE),                          # workspace too small
    (dict(q_ptr=(1 << 20) + 2), sda.SDA_ERR_INVALID_ARG),                  # q misaligned
    (dict(meta=True), sda.SDA_ERR_INVALID_ARG),                            # meta without num_splits
    (dict(q_shape=(1 << 21, 16, 512), plan=sda.sda_plan(8, 16, 1024, 3)),
     sda.SDA_ERR_UNSUPPORTED),                                              # tile positions reach 2^31
])
def test_decode_rejects_bad_arguments_on_the_host(kw, status):
    if kw.get("meta"):
        # num_splits given, meta missing
        T = 4
        plan = sda.sda_plan(8, 16, 2, 3)
        q = _FakeTensor((T, 16, 512))
        cache = sda.Cache(_FakeTensor((1,), 1 << 24), 16, 64, 64 * 528, sda.FP8_528, None)
        lst = sda.SlotList(_FakeTensor((T, 128), 1 << 27), 128, None)
        with pytest.raises(sda.SdaError) as ei:
            sda.sparse_decode_attn(q, cache, lst, None, None, None, 0.05, plan, None, _FakeTensor((T + 1,)),
                                   _FakeTensor((1 << 30,), 1 << 30, itemsize=1), _FakeTensor((T, 16, 512)),
                                   _FakeTensor((T, 16), itemsize=4), stream=0)
        assert ei.value.status == status
        return
    with pytest.raises(sda.SdaError) as ei:
        _call(**kw)
    assert ei.value.status == status
    assert sda.lib().sda_last_error()


def test_schedulers_reject_tile_positions_past_32_bits():
    """Both schedulers count tile positions in 32-bit integers: a call whose T x (tiles per token + F) reaches
    2^31 is refused before anything runs; one just below it is accepted by the host scheduler."""
    plan = sda.sda_plan(8, 16, 1024, 3)
    T = (1 << 31) // (2 + 1 + 1024) + 1   # width 128: two tiles a token, one empty-tile allowance, F = 1024
    with pytest.raises(sda.SdaError) as ei:
        sda.get_sched_meta_host(T, None, 128, None, 0, plan)
    assert ei.value.status == sda.SDA_ERR_UNSUPPORTED
    lst = sda.SlotList(_FakeTensor((T, 128), 1 << 27), 128, None)
    with pytest.raises(sda.SdaError) as ei:
        sda.get_sched_meta(T, lst, None, plan, _FakeTensor((8, 8), 1 << 28), _FakeTensor((T + 1,), 1 << 29), stream=0)
    assert ei.value.status == sda.SDA_ERR_UNSUPPORTED
    meta, ns = sda.get_sched_meta_host(T - 1, None, 128, None, 0, plan)
    assert ns[-1] >= T - 1


def test_extra_cache_without_list_is_rejected():
    L = sda.lib()
    T, H = 2, 16
    cc = sda.sda_cache(1 << 24, 4, 64, sda.FP8_528, 64 * 528, None)
    cl = sda.sda_list(1 << 27, 128, 128, 0, None)
    plan = sda.sda_plan(4, 16, 2, 3)
    rc = L.sda_sparse_decode_attn(1 << 20, 16 * 512, 512, T, H, 512, 512, ctypes.byref(cc), ctypes.byref(cl),
                                  ctypes.byref(cc), None, None, ctypes.c_float(0.1), ctypes.byref(plan), None, None,
                                  1 << 30, 1 << 30, 1 << 31, H * 512, 512, 1 << 32, H, None)
    assert rc == sda.SDA_ERR_INVALID_ARG


def test_combine_rejects_bad_arguments():
    L = sda.lib()
    assert L.sda_combine_splits(2, 16, 256, 1 << 20, 1 << 21, 1 << 22, None, 1 << 23, 8192, 512, 1 << 24, 16,
                                None) == sda.SDA_ERR_UNSUPPORTED
    assert L.sda_combine_splits(2, 16, 512, None, 1 << 21, 1 << 22, None, 1 << 23, 8192, 512, 1 << 24, 16,
                                None) == sda.SDA_ERR_INVALID_ARG
    # head counts the kernel's 16-head workgroups do not cover exactly
    for H in (1, 8, 17, 24, 48, 256):
        assert L.sda_combine_splits(2, H, 512, 1 << 20, 1 << 21, 1 << 22, None, 1 << 23, 8192, 512, 1 << 24, 256,
                                    None) == sda.SDA_ERR_UNSUPPORTED, H
    # out must be 16-byte aligned with strides in multiples of 8 elements (the kernel stores 8 bf16 per lane)
    for out, st, sh in [((1 << 23) + 8, 8192, 512), (1 << 23, 8196, 512), (1 << 23, 8192, 516),
                        (1 << 23, -8, 512), (1 << 23, 8192, 504)]:
        assert L.sda_combine_splits(2, 16, 512, 1 << 20, 1 << 21, 1 << 22, None, out, st, sh, 1 << 24, 16,
                                    None) == sda.SDA_ERR_INVALID_ARG, (out, st, sh)
    assert L.sda_combine_splits(2, 16, 512, (1 << 20) + 8, 1 << 21, 1 << 22, None, 1 << 23, 8192, 512, 1 << 24, 16,
                                None) == sda.SDA_ERR_INVALID_ARG


# ------------------------------------------------------------------ host scheduler

def _check_schedule(meta, ns, T, n0, n1, P):
    """Every (token, tile) is covered by exactly one part, in order; split counts match."""
    tiles = [max(1, -(-a // 64) + -(-b // 64)) for a, b in zip(n0, n1)]
    seq = [(t, i) for t in range(T) for i in range(tiles[t])]
    pos = {ti: k for k, ti in enumerate(seq)}
    covered = []
    touching = [set() for _ in range(T)]
    first_k = {}
    for p in range(P):
        bt, bi, et, ei, bk = meta[p, :5]
        b = pos[(bt, bi)] if bt < T else len(seq)
        e = pos[(et, ei)] if et < T else len(seq)
        assert b <= e
        for k in range(b, e):
            covered.append(seq[k])
            touching[seq[k][0]].add(p)
        if b < e:
            first_k[p] = bk
    assert covered == seq, "parts must tile the (token, tile) sequence in order"
    nsplit = [len(s) for s in touching]
    assert ns[0] == 0 and list(np.diff(ns)) == nsplit
    assert ns[T] <= T + P
    for t in range(T):
        for k, p in enumerate(sorted(touching[t])):
            bt = meta[p, 0]
            if bt == t:
                assert first_k[p] == k
    for p in range(P):
        bt, bi, et, ei = meta[p, :4]
        if bt < T:
            # the begin token's clamped lengths and first split index travel in the record
            assert (meta[p, 5], meta[p, 6], meta[p, 7]) == (n0[bt], n1[bt], ns[bt])
            # a part holds the whole of a token it touches exactly when the token has one split:
            # it starts at the token's first tile (or before) and ends after its last one
            for t in range(bt, min(et + (1 if ei > 0 else 0), T)):
                whole = (t != bt or bi == 0) and (t != et or ei == 0)
                assert whole == (nsplit[t] == 1)
        else:
            assert list(meta[p]) == [T, 0, T, 0, 0, 0, 0, 0]


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("P,F", [(1, 2), (7, 0), (64, 2), (256, 5), (1000, 1)])
def test_host_scheduler_partitions_every_tile_once(seed, P, F):
    rng = np.random.default_rng(seed)
    T = int(rng.integers(1, 300))
    W, X = 128, int(rng.choice([0, 512, 2048]))
    lens = rng.integers(-5, W + 20, size=T).astype(np.int32)
    xl = rng.integers(0, X + 1, size=T).astype(np.int32) if X else None
    plan = sda.sda_plan(P, 16, F, 3)
    meta, ns = sda.get_sched_meta_host(T, lens, W, xl, X, plan)
    n0 = np.clip(lens, 0, W)
    n1 = np.clip(xl, 0, X) if X else np.zeros(T, dtype=np.int32)
    _check_schedule(meta, ns, T, n0, n1, P)


def test_host_scheduler_balances_cost():
    T, W = 512, 2048
    rng = np.random.default_rng(0)
    lens = rng.integers(1, W + 1, size=T).astype(np.int32)
    plan = sda.sda_plan(256, 16, 2, 3)
    meta, ns = sda.get_sched_meta_host(T, lens, W, None, 0, plan)
    tiles = np.maximum(1, -(-lens // 64))
    total = int((tiles + 2).sum())
    Q = -(-total // 256)
    # each part holds at most Q tiles (the quantum), so the busiest part is within one quantum of the mean
    seq_pos = np.concatenate([[0], np.cumsum(tiles)])
    for p in range(256):
        bt, bi, et, ei = meta[p, :4]
        b = seq_pos[bt] + bi if bt < T else seq_pos[T]
        e = seq_pos[et] + ei if et < T else seq_pos[T]
        assert e - b <= Q


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("qpl", [0, 1, 2, 3, 7])
def test_host_scheduler_grouped_lengths_equal_expanded(seed, qpl):
    """A length entry shared by queries_per_len consecutive tokens schedules exactly like the same
    length repeated per token (the s_q queries of a request share its length)."""
    rng = np.random.default_rng(100 + seed)
    T = int(rng.integers(1, 200))
    g = max(qpl, 1)
    W, X = 128, 512
    nreq = -(-T // g)
    lens = rng.integers(-3, W + 5, size=nreq).astype(np.int32)
    xl = rng.integers(0, X + 3, size=nreq).astype(np.int32)
    plan = sda.sda_plan(int(rng.choice([3, 64, 256])), 16, 2, 3)
    m_g, ns_g = sda.get_sched_meta_host(T, lens, W, xl, X, plan, queries_per_len=qpl)
    e = np.arange(T) // g
    m_e, ns_e = sda.get_sched_meta_host(T, lens[e], W, xl[e], X, plan)
    assert np.array_equal(m_g, m_e) and np.array_equal(ns_g, ns_e)


def test_host_scheduler_rejects_negative_queries_per_len():
    plan = sda.sda_plan(4, 16, 2, 3)
    with pytest.raises(sda.SdaError) as ei:
        sda.get_sched_meta_host(4, None, 128, None, 0, plan, queries_per_len=-1)
    assert ei.value.status == sda.SDA_ERR_INVALID_ARG


class _V41Bufs:
    def __init__(self, T=4, H=16, cs_ptr=1 << 34, cs_stride=64, of_stride_h=512, os_stride_h=16, of_ptr=1 << 35):
        self.positions = _FakeTensor((T,), 1 << 36, itemsize=8)
        self.cos_sin = _FakeTensor((100, cs_stride), cs_ptr, strides=(cs_stride, 1), itemsize=4)
        self.out_fp8 = _FakeTensor((T, H, 512), of_ptr, strides=(H * of_stride_h, of_stride_h, 1), itemsize=1)
        self.out_scale = _FakeTensor((T, H, 16), 1 << 37, strides=(H * os_stride_h, os_stride_h, 1), itemsize=1)


def _call_v41(q_shape=(4, 16, 512), fmt=sda.FP8_UE8M0, ws_bytes=None, **kw):
    T, H, dqk = q_shape
    rec = {1: 528, 3: 656, 4: 528, 5: 584}[fmt]
    q = _FakeTensor(q_shape)
    cache = sda.Cache(_FakeTensor((1,), 1 << 24), 16, 64, 64 * rec, fmt, None)
    lst = sda.SlotList(_FakeTensor((T, 128), 1 << 27), 128, None)
    plan = sda.sda_plan(8, 16, 2, 2)
    need = sda.workspace_bytes_v41(T, H, plan)
    ws = _FakeTensor((need if ws_bytes is None else ws_bytes,), 1 << 30, itemsize=1)
    b = _V41Bufs(T, H, **kw)
    sda.sparse_decode_attn_v41(q, cache, lst, None, None, None, 0.05, plan, None, None, ws, b.positions, b.cos_sin,
                               b.out_fp8, b.out_scale, None, stream=0)


@pytest.mark.parametrize("kw,status", [
    (dict(fmt=sda.V32_656, q_shape=(4, 16, 576)), sda.SDA_ERR_UNSUPPORTED),  # V4.1 rows hold 512 dims
    (dict(cs_ptr=(1 << 34) + 4), sda.SDA_ERR_INVALID_ARG),                     # cos_sin misaligned
    (dict(cs_stride=48), sda.SDA_ERR_INVALID_ARG),                             # cos_sin row too short
    (dict(cs_stride=66), sda.SDA_ERR_INVALID_ARG),                             # stride not a multiple of 4
    (dict(of_stride_h=520), sda.SDA_ERR_INVALID_ARG),                          # out_fp8 stride not in 16s
    (dict(of_ptr=(1 << 35) + 8), sda.SDA_ERR_INVALID_ARG),                     # out_fp8 misaligned
    (dict(os_stride_h=8), sda.SDA_ERR_INVALID_ARG),                            # scale row too short
    (dict(ws_bytes=1024), sda.SDA_ERR_WORKSPACE),                              # workspace too small
])
def test_v41_rejects_bad_arguments_on_the_host(kw, status):
    with pytest.raises(sda.SdaError) as ei:
        _call_v41(**kw)
    assert ei.value.status == status


def test_v41_workspace_holds_the_rotated_q():
    plan = sda.sda_plan(64, 32, 2, 2)
    for T, H in ((1, 16), (256, 32), (64, 128)):
        assert sda.workspace_bytes_v41(T, H, plan) >= sda.workspace_bytes(T, H, 512, plan) + T * H * 128
    # the standard workspace is not enough for a V4.1 call
    with pytest.raises(sda.SdaError) as ei:
        _call_v41(ws_bytes=sda.workspace_bytes(4, 16, 512, sda.sda_plan(8, 16, 2, 2)))
    assert ei.value.status == sda.SDA_ERR_WORKSPACE


def test_whole_token_plans_on_the_host():
    """A whole-token plan takes no meta or num_splits, has no schedule, and whole_tokens is 0 or 1."""
    T = 4
    plan = sda.sda_plan(8, 16, 2, 3, 1)
    q = _FakeTensor((T, 16, 512))
    cache = sda.Cache(_FakeTensor((1,), 1 << 24), 16, 64, 64 * 528, sda.FP8_528, None)
    lst = sda.SlotList(_FakeTensor((T, 128), 1 << 27), 128, None)
    ws = _FakeTensor((1 << 30,), 1 << 30, itemsize=1)
    with pytest.raises(sda.SdaError) as ei:
        sda.sparse_decode_attn(q, cache, lst, None, None, None, 0.05, plan, _FakeTensor((8, 8), 1 << 34),
                               _FakeTensor((T + 1,), 1 << 33), ws, _FakeTensor((T, 16, 512)),
                               _FakeTensor((T, 16), itemsize=4), stream=0)
    assert ei.value.status == sda.SDA_ERR_INVALID_ARG and b"whole-token" in sda.lib().sda_last_error()
    with pytest.raises(sda.SdaError) as ei:
        _call(plan=sda.sda_plan(8, 16, 2, 3, 2))
    assert ei.value.status == sda.SDA_ERR_INVALID_ARG
    with pytest.raises(sda.SdaError) as ei:
        sda.get_sched_meta_host(T, np.full(T, 100, np.int32), 128, None, 0, plan)
    assert ei.value.status == sda.SDA_ERR_INVALID_ARG
    with pytest.raises(sda.SdaError) as ei:
        sda.get_sched_meta(T, lst, None, plan, _FakeTensor((8, 8), 1 << 34), _FakeTensor((T + 1,), 1 << 33), 0)
    assert ei.value.status == sda.SDA_ERR_INVALID_ARG
    assert sda.make_plan(64, 128, 512, 128).whole_tokens == 0


def _choose(T, H, d_qk, fmt, lens, width, xfmt=None, xlens=None, xwidth=0, v41=False, qpl=1):
    return sda.auto_plan(T, H, d_qk, width, xwidth if xfmt is not None else 0, lens, xlens, [fmt, xfmt], v41, qpl)


def test_choose_plan_makespan_rule():
    """sda_choose_plan: whole-token plan while its makespan in tiles (longest token, or the even share once
    tokens outnumber parts) is within 1.3x the split plan's plus two (1.0x plus one for V4.1)."""
    F8, F528 = sda.FP8_SLOTSCALE, sda.FP8_528
    # equal tokens, one per part (64 tokens of 2 tiles, 64 parts): whole, 16-head workgroups in one round
    p = _choose(64, 128, 512, F8, np.full(64, 100, np.int32), 128)
    assert (p.whole_tokens, p.heads_per_group, p.num_parts) == (1, 16, 64)
    # a handful of tokens on a GPU-wide split plan (768 parts of 16 heads): the two launches outweigh a tile
    p = _choose(4, 16, 512, F528, np.array([100, 50, 128, 90], np.int32), 128)
    assert (p.num_parts, p.fixed_overhead, p.whole_tokens, p.heads_per_group) == (768, 0, 1, 16)
    # tokens 2 and 10 tiles long (SWA + extra list shape): whole for the plain call, split for V4.1
    lens = np.r_[np.full(128, 128), np.full(128, 64)].astype(np.int32)
    xlens = np.r_[np.full(128, 512), np.full(128, 64)].astype(np.int32)
    p = _choose(256, 32, 512, F528, lens, 128, F528, xlens, 512)
    assert (p.num_parts, p.whole_tokens, p.heads_per_group) == (256, 1, 16)
    p = _choose(256, 32, 512, sda.FP8_UE8M0, lens, 128, sda.FP8_UE8M0, xlens, 512, v41=True)
    assert p.whole_tokens == 0 and p.heads_per_group == 32
    # one long token per workgroup against balanced parts (2 and 34 tiles over 768 parts): split
    lens = np.r_[np.full(256, 128), np.full(256, 64)].astype(np.int32)
    xlens = np.r_[np.full(256, 2048), np.full(256, 64)].astype(np.int32)
    p = _choose(512, 16, 512, F528, lens, 128, sda.NVFP4_288, xlens, 2048)
    assert (p.num_parts, p.whole_tokens) == (768, 0)
    # more tokens than parts: the even share bounds the whole-token makespan; two rounds keep 32 heads
    p = _choose(640, 128, 512, F8, None, 128)
    assert (p.num_parts, p.whole_tokens, p.heads_per_group) == (64, 1, 32)
    # lengths per request repeated over their queries: the same choice as the expanded lengths
    g = _choose(12, 32, 512, F528, np.array([128, 0, 64, 128], np.int32), 128, qpl=3)
    e = _choose(12, 32, 512, F528, np.repeat(np.array([128, 0, 64, 128], np.int32), 3), 128)
    assert (g.whole_tokens, g.heads_per_group, g.num_parts) == (e.whole_tokens, e.heads_per_group, e.num_parts)


def test_choose_plan_head_grouping():
    """16 heads per workgroup only for whole-token calls on the fp8 ring kernel with 512-dim records (no NVFP4 or
    MODEL1 list, ue8m0 lists only with one another) whose T x H/16 workgroups fit two per CU."""
    L = np.full(256, 128, np.int32)
    F528, UE, M1, F4 = sda.FP8_528, sda.FP8_UE8M0, sda.MODEL1_584, sda.NVFP4_288
    assert _choose(256, 32, 512, F528, L, 128, F528, L, 128).heads_per_group == 16
    assert _choose(256, 32, 512, UE, L, 128, UE, L, 128).heads_per_group == 16
    assert _choose(256, 32, 512, UE, L, 128, F528, L, 128).heads_per_group == 32   # staged kernel
    assert _choose(256, 32, 512, M1, L, 128, M1, L, 128).heads_per_group == 32     # 592-byte ring rows
    assert _choose(256, 32, 512, F528, L, 128, F4, L, 128).heads_per_group == 32   # staged kernel
    p = _choose(128, 128, 576, sda.V32_656, None, 2048)
    assert (p.whole_tokens, p.heads_per_group) == (1, 64)


def test_choose_plan_rejects_bad_arguments():
    for kw, status in [(dict(fmt=9), sda.SDA_ERR_UNSUPPORTED), (dict(fmt=sda.V32_656), sda.SDA_ERR_UNSUPPORTED),
                       (dict(xfmt=sda.V32_656, xwidth=64), sda.SDA_ERR_UNSUPPORTED),
                       (dict(H=24), sda.SDA_ERR_UNSUPPORTED), (dict(T=0), sda.SDA_ERR_INVALID_ARG),
                       (dict(qpl=-1), sda.SDA_ERR_INVALID_ARG)]:
        args = dict(T=4, H=16, d_qk=512, fmt=sda.FP8_528, lens=None, width=64)
        args.update(kw)
        with pytest.raises(sda.SdaError) as ei:
            _choose(**args)
        assert ei.value.status == status, kw
    # extra lengths without an extra list
    plan = sda.sda_plan()
    L = np.full(4, 10, np.int32)
    rc = sda.lib().sda_choose_plan(4, 16, 512, sda.FP8_528, None, 64, sda.FP8_528, L.ctypes.data, 0, 1, 0, 256,
                                   ctypes.byref(plan))
    assert rc == sda.SDA_ERR_INVALID_ARG


def test_choose_plan_on_the_benchmark_workloads():
    """The plan bench.py times, on the host-side lengths of each workload: whole-token plans except where one
    long token (C4) or the V4.1 epilogue (c8) favours the split schedule; 16 heads per workgroup only on fp8
    ring-kernel calls with 512-dim records."""
    import workloads as wl
    from sliding_window_decode_amd.inputs import plan_for

    want = {"c1_tiny_swa": (1, 16), "c2_swa_h128": (1, 16), "c3_swa_fp8extra": (1, 16),
            "c4_swa_nvfp4extra": (0, None), "c5_topk_v32": (1, 64), "c6_swa_ue8m0": (1, 16),
            "c7_swa_model1": (1, 32), "c8_v41_ue8m0": (0, None)}
    for name, (whole, hb) in want.items():
        w = wl.make_workload(name, seed=0)
        X = w.xlst.width if w.xlst is not None else 0
        plan = plan_for(w)
        split = sda.make_plan(w.T, w.H, w.d_qk, w.lst.width, X)
        assert plan.whole_tokens == whole, name
        assert plan.heads_per_group == (hb if whole else split.heads_per_group), name
        assert (plan.num_parts, plan.precision) == (split.num_parts, split.precision), name
