"""Python binding of libsda (include/sda.h): argument marshalling over ctypes.

Every step of the decode path runs in the HIP library; this module only turns
torch tensors (device memory) and the current HIP stream into the C ABI's plain
pointers and sizes. If libsda.so has not been built, importing works but every
call raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsda.so")

FP8_SLOTSCALE, FP8_528, NVFP4_288, V32_656, FP8_UE8M0, MODEL1_584 = 0, 1, 2, 3, 4, 5
META_INTS = 8

SDA_OK, SDA_ERR_INVALID_ARG, SDA_ERR_UNSUPPORTED, SDA_ERR_WORKSPACE, SDA_ERR_HIP = 0, -1, -2, -3, -4

EXPORTED_SYMBOLS = ("sda_make_plan", "sda_choose_plan", "sda_workspace_bytes", "sda_get_sched_meta", "sda_get_sched_meta_host",
                    "sda_sparse_decode_attn", "sda_decode_splits", "sda_workspace_lse_offset",
                    "sda_combine_splits", "sda_status_string", "sda_last_error", "sda_record_bytes",
                    "sda_format_dims", "sda_workspace_bytes_v41", "sda_sparse_decode_attn_v41",
                    "sda_noalloc_workspace_bytes", "sda_sparse_decode_attn_noalloc")
SCRATCH_BYTES = 64 << 20  # SDA_SCRATCH_BYTES


class SdaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"sda status {status}: {msg}")
        self.status = status


class sda_cache(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("num_pages", ctypes.c_int64), ("page_size", ctypes.c_int32),
                ("format", ctypes.c_int32), ("page_stride", ctypes.c_int64), ("slot_scale", ctypes.c_void_p)]


class sda_list(ctypes.Structure):
    _fields_ = [("idx", ctypes.c_void_p), ("row_stride", ctypes.c_int64), ("width", ctypes.c_int32),
                ("queries_per_len", ctypes.c_int32), ("lens", ctypes.c_void_p)]


class sda_v41(ctypes.Structure):
    _fields_ = [("positions", ctypes.c_void_p), ("cos_sin", ctypes.c_void_p), ("cs_stride", ctypes.c_int64),
                ("num_positions", ctypes.c_int64), ("out_fp8", ctypes.c_void_p), ("of_stride_t", ctypes.c_int64),
                ("of_stride_h", ctypes.c_int64), ("out_scale", ctypes.c_void_p), ("os_stride_t", ctypes.c_int64),
                ("os_stride_h", ctypes.c_int64)]


class sda_plan(ctypes.Structure):
    _fields_ = [("num_parts", ctypes.c_int32), ("heads_per_group", ctypes.c_int32),
                ("fixed_overhead", ctypes.c_int32), ("precision", ctypes.c_int32),
                ("whole_tokens", ctypes.c_int32)]

    def __repr__(self):
        return (f"sda_plan(num_parts={self.num_parts}, heads_per_group={self.heads_per_group}, "
                f"fixed_overhead={self.fixed_overhead}, precision={self.precision}, "
                f"whole_tokens={self.whole_tokens})")


_lib = None


def lib():
    """The loaded libsda.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with sliding_window_decode_amd/build.py "
                               "(or __graft_entry__.build()); there is no fallback implementation")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
        L.sda_make_plan.argtypes = [i32, i32, i32, i32, i32, i32, ctypes.POINTER(sda_plan)]
        L.sda_choose_plan.argtypes = [i32, i32, i32, i32, vp, i32, i32, vp, i32, i32, i32, i32,
                                      ctypes.POINTER(sda_plan)]
        L.sda_workspace_bytes.argtypes = [i32, i32, i32, ctypes.POINTER(sda_plan)]
        L.sda_workspace_bytes.restype = sz
        L.sda_get_sched_meta.argtypes = [i32, ctypes.POINTER(sda_list), ctypes.POINTER(sda_list),
                                         ctypes.POINTER(sda_plan), vp, vp, vp]
        L.sda_get_sched_meta_host.argtypes = [i32, i32, vp, i32, vp, i32, ctypes.POINTER(sda_plan), vp, vp]
        L.sda_sparse_decode_attn.argtypes = [vp, i64, i64, i32, i32, i32, i32, ctypes.POINTER(sda_cache),
                                             ctypes.POINTER(sda_list), ctypes.POINTER(sda_cache),
                                             ctypes.POINTER(sda_list), vp, ctypes.c_float, ctypes.POINTER(sda_plan),
                                             vp, vp, vp, sz, vp, i64, i64, vp, i64, vp]
        L.sda_decode_splits.argtypes = L.sda_sparse_decode_attn.argtypes
        L.sda_sparse_decode_attn_noalloc.argtypes = [vp, i64, i64, i32, i32, i32, i32, ctypes.POINTER(sda_cache),
                                                     ctypes.POINTER(sda_list), ctypes.POINTER(sda_cache),
                                                     ctypes.POINTER(sda_list), vp, ctypes.c_float,
                                                     ctypes.POINTER(sda_plan), vp, vp, vp, i64, i64, vp, i64, vp]
        L.sda_noalloc_workspace_bytes.argtypes = [i32, i32, i32, ctypes.POINTER(sda_plan)]
        L.sda_noalloc_workspace_bytes.restype = sz
        L.sda_workspace_bytes_v41.argtypes = [i32, i32, ctypes.POINTER(sda_plan)]
        L.sda_workspace_bytes_v41.restype = sz
        L.sda_sparse_decode_attn_v41.argtypes = [vp, i64, i64, i32, i32, ctypes.POINTER(sda_cache),
                                                 ctypes.POINTER(sda_list), ctypes.POINTER(sda_cache),
                                                 ctypes.POINTER(sda_list), vp, ctypes.c_float,
                                                 ctypes.POINTER(sda_plan), vp, vp, vp, sz, ctypes.POINTER(sda_v41),
                                                 vp, i64, vp]
        L.sda_workspace_lse_offset.argtypes = [i32, i32, i32, ctypes.POINTER(sda_plan)]
        L.sda_workspace_lse_offset.restype = sz
        L.sda_combine_splits.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, i64, i64, vp, i64, vp]
        L.sda_status_string.argtypes = [i32]
        L.sda_status_string.restype = ctypes.c_char_p
        L.sda_last_error.restype = ctypes.c_char_p
        L.sda_record_bytes.argtypes = [i32]
        L.sda_format_dims.argtypes = [i32]
        _lib = L
    return _lib


def _check(status: int):
    if status != SDA_OK:
        L = lib()
        raise SdaError(status, f"{L.sda_status_string(status).decode()}: {L.sda_last_error().decode()}")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


@dataclasses.dataclass
class Cache:
    """A paged cache in device memory: `data` holds num_pages * page_stride bytes."""
    data: "object"                # torch uint8 tensor (device)
    num_pages: int
    page_size: int
    page_stride: int
    format: int
    slot_scale: "object" = None   # torch float32 tensor (device), FP8_SLOTSCALE only

    def c(self) -> sda_cache:
        return sda_cache(_ptr(self.data), self.num_pages, self.page_size, self.format, self.page_stride,
                         _ptr(self.slot_scale))


@dataclasses.dataclass
class SlotList:
    idx: "object"                 # torch int32 [T, row_stride] (device)
    width: int
    lens: "object" = None         # torch int32 [ceil(T / queries_per_len)] (device) or None
    queries_per_len: int = 1      # consecutive tokens (queries of one request) sharing a length entry

    def c(self) -> sda_list:
        return sda_list(_ptr(self.idx), self.idx.stride(0), self.width, self.queries_per_len, _ptr(self.lens))


def make_plan(T: int, H: int, d_qk: int, width: int, extra_width: int = 0, num_cus: int = 256) -> sda_plan:
    plan = sda_plan()
    _check(lib().sda_make_plan(T, H, d_qk, width, extra_width, num_cus, ctypes.byref(plan)))
    return plan


def auto_plan(T: int, H: int, d_qk: int, width: int, extra_width: int, lens, extra_lens, formats,
              v41: bool = False, queries_per_len: int = 1, num_cus: int = 256) -> sda_plan:
    """sda_choose_plan: the library's plan for a call whose lengths the caller holds on the host (numpy int32
    arrays, one entry per queries_per_len tokens, or None = the width). formats: the record format of each
    list (None for no extra list)."""
    import numpy as np
    plan = sda_plan()
    l0 = None if lens is None else np.ascontiguousarray(lens, dtype=np.int32)
    l1 = None if extra_lens is None or extra_width <= 0 else np.ascontiguousarray(extra_lens, dtype=np.int32)
    xf = formats[1] if len(formats) > 1 and formats[1] is not None else -1
    _check(lib().sda_choose_plan(T, H, d_qk, formats[0], None if l0 is None else l0.ctypes.data, width, xf,
                                 None if l1 is None else l1.ctypes.data, extra_width if xf >= 0 else 0,
                                 queries_per_len, 1 if v41 else 0, num_cus, ctypes.byref(plan)))
    return plan


def workspace_bytes(T: int, H: int, d_v: int, plan: sda_plan) -> int:
    return int(lib().sda_workspace_bytes(T, H, d_v, ctypes.byref(plan)))


def get_sched_meta(T: int, lst: SlotList, extra: Optional[SlotList], plan: sda_plan, meta, num_splits, stream=None):
    cl = lst.c()
    xl = extra.c() if extra is not None else None
    _check(lib().sda_get_sched_meta(T, ctypes.byref(cl), ctypes.byref(xl) if xl is not None else None,
                                    ctypes.byref(plan), _ptr(meta), _ptr(num_splits), _stream(stream)))


def get_sched_meta_host(T: int, lens, width: int, extra_lens, extra_width: int, plan: sda_plan,
                        queries_per_len: int = 1):
    """Host schedule from numpy int32 lengths (or None; one entry per queries_per_len tokens): returns
    (meta [P, 8], num_splits [T+1]) numpy arrays."""
    import numpy as np
    meta = np.zeros((plan.num_parts, META_INTS), dtype=np.int32)
    ns = np.zeros(T + 1, dtype=np.int32)
    l0 = None if lens is None else np.ascontiguousarray(lens, dtype=np.int32)
    l1 = None if extra_lens is None else np.ascontiguousarray(extra_lens, dtype=np.int32)
    _check(lib().sda_get_sched_meta_host(T, queries_per_len, None if l0 is None else l0.ctypes.data, width,
                                         None if l1 is None else l1.ctypes.data, extra_width, ctypes.byref(plan),
                                         meta.ctypes.data, ns.ctypes.data))
    return meta, ns


def _decode_args(q, cache, lst, extra_cache, extra_lst, attn_sink, scale, plan, meta, num_splits, workspace, out,
                 lse, stream):
    T, H, d_qk = q.shape
    d_v = 512 if out is None else out.shape[-1]
    cc, cl = cache.c(), lst.c()
    xc = extra_cache.c() if extra_cache is not None else None
    xl = extra_lst.c() if extra_lst is not None else None
    return (_ptr(q), q.stride(0), q.stride(1), T, H, d_qk, d_v, ctypes.byref(cc), ctypes.byref(cl),
            ctypes.byref(xc) if xc is not None else None, ctypes.byref(xl) if xl is not None else None,
            _ptr(attn_sink), ctypes.c_float(scale), ctypes.byref(plan), _ptr(meta), _ptr(num_splits),
            _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
            _ptr(out), 0 if out is None else out.stride(0), 0 if out is None else out.stride(1), _ptr(lse),
            0 if lse is None else lse.stride(0), _stream(stream))


def _decode_call(fn, q, cache, lst, extra_cache, extra_lst, attn_sink, scale, plan, meta, num_splits, workspace,
                 out, lse, stream):
    _check(fn(*_decode_args(q, cache, lst, extra_cache, extra_lst, attn_sink, scale, plan, meta, num_splits,
                            workspace, out, lse, stream)))


def _prepared(fn, args):
    def call():
        rc = fn(*args)
        if rc != SDA_OK:
            _check(rc)
    return call


def prepare_sparse_decode_attn(q, cache: Cache, lst: SlotList, extra_cache: Optional[Cache],
                               extra_lst: Optional[SlotList], attn_sink, scale: float, plan: sda_plan, meta,
                               num_splits, workspace, out, lse, stream=None):
    """sparse_decode_attn with its arguments marshalled once: returns a callable that enqueues the op on the
    stream current now (for launch loops; the tensors must stay alive)."""
    return _prepared(lib().sda_sparse_decode_attn, _decode_args(q, cache, lst, extra_cache, extra_lst, attn_sink,
                                                                scale, plan, meta, num_splits, workspace, out, lse,
                                                                stream))


def prepare_decode_splits(q, cache: Cache, lst: SlotList, extra_cache: Optional[Cache], extra_lst: Optional[SlotList],
                          attn_sink, scale: float, plan: sda_plan, meta, num_splits, workspace, out, lse, stream=None):
    """decode_splits with its arguments marshalled once (see prepare_sparse_decode_attn)."""
    return _prepared(lib().sda_decode_splits, _decode_args(q, cache, lst, extra_cache, extra_lst, attn_sink, scale,
                                                           plan, meta, num_splits, workspace, out, lse, stream))


def prepare_get_sched_meta(T: int, lst: SlotList, extra: Optional[SlotList], plan: sda_plan, meta, num_splits,
                           stream=None):
    """get_sched_meta with its arguments marshalled once (see prepare_sparse_decode_attn)."""
    cl = lst.c()
    xl = extra.c() if extra is not None else None
    return _prepared(lib().sda_get_sched_meta, (T, ctypes.byref(cl), ctypes.byref(xl) if xl is not None else None,
                                                ctypes.byref(plan), _ptr(meta), _ptr(num_splits), _stream(stream)))


def prepare_combine_splits(o_accum, lse_accum, num_splits, attn_sink, out, lse, stream=None):
    """combine_splits with its arguments marshalled once (see prepare_sparse_decode_attn)."""
    T = num_splits.shape[0] - 1
    H, d_v = out.shape[1], out.shape[2]
    return _prepared(lib().sda_combine_splits, (T, H, d_v, _ptr(o_accum), _ptr(lse_accum), _ptr(num_splits),
                                                _ptr(attn_sink), _ptr(out), out.stride(0), out.stride(1), _ptr(lse),
                                                lse.stride(0), _stream(stream)))


def sparse_decode_attn(q, cache: Cache, lst: SlotList, extra_cache: Optional[Cache], extra_lst: Optional[SlotList],
                       attn_sink, scale: float, plan: sda_plan, meta, num_splits, workspace, out, lse, stream=None):
    """Whole op: (scheduler if meta is None) + decode + combine.
    q [T, H, d_qk] bf16, out [T, H, 512] bf16, lse [T, H] fp32 (device tensors, strided rows allowed)."""
    _decode_call(lib().sda_sparse_decode_attn, q, cache, lst, extra_cache, extra_lst, attn_sink, scale, plan, meta,
                 num_splits, workspace, out, lse, stream)


def decode_splits(q, cache: Cache, lst: SlotList, extra_cache: Optional[Cache], extra_lst: Optional[SlotList],
                  attn_sink, scale: float, plan: sda_plan, meta, num_splits, workspace, out, lse, stream=None):
    """The decode kernel only (final rows for unsplit tokens, partials in the workspace for the others; with
    out=None every token leaves as a partial, as in the V4.1 call)."""
    _decode_call(lib().sda_decode_splits, q, cache, lst, extra_cache, extra_lst, attn_sink, scale, plan, meta,
                 num_splits, workspace, out, lse, stream)


def sparse_decode_attn_noalloc(q, cache: Cache, lst: SlotList, extra_cache: Optional[Cache],
                               extra_lst: Optional[SlotList], attn_sink, scale: float, plan: sda_plan, meta,
                               num_splits, out, lse, stream=None):
    """The whole op with the library's static scratch as its workspace (no workspace argument)."""
    T, H, d_qk = q.shape
    cc, cl = cache.c(), lst.c()
    xc = extra_cache.c() if extra_cache is not None else None
    xl = extra_lst.c() if extra_lst is not None else None
    _check(lib().sda_sparse_decode_attn_noalloc(
        _ptr(q), q.stride(0), q.stride(1), T, H, d_qk, out.shape[-1], ctypes.byref(cc), ctypes.byref(cl),
        ctypes.byref(xc) if xc is not None else None, ctypes.byref(xl) if xl is not None else None,
        _ptr(attn_sink), ctypes.c_float(scale), ctypes.byref(plan), _ptr(meta), _ptr(num_splits),
        _ptr(out), out.stride(0), out.stride(1), _ptr(lse), lse.stride(0), _stream(stream)))


def noalloc_workspace_bytes(T: int, H: int, d_v: int, plan: sda_plan) -> int:
    return int(lib().sda_noalloc_workspace_bytes(T, H, d_v, ctypes.byref(plan)))


def workspace_bytes_v41(T: int, H: int, plan: sda_plan) -> int:
    return int(lib().sda_workspace_bytes_v41(T, H, ctypes.byref(plan)))


def sparse_decode_attn_v41(q, cache: Cache, lst: SlotList, extra_cache: Optional[Cache], extra_lst: Optional[SlotList],
                           attn_sink, scale: float, plan: sda_plan, meta, num_splits, workspace, positions, cos_sin,
                           out_fp8, out_scale, lse=None, stream=None):
    """V4.1 decode: q [T, H, 512] bf16 before RoPE, positions [T] int64, cos_sin [P, >=64] fp32; writes out_fp8
    [T, H, 512] uint8 (e4m3 codes), out_scale [T, H, 16] uint8 (ue8m0) and, if given, lse [T, H] fp32."""
    T, H, _ = q.shape
    cc, cl = cache.c(), lst.c()
    xc = extra_cache.c() if extra_cache is not None else None
    xl = extra_lst.c() if extra_lst is not None else None
    v = sda_v41(_ptr(positions), _ptr(cos_sin), cos_sin.stride(0), cos_sin.shape[0], _ptr(out_fp8), out_fp8.stride(0),
                out_fp8.stride(1), _ptr(out_scale), out_scale.stride(0), out_scale.stride(1))
    _check(lib().sda_sparse_decode_attn_v41(
        _ptr(q), q.stride(0), q.stride(1), T, H, ctypes.byref(cc), ctypes.byref(cl),
        ctypes.byref(xc) if xc is not None else None, ctypes.byref(xl) if xl is not None else None,
        _ptr(attn_sink), ctypes.c_float(scale), ctypes.byref(plan), _ptr(meta), _ptr(num_splits),
        _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(), ctypes.byref(v),
        _ptr(lse), 0 if lse is None else lse.stride(0), _stream(stream)))


def workspace_lse_offset(T: int, H: int, d_v: int, plan: sda_plan) -> int:
    return int(lib().sda_workspace_lse_offset(T, H, d_v, ctypes.byref(plan)))


def combine_splits(o_accum, lse_accum, num_splits, attn_sink, out, lse, stream=None):
    """o_accum [S, H, 512] fp32, lse_accum [S, H] fp32, num_splits [T+1] int32; writes out/lse rows of split tokens."""
    T = num_splits.shape[0] - 1
    H, d_v = out.shape[1], out.shape[2]
    _check(lib().sda_combine_splits(T, H, d_v, _ptr(o_accum), _ptr(lse_accum), _ptr(num_splits), _ptr(attn_sink),
                                    _ptr(out), out.stride(0), out.stride(1), _ptr(lse), lse.stride(0),
                                    _stream(stream)))


class Decoder:
    """Holds the plan, scheduler arrays and workspace for one decode shape (allocated by torch once)."""

    def __init__(self, T: int, H: int, d_qk: int, width: int, extra_width: int = 0, device="cuda",
                 plan: Optional[sda_plan] = None):
        import torch
        self.T, self.H, self.d_qk = T, H, d_qk
        self.plan = plan if plan is not None else make_plan(T, H, d_qk, width, extra_width)
        self.meta = torch.empty((self.plan.num_parts, META_INTS), dtype=torch.int32, device=device)
        self.num_splits = torch.empty(T + 1, dtype=torch.int32, device=device)
        nbytes = workspace_bytes(T, H, 512, self.plan)
        if d_qk == 512:  # room for the V4.1 call's rotated query dims as well
            nbytes = max(nbytes, workspace_bytes_v41(T, H, self.plan))
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)

    def schedule(self, lst: SlotList, extra: Optional[SlotList] = None, stream=None):
        """Runs the scheduler (nothing for a whole-token plan, which has no schedule)."""
        if not self.plan.whole_tokens:
            get_sched_meta(self.T, lst, extra, self.plan, self.meta, self.num_splits, stream)

    @property
    def sched_arrays(self):
        """(meta, num_splits) to pass to the decode calls: None for a whole-token plan."""
        return (None, None) if self.plan.whole_tokens else (self.meta, self.num_splits)

    def __call__(self, q, cache, lst, extra_cache=None, extra_lst=None, attn_sink=None, scale=None, out=None,
                 lse=None, schedule=True, stream=None):
        import torch
        if scale is None:
            scale = self.d_qk ** -0.5
        if out is None:
            out = torch.empty((self.T, self.H, 512), dtype=torch.bfloat16, device=q.device)
        if lse is None:
            lse = torch.empty((self.T, self.H), dtype=torch.float32, device=q.device)
        if schedule:
            self.schedule(lst, extra_lst, stream)
        meta, num_splits = self.sched_arrays
        sparse_decode_attn(q, cache, lst, extra_cache, extra_lst, attn_sink, scale, self.plan, meta, num_splits,
                           self.workspace, out, lse, stream)
        return out, lse

    def v41(self, q, cache, lst, extra_cache, extra_lst, attn_sink, scale, positions, cos_sin, out_fp8=None,
            out_scale=None, lse=None, schedule=True, stream=None):
        """The V4.1 call (Q RoPE, decode, inverse RoPE and MXFP8 output): returns (out_fp8, out_scale, lse)."""
        import torch
        if out_fp8 is None:
            out_fp8 = torch.empty((self.T, self.H, 512), dtype=torch.uint8, device=q.device)
        if out_scale is None:
            out_scale = torch.empty((self.T, self.H, 16), dtype=torch.uint8, device=q.device)
        if lse is None:
            lse = torch.empty((self.T, self.H), dtype=torch.float32, device=q.device)
        if schedule:
            self.schedule(lst, extra_lst, stream)
        meta, num_splits = self.sched_arrays
        sparse_decode_attn_v41(q, cache, lst, extra_cache, extra_lst, attn_sink, scale, self.plan, meta, num_splits,
                               self.workspace, positions, cos_sin, out_fp8, out_scale, lse, stream)
        return out_fp8, out_scale, lse
