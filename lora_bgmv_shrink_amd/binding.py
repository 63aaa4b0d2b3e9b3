"""Thin ctypes binding over liblora_mi355x.so.

Argument marshalling only: every step of the layer runs in the library's
HIP kernels.  PyTorch supplies device memory (tensor ``data_ptr()``) and the
current stream.  Output tensors and zero-filled workspaces are allocated
here with torch when the caller does not pass them.

The functions carry the C names (see include/lora_mi355x.h for the
semantics, layouts and error behaviour of each).  Calls that take a base
weight have no default for its storage (``w_layout``): LORA_W_OUT_IN
([d_out, d_in]) is the fast one, and the caller says which it holds.  A non-OK status raises
``LoraError``.  Importing this module without the built library raises
``ImportError``; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch  # loads the HIP runtime the library binds to

from .build import LIB_PATH

(LORA_OK, LORA_E_INVALID, LORA_E_UNSUPPORTED, LORA_E_WORKSPACE, LORA_E_ID_RANGE, LORA_E_DEVICE,
 LORA_E_NOT_RESIDENT, LORA_E_SCRATCH) = range(8)
LORA_NOALLOC_SCRATCH_BYTES = 64 << 20
LORA_F32, LORA_BF16 = 0, 1
LORA_LAYOUT_UNIFORM, LORA_LAYOUT_RAGGED = 0, 1
LORA_MODE_AUTO, LORA_MODE_BGMV, LORA_MODE_SGMV = 0, 1, 2
LORA_W_IN_OUT, LORA_W_OUT_IN = 0, 1
LORA_CACHE_RESIDENT, LORA_CACHE_LOADING, LORA_CACHE_DEFERRED = 0, 1, 2
LORA_CACHE_HOST_ONLY, LORA_CACHE_ANY_RANK, LORA_CACHE_EXPLICIT_POLL = 1, 2, 4

# Every symbol the C header declares.
EXPORTS = [
    "lora_status_string", "lora_adapter_param_count", "lora_pool_ragged_offsets", "lora_pool_create",
    "lora_pool_destroy", "lora_pool_param_count", "lora_pool_last_error", "lora_workspace_clear",
    "lora_segments_workspace", "lora_segments_build", "lora_bgmv_shrink",
    "lora_bgmv_expand", "lora_sgmv_shrink_workspace", "lora_sgmv_shrink", "lora_sgmv_expand", "lora_layer_workspace",
    "lora_layer_apply", "lora_base_gemm_expand_workspace", "lora_base_gemm_expand", "lora_decode_workspace",
    "lora_decode_stream",
    "lora_decode_finish", "lora_merge_adapter",
    "lora_cache_blob_layout", "lora_cache_create", "lora_cache_destroy", "lora_cache_register",
    "lora_cache_pin", "lora_cache_hold", "lora_cache_request", "lora_cache_poll", "lora_cache_wait",
    "lora_cache_map", "lora_cache_release", "lora_cache_pool", "lora_cache_slot_of", "lora_cache_stats",
    "lora_decode_stream_q4",
    "lora_sched_create", "lora_sched_destroy", "lora_sched_submit", "lora_sched_step", "lora_sched_queued",
    "lora_layer_apply_noalloc", "lora_layer_q4_workspace", "lora_layer_apply_q4",
]


class LoraError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_lib.lora_status_string(status).decode()}")


class CacheStatsT(ctypes.Structure):
    _fields_ = [(k, ctypes.c_int64) for k in (
        "requests", "hits", "pending", "loads_started", "deferred_load_cap", "deferred_no_slot",
        "loads_completed", "evictions", "bytes_loaded", "bytes_resident")] + \
        [(k, ctypes.c_int32) for k in ("n_slots", "slots_resident", "slots_loading", "slots_bound")]


class SchedConfigT(ctypes.Structure):
    _fields_ = [("w_fair", ctypes.c_double), ("w_local", ctypes.c_double), ("max_adapters", ctypes.c_int32),
                ("max_rows", ctypes.c_int32), ("rank_groups", ctypes.c_int32)]


class SchedStepT(ctypes.Structure):
    _fields_ = [(k, ctypes.c_int32) for k in (
        "admitted", "rows", "distinct_adapters", "skipped_rows", "skipped_cap", "skipped_rank_group",
        "deferred_not_resident", "queued")] + [("max_wait_admitted", ctypes.c_double),
                                               ("max_wait_queued", ctypes.c_double)]


class SegmentsT(ctypes.Structure):
    _fields_ = [("perm", ctypes.c_void_p), ("seg_ids", ctypes.c_void_p), ("seg_off", ctypes.c_void_p),
                ("n_seg", ctypes.c_void_p), ("cap", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m lora_bgmv_shrink_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    p, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    st = ctypes.c_int
    sig = {
        "lora_status_string": (ctypes.c_char_p, [st]),
        "lora_adapter_param_count": (i64, [i32, i32, i32]),
        "lora_pool_ragged_offsets": (st, [i32, p, i32, i32, p, p, p, p]),
        "lora_pool_create": (st, [p, st, st, i32, i32, i32, i32, p, p, p, p, p, p]),
        "lora_pool_destroy": (st, [p]),
        "lora_pool_param_count": (i64, [p, i32]),
        "lora_pool_last_error": (st, [p, p, p]),
        "lora_workspace_clear": (st, [p, sz, p]),
        "lora_segments_workspace": (st, [i32, i32, p]),
        "lora_segments_build": (st, [p, i32, i32, p, p, p, sz, p]),
        "lora_bgmv_shrink": (st, [p, p, i64, p, i32, p, i64, p]),
        "lora_bgmv_expand": (st, [p, p, i64, p, i32, p, st, i64, ctypes.c_int, p]),
        "lora_sgmv_shrink_workspace": (st, [p, i32, p]),
        "lora_sgmv_shrink": (st, [p, p, i64, p, i32, p, i64, p, sz, p]),
        "lora_sgmv_expand": (st, [p, p, i64, p, i32, p, st, i64, ctypes.c_int, p]),
        "lora_layer_workspace": (st, [p, i32, st, p]),
        "lora_layer_apply": (st, [p, p, i64, p, i64, st, p, p, i32, p, st, i64, st, p, sz, p]),
        "lora_base_gemm_expand_workspace": (st, [p, i32, p]),
        "lora_base_gemm_expand": (st, [p, p, i64, p, i64, st, p, p, i64, i32, p, st, i64, p, sz, p]),
        "lora_decode_workspace": (st, [p, i32, ctypes.c_int, p]),
        "lora_decode_stream": (st, [p, p, i64, p, i64, p, i32, ctypes.c_int, p, sz, p]),
        "lora_decode_finish": (st, [p, p, i32, ctypes.c_int, p, st, i64, p, sz, p]),
        "lora_merge_adapter": (st, [p, i32, p, i64, st, ctypes.c_float, p]),
        "lora_cache_blob_layout": (st, [p, i32, p, p, p]),
        "lora_cache_create": (st, [p, st, i32, p, p, i32, i32, i32, i32, i32]),
        "lora_cache_destroy": (st, [p]),
        "lora_cache_register": (st, [p, i32, i32, ctypes.c_float, p]),
        "lora_cache_pin": (st, [p, i32, i32]),
        "lora_cache_hold": (st, [p, i32, i32]),
        "lora_cache_request": (st, [p, i32, p]),
        "lora_cache_poll": (st, [p, p]),
        "lora_cache_wait": (st, [p]),
        "lora_cache_map": (st, [p, p, i32, p, p]),
        "lora_cache_release": (st, [p, p]),
        "lora_cache_pool": (p, [p, i32]),
        "lora_cache_slot_of": (i32, [p, i32]),
        "lora_cache_stats": (st, [p, p]),
        "lora_decode_stream_q4": (st, [p, p, i64, p, i64, p, i64, p, i32, ctypes.c_int, p, sz, p]),
        "lora_sched_create": (st, [p, p, i32, p, p]),
        "lora_sched_destroy": (st, [p]),
        "lora_sched_submit": (st, [p, i64, i32, i32, ctypes.c_double]),
        "lora_sched_step": (st, [p, ctypes.c_double, i32, p, p, p, p, p]),
        "lora_sched_queued": (i32, [p]),
        "lora_layer_apply_noalloc": (st, [p, p, i64, p, i64, st, p, p, i32, p, st, i64, st, p]),
        "lora_layer_q4_workspace": (st, [p, i32, p]),
        "lora_layer_apply_q4": (st, [p, p, i64, p, i64, p, i64, p, p, i32, p, st, i64, p, sz, p]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()


def library():
    """The loaded ctypes library (for symbol checks)."""
    return _lib


def _check(status: int, where: str):
    if status != LORA_OK:
        raise LoraError(status, where)


def _dt(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return LORA_BF16
    if t == torch.float32:
        return LORA_F32
    raise TypeError(f"unsupported dtype {t}")


def _stream(dev) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _ld(t: torch.Tensor) -> int:
    assert t.dim() == 2 and t.stride(1) == 1, "expected a row-major 2-D tensor"
    return t.stride(0)


# --------------------------------------------------------------------------
# Pools
# --------------------------------------------------------------------------

@dataclass
class Pool:
    handle: ctypes.c_void_p
    dtype: torch.dtype
    n_adapters: int
    d_in: int
    d_out: int
    r_max: int
    A: torch.Tensor
    B: torch.Tensor
    owned: bool = True   # False for the pools of an adapter cache (the cache frees them)

    def destroy(self):
        if self.handle and self.owned:
            _check(_lib.lora_pool_destroy(self.handle), "lora_pool_destroy")
            self.handle = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def lora_adapter_param_count(rank: int, d_in: int, d_out: int) -> int:
    return int(_lib.lora_adapter_param_count(rank, d_in, d_out))


def lora_pool_ragged_offsets(ranks, d_in: int, d_out: int):
    ranks = np.ascontiguousarray(ranks, np.int32)
    n = ranks.shape[0]
    a_off = np.zeros(n, np.int64)
    b_off = np.zeros(n, np.int64)
    ta = ctypes.c_int64()
    tb = ctypes.c_int64()
    _check(_lib.lora_pool_ragged_offsets(n, ranks.ctypes.data, d_in, d_out, a_off.ctypes.data,
                                         b_off.ctypes.data, ctypes.byref(ta), ctypes.byref(tb)),
           "lora_pool_ragged_offsets")
    return a_off, b_off, ta.value, tb.value


def lora_pool_create(layout: int, A: torch.Tensor, B: torch.Tensor, n_adapters: int, d_in: int,
                     d_out: int, r_max: int, scales, ranks=None, a_off=None, b_off=None) -> Pool:
    assert A.is_cuda and B.is_cuda and A.dtype == B.dtype and A.is_contiguous() and B.is_contiguous()
    sc = np.ascontiguousarray(np.broadcast_to(np.asarray(scales, np.float32), (n_adapters,)))
    h = ctypes.c_void_p()
    args_r = [None, None, None]
    keep = []
    if layout == LORA_LAYOUT_RAGGED:
        for k, arr, dt in ((0, ranks, np.int32), (1, a_off, np.int64), (2, b_off, np.int64)):
            a = np.ascontiguousarray(arr, dt)
            keep.append(a)
            args_r[k] = a.ctypes.data
    with torch.cuda.device(A.device):
        _check(_lib.lora_pool_create(ctypes.byref(h), layout, _dt(A.dtype), n_adapters, d_in, d_out, r_max,
                                     args_r[0], args_r[1], args_r[2], _ptr(A), _ptr(B), sc.ctypes.data),
               "lora_pool_create")
    return Pool(h, A.dtype, n_adapters, d_in, d_out, r_max, A, B)


def lora_pool_destroy(pool: Pool):
    pool.destroy()


def lora_pool_param_count(pool: Pool, adapter: int) -> int:
    return int(_lib.lora_pool_param_count(pool.handle, adapter))


def lora_pool_last_error(pool: Pool) -> int:
    """Synchronize the current stream and return (and clear) the device error word."""
    v = ctypes.c_int32()
    st = _lib.lora_pool_last_error(pool.handle, ctypes.c_void_p(_stream(pool.A.device)), ctypes.byref(v))
    if st not in (LORA_OK, LORA_E_ID_RANGE):
        _check(st, "lora_pool_last_error")
    return int(v.value)


def lora_workspace_clear(ws: torch.Tensor):
    _check(_lib.lora_workspace_clear(_ptr(ws), ws.numel() * ws.element_size(),
                                     ctypes.c_void_p(_stream(ws.device))), "lora_workspace_clear")


def _workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


# --------------------------------------------------------------------------
# Segments
# --------------------------------------------------------------------------

@dataclass
class Segments:
    perm: torch.Tensor
    seg_ids: torch.Tensor
    seg_off: torch.Tensor
    n_seg: torch.Tensor
    cap: int

    def c_struct(self) -> SegmentsT:
        return SegmentsT(self.perm.data_ptr(), self.seg_ids.data_ptr(), self.seg_off.data_ptr(),
                         self.n_seg.data_ptr(), self.cap)

    def host(self):
        """(perm, seg_ids, seg_off) as numpy, trimmed to n_seg (synchronizes)."""
        k = int(self.n_seg.item())
        return (self.perm.cpu().numpy(), self.seg_ids[:k].cpu().numpy(), self.seg_off[:k + 1].cpu().numpy())


def segments_alloc(n_rows: int, n_adapters: int, device) -> Segments:
    cap = max(1, min(n_rows, n_adapters + 1))
    z = lambda n: torch.zeros(max(n, 1), dtype=torch.int32, device=device)
    return Segments(z(n_rows), z(cap), z(cap + 1), z(1), cap)


def lora_segments_build(ids: torch.Tensor, n_adapters: int, seg: Optional[Segments] = None,
                        status: Optional[torch.Tensor] = None) -> Segments:
    assert ids.is_cuda and ids.dtype == torch.int32 and ids.is_contiguous()
    n = ids.numel()
    seg = seg or segments_alloc(n, n_adapters, ids.device)
    ws_b = ctypes.c_size_t()
    _check(_lib.lora_segments_workspace(n, n_adapters, ctypes.byref(ws_b)), "lora_segments_workspace")
    ws = _workspace(ws_b.value, ids.device)
    cs = seg.c_struct()
    _check(_lib.lora_segments_build(_ptr(ids), n, n_adapters, ctypes.byref(cs), _ptr(status), _ptr(ws),
                                    ws_b.value, ctypes.c_void_p(_stream(ids.device))),
           "lora_segments_build")
    return seg


# --------------------------------------------------------------------------
# BGMV / SGMV
# --------------------------------------------------------------------------

def _t_out(pool: Pool, n: int, t: Optional[torch.Tensor], device) -> torch.Tensor:
    if t is None:
        t = torch.empty((n, pool.r_max), dtype=torch.float32, device=device)
    assert t.dtype == torch.float32 and t.shape[0] == n
    return t


def lora_bgmv_shrink(pool: Pool, x: torch.Tensor, ids: torch.Tensor, t: Optional[torch.Tensor] = None) -> torch.Tensor:
    n = ids.numel()
    t = _t_out(pool, n, t, x.device)
    _check(_lib.lora_bgmv_shrink(pool.handle, _ptr(x), _ld(x), _ptr(ids), n, _ptr(t), _ld(t),
                                 ctypes.c_void_p(_stream(x.device))), "lora_bgmv_shrink")
    return t


def _y_out(pool, n, y, y_dtype, device, accumulate):
    if y is None:
        assert not accumulate, "accumulate needs an existing y"
        y = torch.empty((n, pool.d_out), dtype=y_dtype or pool.dtype, device=device)
    return y


def lora_bgmv_expand(pool: Pool, t: torch.Tensor, ids: torch.Tensor, y: Optional[torch.Tensor] = None,
                     y_dtype: Optional[torch.dtype] = None, accumulate: bool = False) -> torch.Tensor:
    n = ids.numel()
    y = _y_out(pool, n, y, y_dtype, t.device, accumulate)
    _check(_lib.lora_bgmv_expand(pool.handle, _ptr(t), _ld(t), _ptr(ids), n, _ptr(y), _dt(y.dtype), _ld(y),
                                 int(bool(accumulate)), ctypes.c_void_p(_stream(t.device))),
           "lora_bgmv_expand")
    return y


def lora_sgmv_shrink_workspace(pool: Pool, n_rows: int) -> int:
    v = ctypes.c_size_t()
    _check(_lib.lora_sgmv_shrink_workspace(pool.handle, n_rows, ctypes.byref(v)), "lora_sgmv_shrink_workspace")
    return v.value


def lora_sgmv_shrink(pool: Pool, x: torch.Tensor, seg: Segments, t: Optional[torch.Tensor] = None,
                     ws: Optional[torch.Tensor] = None, split: bool = True) -> torch.Tensor:
    """With ``split`` (and no ``ws`` given) a workspace of the size the
    library asks for is allocated, so K is split when it pays."""
    n = x.shape[0]
    t = _t_out(pool, n, t, x.device)
    if ws is None and split:
        ws = _workspace(lora_sgmv_shrink_workspace(pool, n), x.device)
    cs = seg.c_struct()
    _check(_lib.lora_sgmv_shrink(pool.handle, _ptr(x), _ld(x), ctypes.byref(cs), n, _ptr(t), _ld(t), _ptr(ws),
                                 0 if ws is None else ws.numel(), ctypes.c_void_p(_stream(x.device))),
           "lora_sgmv_shrink")
    return t


def lora_sgmv_expand(pool: Pool, t: torch.Tensor, seg: Segments, y: Optional[torch.Tensor] = None,
                     y_dtype: Optional[torch.dtype] = None, accumulate: bool = False) -> torch.Tensor:
    n = t.shape[0]
    y = _y_out(pool, n, y, y_dtype, t.device, accumulate)
    cs = seg.c_struct()
    _check(_lib.lora_sgmv_expand(pool.handle, _ptr(t), _ld(t), ctypes.byref(cs), n, _ptr(y), _dt(y.dtype),
                                 _ld(y), int(bool(accumulate)), ctypes.c_void_p(_stream(t.device))),
           "lora_sgmv_expand")
    return y


# --------------------------------------------------------------------------
# Layer
# --------------------------------------------------------------------------

def lora_layer_workspace(pool: Pool, n_rows: int, mode: int = LORA_MODE_AUTO) -> int:
    b = ctypes.c_size_t()
    _check(_lib.lora_layer_workspace(pool.handle, n_rows, mode, ctypes.byref(b)), "lora_layer_workspace")
    return b.value


def lora_layer_apply(pool: Pool, x: torch.Tensor, W: torch.Tensor, ids: torch.Tensor,
                     w_layout: int, seg: Optional[Segments] = None,
                     y: Optional[torch.Tensor] = None, y_dtype: Optional[torch.dtype] = None,
                     mode: int = LORA_MODE_AUTO, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    n = ids.numel()
    y = _y_out(pool, n, y, y_dtype, x.device, False)
    need = lora_layer_workspace(pool, n, mode)
    if ws is None:
        ws = _workspace(need, x.device)
    cs = None if seg is None else seg.c_struct()
    _check(_lib.lora_layer_apply(pool.handle, _ptr(x), _ld(x), _ptr(W), _ld(W), w_layout, _ptr(ids),
                                 None if cs is None else ctypes.byref(cs), n, _ptr(y), _dt(y.dtype), _ld(y),
                                 mode, _ptr(ws), 0 if ws is None else ws.numel(),
                                 ctypes.c_void_p(_stream(x.device))), "lora_layer_apply")
    return y


def lora_layer_apply_noalloc(pool: Pool, x: torch.Tensor, W: torch.Tensor, ids: torch.Tensor,
                             w_layout: int, y: torch.Tensor, seg: Optional[Segments] = None,
                             mode: int = LORA_MODE_AUTO) -> torch.Tensor:
    """lora_layer_apply with the library's static scratch instead of a
    workspace; y must be given (nothing is allocated here either)."""
    n = ids.numel()
    cs = None if seg is None else seg.c_struct()
    _check(_lib.lora_layer_apply_noalloc(pool.handle, _ptr(x), _ld(x), _ptr(W), _ld(W), w_layout, _ptr(ids),
                                         None if cs is None else ctypes.byref(cs), n, _ptr(y), _dt(y.dtype),
                                         _ld(y), mode, ctypes.c_void_p(_stream(x.device))),
           "lora_layer_apply_noalloc")
    return y


def lora_base_gemm_expand_workspace(pool: Pool, n_rows: int) -> int:
    v = ctypes.c_size_t()
    _check(_lib.lora_base_gemm_expand_workspace(pool.handle, n_rows, ctypes.byref(v)),
           "lora_base_gemm_expand_workspace")
    return v.value


def lora_base_gemm_expand(pool: Pool, x: torch.Tensor, W: torch.Tensor, ids: torch.Tensor,
                          t: Optional[torch.Tensor], w_layout: int,
                          y: Optional[torch.Tensor] = None, y_dtype: Optional[torch.dtype] = None,
                          ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    n = ids.numel()
    y = _y_out(pool, n, y, y_dtype, x.device, False)
    if t is not None and ws is None:
        ws = _workspace(lora_base_gemm_expand_workspace(pool, n), x.device)
    _check(_lib.lora_base_gemm_expand(pool.handle, _ptr(x), _ld(x), _ptr(W), _ld(W), w_layout, _ptr(ids),
                                      _ptr(t), 0 if t is None else _ld(t), n, _ptr(y), _dt(y.dtype), _ld(y),
                                      _ptr(ws), 0 if ws is None else ws.numel(),
                                      ctypes.c_void_p(_stream(x.device))), "lora_base_gemm_expand")
    return y


def lora_decode_workspace(pool: Pool, n_rows: int, with_lora: bool = True) -> int:
    v = ctypes.c_size_t()
    _check(_lib.lora_decode_workspace(pool.handle, n_rows, int(bool(with_lora)), ctypes.byref(v)),
           "lora_decode_workspace")
    return v.value


def lora_decode_stream(pool: Pool, x: torch.Tensor, W: torch.Tensor, ids: torch.Tensor, ws: torch.Tensor,
                       with_lora: bool = True):
    _check(_lib.lora_decode_stream(pool.handle, _ptr(x), _ld(x), _ptr(W), _ld(W), _ptr(ids), ids.numel(),
                                   int(bool(with_lora)), _ptr(ws), ws.numel(), ctypes.c_void_p(_stream(x.device))),
           "lora_decode_stream")


def lora_decode_stream_q4(pool: Pool, x: torch.Tensor, Wq: torch.Tensor, w_scale: torch.Tensor, ids: torch.Tensor,
                          ws: torch.Tensor, with_lora: bool = True):
    """Stream launch over a 4-bit base: Wq [d_out, ldq] uint8, w_scale
    [d_out, lds] fp32 (see the header for the format)."""
    assert Wq.dtype == torch.uint8 and w_scale.dtype == torch.float32
    _check(_lib.lora_decode_stream_q4(pool.handle, _ptr(x), _ld(x), _ptr(Wq), _ld(Wq), _ptr(w_scale), _ld(w_scale),
                                      _ptr(ids), ids.numel(), int(bool(with_lora)), _ptr(ws), ws.numel(),
                                      ctypes.c_void_p(_stream(x.device))), "lora_decode_stream_q4")


def lora_decode_finish(pool: Pool, ids: torch.Tensor, ws: torch.Tensor, y: torch.Tensor, with_lora: bool = True):
    _check(_lib.lora_decode_finish(pool.handle, _ptr(ids), ids.numel(), int(bool(with_lora)), _ptr(y), _dt(y.dtype),
                                   _ld(y), _ptr(ws), ws.numel(), ctypes.c_void_p(_stream(y.device))),
           "lora_decode_finish")
    return y


def lora_layer_q4_workspace(pool: Pool, n_rows: int) -> int:
    v = ctypes.c_size_t()
    _check(_lib.lora_layer_q4_workspace(pool.handle, n_rows, ctypes.byref(v)), "lora_layer_q4_workspace")
    return v.value


def lora_layer_apply_q4(pool: Pool, x: torch.Tensor, Wq: torch.Tensor, w_scale: torch.Tensor, ids: torch.Tensor,
                        seg: Optional[Segments] = None, y: Optional[torch.Tensor] = None,
                        y_dtype: Optional[torch.dtype] = None, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The layer over a 4-bit base: Wq [d_out, ldq] uint8, w_scale [d_out,
    lds] fp32 (format in the header)."""
    assert Wq.dtype == torch.uint8 and w_scale.dtype == torch.float32
    n = ids.numel()
    y = _y_out(pool, n, y, y_dtype, x.device, False)
    if ws is None:
        ws = _workspace(lora_layer_q4_workspace(pool, n), x.device)
    cs = None if seg is None else seg.c_struct()
    _check(_lib.lora_layer_apply_q4(pool.handle, _ptr(x), _ld(x), _ptr(Wq), _ld(Wq), _ptr(w_scale), _ld(w_scale),
                                    _ptr(ids), None if cs is None else ctypes.byref(cs), n, _ptr(y), _dt(y.dtype),
                                    _ld(y), _ptr(ws), 0 if ws is None else ws.numel(),
                                    ctypes.c_void_p(_stream(x.device))), "lora_layer_apply_q4")
    return y


def lora_merge_adapter(pool: Pool, W: torch.Tensor, adapter: int, w_layout: int,
                       sign: float = 1.0) -> torch.Tensor:
    """W += sign * s_a * A_a B_a in place (W of the pool's dtype, stored per
    ``w_layout``); returns W."""
    assert W.is_cuda and W.dim() == 2 and W.stride(1) == 1
    _check(_lib.lora_merge_adapter(pool.handle, int(adapter), _ptr(W), _ld(W), int(w_layout), float(sign),
                                   ctypes.c_void_p(_stream(W.device))), "lora_merge_adapter")
    return W


# --------------------------------------------------------------------------
# Adapter slot cache
# --------------------------------------------------------------------------

class Cache:
    """An adapter slot cache (lora_cache_*).  ``parts`` lists the (d_in,
    d_out) of every projection an adapter carries.  ``register`` packs an
    adapter's per-part A/B tensors into one pinned host blob in the layout
    lora_cache_blob_layout gives and keeps it alive while the cache lives.
    With ``host_only`` no device memory is used (policy only)."""

    def __init__(self, dtype: torch.dtype, parts, r_max: int, n_adapters: int, n_slots: int,
                 max_loads_in_flight: int, host_only: bool = False, any_rank: bool = False,
                 device=None, explicit_poll: bool = False):
        self.dtype = dtype
        self.parts = [(int(a), int(b)) for a, b in parts]
        self.r_max, self.n_adapters, self.n_slots = r_max, n_adapters, n_slots
        self.host_only = host_only
        self.device = torch.device(device) if device is not None else None
        d_in = np.ascontiguousarray([a for a, _ in self.parts], np.int32)
        d_out = np.ascontiguousarray([b for _, b in self.parts], np.int32)
        flags = ((LORA_CACHE_HOST_ONLY if host_only else 0) | (LORA_CACHE_ANY_RANK if any_rank else 0) |
                 (LORA_CACHE_EXPLICIT_POLL if explicit_poll else 0))
        h = ctypes.c_void_p()
        if host_only:
            st = _lib.lora_cache_create(ctypes.byref(h), _dt(dtype), len(self.parts), d_in.ctypes.data,
                                        d_out.ctypes.data, r_max, n_adapters, n_slots, max_loads_in_flight, flags)
        else:
            with torch.cuda.device(self.device):
                st = _lib.lora_cache_create(ctypes.byref(h), _dt(dtype), len(self.parts), d_in.ctypes.data,
                                            d_out.ctypes.data, r_max, n_adapters, n_slots, max_loads_in_flight,
                                            flags)
        _check(st, "lora_cache_create")
        self.handle = h
        self.blobs = {}
        self._pools = {}
        self._scheds = []

    def blob_layout(self, rank: int):
        n = len(self.parts)
        a_off = np.zeros(n, np.int64)
        b_off = np.zeros(n, np.int64)
        total = ctypes.c_int64()
        _check(_lib.lora_cache_blob_layout(self.handle, rank, a_off.ctypes.data, b_off.ctypes.data,
                                           ctypes.byref(total)), "lora_cache_blob_layout")
        return a_off, b_off, total.value

    def register(self, adapter: int, rank: int, scale: float, A_parts=None, B_parts=None):
        """A_parts[p]: [d_in_p, rank], B_parts[p]: [rank, d_out_p] (any device)."""
        blob_ptr = None
        if not self.host_only:
            a_off, b_off, total = self.blob_layout(rank)
            blob = torch.zeros(total, dtype=self.dtype, pin_memory=True)
            for p, (di, do) in enumerate(self.parts):
                Ap, Bp = A_parts[p], B_parts[p]
                assert tuple(Ap.shape) == (di, rank) and tuple(Bp.shape) == (rank, do)
                blob[a_off[p]:a_off[p] + di * rank].copy_(Ap.reshape(-1))
                blob[b_off[p]:b_off[p] + rank * do].copy_(Bp.reshape(-1))
            self.blobs[adapter] = blob
            blob_ptr = _ptr(blob)
        _check(_lib.lora_cache_register(self.handle, adapter, rank, float(scale), blob_ptr),
               "lora_cache_register")

    def register_blob(self, adapter: int, rank: int, scale: float, blob: torch.Tensor):
        """Register an adapter whose host blob is already packed (a pinned
        1-D tensor of the cache dtype, ``blob_layout(rank)[2]`` elements)."""
        assert blob.dim() == 1 and blob.dtype == self.dtype and not blob.is_cuda
        assert blob.numel() == self.blob_layout(rank)[2]
        self.blobs[adapter] = blob
        _check(_lib.lora_cache_register(self.handle, adapter, rank, float(scale), _ptr(blob)),
               "lora_cache_register")

    def pin(self, adapter: int, pinned: bool = True):
        _check(_lib.lora_cache_pin(self.handle, adapter, int(bool(pinned))), "lora_cache_pin")

    def hold(self, adapter: int, delta: int):
        _check(_lib.lora_cache_hold(self.handle, adapter, int(delta)), "lora_cache_hold")

    def request(self, adapter: int) -> int:
        v = ctypes.c_int()
        _check(_lib.lora_cache_request(self.handle, adapter, ctypes.byref(v)), "lora_cache_request")
        return int(v.value)

    def poll(self) -> int:
        v = ctypes.c_int32()
        _check(_lib.lora_cache_poll(self.handle, ctypes.byref(v)), "lora_cache_poll")
        return int(v.value)

    def wait(self):
        _check(_lib.lora_cache_wait(self.handle), "lora_cache_wait")

    def _stream(self):
        return None if self.host_only else ctypes.c_void_p(_stream(self.device))

    def map(self, adapters) -> np.ndarray:
        """Host adapter ids -> host slot ids (raises LoraError with status
        LORA_E_NOT_RESIDENT when one is not resident)."""
        a = np.ascontiguousarray(adapters, np.int32)
        out = np.zeros(max(a.size, 1), np.int32)
        _check(_lib.lora_cache_map(self.handle, a.ctypes.data, a.size, out.ctypes.data, self._stream()),
               "lora_cache_map")
        return out[:a.size]

    def release(self):
        _check(_lib.lora_cache_release(self.handle, self._stream()), "lora_cache_release")

    def pool(self, part: int) -> Pool:
        if part not in self._pools:
            h = _lib.lora_cache_pool(self.handle, part)
            if not h:
                raise LoraError(LORA_E_INVALID, "lora_cache_pool")
            z = torch.empty(0, dtype=self.dtype, device=self.device)
            di, do = self.parts[part]
            self._pools[part] = Pool(ctypes.c_void_p(h), self.dtype, self.n_slots, di, do, self.r_max, z, z,
                                     owned=False)
        return self._pools[part]

    def slot_of(self, adapter: int) -> int:
        return int(_lib.lora_cache_slot_of(self.handle, adapter))

    def stats(self) -> dict:
        s = CacheStatsT()
        _check(_lib.lora_cache_stats(self.handle, ctypes.byref(s)), "lora_cache_stats")
        return {k: int(getattr(s, k)) for k, _ in CacheStatsT._fields_}

    def destroy(self):
        for sc in getattr(self, "_scheds", []):
            sc.destroy()
        if getattr(self, "handle", None):
            _check(_lib.lora_cache_destroy(self.handle), "lora_cache_destroy")
            self.handle = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


# --------------------------------------------------------------------------
# Adapter-aware admission
# --------------------------------------------------------------------------

class Scheduler:
    """lora_sched_*: forms each step's batch from a request queue.  ``cache``
    (a ``Cache`` or None) gates admission on residency."""

    def __init__(self, n_adapters: int, w_fair: float = 1.0, w_local: float = 0.35, max_adapters: int = 32,
                 max_rows: int = 256, rank_groups: bool = False, ranks=None, cache: Optional[Cache] = None):
        cfg = SchedConfigT(float(w_fair), float(w_local), int(max_adapters), int(max_rows), int(bool(rank_groups)))
        rk = None if ranks is None else np.ascontiguousarray(ranks, np.int32)
        h = ctypes.c_void_p()
        _check(_lib.lora_sched_create(ctypes.byref(h), ctypes.byref(cfg), n_adapters,
                                      None if rk is None else rk.ctypes.data,
                                      None if cache is None else cache.handle), "lora_sched_create")
        self.handle = h
        self.cache = cache   # kept alive: the scheduler holds adapters in it
        if cache is not None:
            cache._scheds.append(self)   # the cache destroys its schedulers first

    def submit(self, request: int, adapter: int, rows: int, arrival: float):
        _check(_lib.lora_sched_submit(self.handle, int(request), int(adapter), int(rows), float(arrival)),
               "lora_sched_submit")

    def step(self, now: float, capacity: int):
        """-> (requests, adapters, rows, waits) numpy arrays, info dict."""
        cap = max(int(capacity), 1)
        req = np.zeros(cap, np.int64)
        ad = np.zeros(cap, np.int32)
        rw = np.zeros(cap, np.int32)
        wt = np.zeros(cap, np.float64)
        info = SchedStepT()
        _check(_lib.lora_sched_step(self.handle, float(now), int(capacity), req.ctypes.data, ad.ctypes.data,
                                    rw.ctypes.data, wt.ctypes.data, ctypes.byref(info)), "lora_sched_step")
        k = info.admitted
        d = {f: getattr(info, f) for f, _ in SchedStepT._fields_}
        return (req[:k], ad[:k], rw[:k], wt[:k]), d

    def queued(self) -> int:
        return int(_lib.lora_sched_queued(self.handle))

    def destroy(self):
        if getattr(self, "handle", None):
            _check(_lib.lora_sched_destroy(self.handle), "lora_sched_destroy")
            self.handle = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass
