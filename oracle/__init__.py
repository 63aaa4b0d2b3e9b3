"""fp64 CPU oracle for the multi-LoRA batched layer (ctypes shim over lora_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may use this package; the product path
(``lora_bgmv_shrink_amd``) never imports it, and this package imports
nothing from the product.

The arithmetic lives in ``lora_oracle.c`` (see its header for the pages'
definitions it follows).  This file only marshals numpy arrays.

Parity pins for every function here are in ``tests/test_oracle_pins.py``;
none of them is unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "lora_oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")

_lock = threading.Lock()
_lib = None


def build(src: str = SRC, out: str = LIB, extra=()) -> str:
    """Compile the oracle with gcc (-O3, OpenMP, strict C11: no fast-math, no
    contraction into fused multiply-adds)."""
    cmd = ["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c11", *extra, src, "-o", out + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _bind(lib):
    i64, i32, p = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    lib.oracle_segments.restype = i64
    lib.oracle_segments.argtypes = [p, i64, i32, p, p, p, p]
    lib.oracle_layer.restype = i64
    lib.oracle_layer.argtypes = [i64, i64, i64, p, p, p, i32, p, p, p, p, p, p, i32,
                                 p, i64, p, p, p, ctypes.c_int]
    lib.oracle_count_bad_ids.restype = i64
    lib.oracle_count_bad_ids.argtypes = [p, i64, i32]
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_merge.restype = ctypes.c_int
    lib.oracle_merge.argtypes = [i64, i64, p, i32, i32, p, p, p, p, p, p, ctypes.c_double, ctypes.c_int]
    lib.oracle_dequant_q4.restype = None
    lib.oracle_dequant_q4.argtypes = [i64, i64, p, i64, p, i64, i64, p]
    return lib


def load(path: Optional[str] = None):
    """Load (building when absent or stale) and return the ctypes library.
    LORA_ORACLE_LIB names a prebuilt copy to load instead (the sanitizer
    run's instrumented build)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    with _lock:
        if _lib is None and os.environ.get("LORA_ORACLE_LIB"):
            _lib = _bind(ctypes.CDLL(os.environ["LORA_ORACLE_LIB"]))
        if _lib is None:
            if (not os.path.exists(LIB)) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
                build()
            _lib = _bind(ctypes.CDLL(LIB))
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


@dataclass
class OraclePool:
    """A packed pool in fp64: adapter u is ``A[a_off[u]:...]`` as [d_in, r_u]
    and ``B[b_off[u]:...]`` as [r_u, d_out] (row-major)."""
    n_adapters: int
    d_in: int
    d_out: int
    r_max: int
    ranks: np.ndarray
    a_off: np.ndarray
    b_off: np.ndarray
    A: np.ndarray
    B: np.ndarray
    scales: np.ndarray

    @staticmethod
    def uniform(A3: np.ndarray, B3: np.ndarray, scales) -> "OraclePool":
        n, d_in, r = A3.shape
        d_out = B3.shape[2]
        u = np.arange(n, dtype=np.int64)
        return OraclePool(n, d_in, d_out, r, np.full(n, r, np.int32), u * d_in * r, u * r * d_out,
                          _c(A3, np.float64).reshape(-1), _c(B3, np.float64).reshape(-1),
                          _c(np.broadcast_to(np.asarray(scales, np.float64), (n,)), np.float64))


def segments(ids, n_adapters: int, lib=None):
    """Stable group-by of ``ids``: returns (perm, seg_ids, seg_off, n_bad)."""
    lib = lib or load()
    ids = _c(ids, np.int32)
    n = ids.shape[0]
    perm = np.empty(n, np.int32)
    cap = min(n, n_adapters + 1) + 1
    seg_ids = np.empty(cap, np.int32)
    seg_off = np.empty(cap + 1, np.int32)
    n_seg = np.zeros(1, np.int32)
    bad = lib.oracle_segments(_ptr(ids), n, int(n_adapters), _ptr(perm), _ptr(seg_ids),
                              _ptr(seg_off), _ptr(n_seg))
    k = int(n_seg[0])
    return perm, seg_ids[:k].copy(), seg_off[:k + 1].copy(), int(bad)


def layer(x, W, ids, pool: OraclePool, rows: Optional[Sequence[int]] = None,
          want=("t", "lora", "y"), threads: int = 0, lib=None):
    """Run the oracle.  ``x`` [n, d_in] and ``W`` [d_in, d_out] (or None) are
    widened to fp64.  Returns a dict with the requested outputs (full-size
    arrays; rows outside ``rows`` are zero) and ``bad`` (invalid-id count)."""
    lib = lib or load()
    x = _c(x, np.float64)
    n, d_in = x.shape
    assert d_in == pool.d_in
    Wd = None if W is None else _c(W, np.float64)
    if Wd is not None:
        assert Wd.shape == (pool.d_in, pool.d_out)
    ids = _c(ids, np.int32)
    assert ids.shape == (n,)
    sel = None if rows is None else _c(rows, np.int64)
    out = {}
    t = np.zeros((n, pool.r_max)) if "t" in want else None
    lo = np.zeros((n, pool.d_out)) if "lora" in want else None
    y = np.zeros((n, pool.d_out)) if "y" in want else None
    bad = lib.oracle_layer(n, d_in, pool.d_out, _ptr(x), _ptr(Wd), _ptr(ids), pool.n_adapters,
                           _ptr(_c(pool.ranks, np.int32)), _ptr(_c(pool.a_off, np.int64)),
                           _ptr(_c(pool.b_off, np.int64)), _ptr(_c(pool.A, np.float64)),
                           _ptr(_c(pool.B, np.float64)), _ptr(_c(pool.scales, np.float64)),
                           pool.r_max, _ptr(sel), 0 if sel is None else sel.shape[0],
                           _ptr(t), _ptr(lo), _ptr(y), int(threads))
    if t is not None:
        out["t"] = t
    if lo is not None:
        out["lora"] = lo
    if y is not None:
        out["y"] = y
    out["bad"] = int(bad)
    return out


def merge(W, pool: OraclePool, adapter: int, sign: float = 1.0, threads: int = 0, lib=None) -> np.ndarray:
    """``W + sign * s_a * A_a B_a`` in fp64 for ``W`` [d_in, d_out] (a new
    array; ``W`` is not modified).  Raises for an adapter outside the pool."""
    lib = lib or load()
    out = np.array(_c(W, np.float64), dtype=np.float64, copy=True)
    assert out.shape == (pool.d_in, pool.d_out)
    rc = lib.oracle_merge(pool.d_in, pool.d_out, _ptr(out), int(adapter), pool.n_adapters,
                          _ptr(_c(pool.ranks, np.int32)), _ptr(_c(pool.a_off, np.int64)),
                          _ptr(_c(pool.b_off, np.int64)), _ptr(_c(pool.A, np.float64)),
                          _ptr(_c(pool.B, np.float64)), _ptr(_c(pool.scales, np.float64)),
                          float(sign), int(threads))
    if rc != 0:
        raise ValueError(f"adapter {adapter} outside [0, {pool.n_adapters})")
    return out


def dequant_q4(q, scale, d_in: int, group: int = 128, lib=None) -> np.ndarray:
    """4-bit base weight -> fp64 W [d_in, d_out].  ``q`` [d_out, ldq] uint8
    (two signed nibbles per byte, low nibble first), ``scale`` [d_out, lds]
    (widened to fp64 exactly)."""
    lib = lib or load()
    q = _c(q, np.uint8)
    sc = _c(scale, np.float64)
    d_out = q.shape[0]
    assert q.shape[1] * 2 >= d_in and sc.shape[0] == d_out and sc.shape[1] * group >= d_in
    W = np.empty((d_in, d_out), np.float64)
    lib.oracle_dequant_q4(d_in, d_out, _ptr(q), q.shape[1], _ptr(sc), sc.shape[1], group, _ptr(W))
    return W


def max_threads(lib=None) -> int:
    return int((lib or load()).oracle_max_threads())
