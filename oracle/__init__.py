"""CPU oracle for batched row-wise top-k -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import anything under ``oracle/``. The GPU library and its
Python binding never do, and the two sides share no code.

Contents
* :func:`topk` -- the plain definition (C full sort, ``topk_sort.c``): per row,
  all positions ordered by (key descending, index ascending), first k kept.
* :func:`keys` -- the order-preserving key of "CUDA 算子笔记 4" (milkfeng.top),
  section "改造 Radix Sort" (float_to_key), for 32- and 16-bit patterns.
* :mod:`oracle.model` -- the DeepSelect method model (DeepSelect deep-dive,
  section "算法"), instrumented for the quantities of its analysis section.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle_topk.so")

F32, BF16 = 0, 1
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH) or (
            os.path.getmtime(LIB_PATH) < os.path.getmtime(os.path.join(HERE, "topk_sort.c"))
        ):
            from oracle.build import build

            build()
        lib = ctypes.CDLL(LIB_PATH)
        lib.oracle_topk.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_int]
        lib.oracle_topk.restype = ctypes.c_int
        lib.oracle_key.argtypes = [ctypes.c_int, ctypes.c_uint32]
        lib.oracle_key.restype = ctypes.c_uint32
        _lib = lib
    return _lib


def raw_bits(x: np.ndarray) -> tuple[np.ndarray, int]:
    """(raw pattern array, dtype code) for float32 input or uint16 bfloat16 bits."""
    if x.dtype == np.float32:
        return x.view(np.uint32), F32
    if x.dtype == np.uint32:
        return x, F32
    if x.dtype == np.uint16:
        return x, BF16
    raise TypeError(f"oracle takes float32 or raw bfloat16 (uint16) rows, not {x.dtype}")


def keys(x: np.ndarray) -> np.ndarray:
    """Order-preserving unsigned key of every element (uint32 array).

    "CUDA 算子笔记 4", section "改造 Radix Sort": if the sign bit is set flip all
    bits, else flip only the sign bit; the 16-bit rule is the same on 16 bits.
    """
    raw, dt = raw_bits(np.asarray(x))
    u = raw.astype(np.uint32)
    if dt == F32:
        return np.where(u & np.uint32(0x80000000), ~u, u | np.uint32(0x80000000)).astype(np.uint32)
    return np.where(u & np.uint32(0x8000), (~u) & np.uint32(0xFFFF), u | np.uint32(0x8000)).astype(np.uint32)


def key_c(dtype: int, raw: int) -> int:
    """The C oracle's own key function (for cross-checks in tests)."""
    return int(_load().oracle_key(dtype, raw))


def topk(x: np.ndarray, k: int, nthreads: int | None = None):
    """Plain-definition top-k of every row of ``x`` ([batch, N]).

    Returns (vals, idx): vals holds the raw patterns (uint32 for float32 input,
    uint16 for bfloat16 bits) of the k selected elements in (key desc, index
    asc) order; idx the int32 columns.
    """
    x = np.ascontiguousarray(x)
    if x.ndim != 2:
        raise ValueError("oracle.topk expects a 2-D [batch, N] array")
    raw, dt = raw_bits(x)
    batch, n = raw.shape
    vals = np.empty((batch, k), dtype=raw.dtype)
    idx = np.empty((batch, k), dtype=np.int32)
    if nthreads is None:
        nthreads = os.cpu_count() or 1
    rc = _load().oracle_topk(raw.ctypes.data, dt, batch, n, n, k, vals.ctypes.data,
                             idx.ctypes.data, int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_topk rejected the arguments (status {rc})")
    return vals, idx
