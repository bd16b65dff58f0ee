"""CPU oracle for exact per-row top-k over ragged fp32 rows.

Test infrastructure. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` import this package; the product library
under ``exact_row_top_fp32_amd/`` never does, and this package imports nothing
from it. The arithmetic lives in ``topk_oracle.c`` (a full ``qsort`` of each
row); this module compiles it with gcc and marshals numpy arrays into it.

What the oracle computes is the plain definition of the result, from
"dsv4.1: Top-k kernels and candidate selection" (sglang PR #39648 report),
code excerpts, the docstring of the bf16 top-k entry, and "Fix incorrect
sparse-attention top-k selection when candidate bins overflow" (sglang PR
#37625), scope update in the comment thread:

* ``L = clamp(lengths[b], 0, n_cols)``, ``m = min(k, L)``;
* rank the positions ``[0, L)`` by value, descending, with ``+0`` above ``-0``
  and equal values by index, ascending;
* slots ``[0, m)`` get the first ``m`` positions (mapped through the page table
  in paged mode), slots ``[m, k)`` get ``-1``.

NaN inside ``[0, L)`` is outside the contract and raises ``ValueError``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import time

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "topk_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_topk.so")
_lib = None


def build() -> str:
    """Compile the C oracle into ``oracle/liboracle_topk.so`` (gcc, OpenMP)."""
    global _lib
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    _lib = None
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        lib.oracle_topk.restype = ctypes.c_int
        lib.oracle_topk.argtypes = [
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
        ]
        lib.oracle_max_threads.restype = ctypes.c_int
        lib.oracle_max_threads.argtypes = []
        _lib = lib
    return _lib


def max_threads() -> int:
    """Threads the oracle's parallel loop over rows uses by default."""
    return int(_load().oracle_max_threads())


def topk(scores: np.ndarray, lengths, k: int, *, n_cols: int | None = None,
         page_table: np.ndarray | None = None, page_size: int = 0,
         threads: int = 0) -> np.ndarray:
    """Exact top-k of every row; returns int32 ``[batch, k]``, best first.

    ``scores`` is a 2-D float32 array whose rows may be longer than ``n_cols``
    (the row stride is ``scores.strides[0]``); ``lengths`` is int32 ``[batch]``
    or ``None`` (every row has ``n_cols`` scores).
    """
    lib = _load()
    if scores.dtype != np.float32 or scores.ndim != 2 or scores.strides[1] != 4:
        raise ValueError("scores must be a 2-D float32 array with unit column stride")
    batch = scores.shape[0]
    # a single row's stride is meaningless (numpy reports 0 for a new axis)
    row_stride = scores.strides[0] // 4 if batch > 1 else scores.shape[1]
    if n_cols is None:
        n_cols = scores.shape[1]
    if lengths is not None:
        lengths = np.ascontiguousarray(lengths, dtype=np.int32)
        if lengths.shape != (batch,):
            raise ValueError("lengths must have shape [batch]")
    pt_ptr, pt_stride = None, 0
    if page_table is not None:
        page_table = np.ascontiguousarray(page_table, dtype=np.int32)
        pt_ptr, pt_stride = page_table.ctypes.data, page_table.shape[1]
    out = np.empty((batch, k), dtype=np.int32)
    rc = lib.oracle_topk(
        scores.ctypes.data if batch else None, batch, row_stride, n_cols,
        lengths.ctypes.data if lengths is not None else None, k,
        pt_ptr, pt_stride, page_size, out.ctypes.data if batch else None, threads)
    if rc == 2:
        raise ValueError("NaN inside a row's valid range is outside the oracle's contract")
    if rc != 0:
        raise ValueError(f"oracle_topk rejected its arguments (code {rc})")
    return out


def timed_topk(*args, **kwargs):
    """``topk`` plus its wall time in seconds (for the CPU baseline)."""
    t0 = time.perf_counter()
    out = topk(*args, **kwargs)
    return out, time.perf_counter() - t0
