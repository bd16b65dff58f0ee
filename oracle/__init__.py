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

Three more definitions, from the same sglang report (implementation section 2
and code excerpts), for the kernels that sit beside this selection:

* ``topk_bf16``: the same selection over bf16 scores (rows of at most 16384,
  k at most 2048); a bf16 value widens exactly to the fp32 whose top 16 bits
  it is, and the fp32 definition above applies to the widened row;
* ``amax8``: the two-level indexer's level-one keys, the largest of every 8
  scores, the newest block +inf, rows with at most ``topk`` blocks untouched;
* ``sort_candidate_blocks``: the selected block ids of a row in ascending
  order, with their pool slots.
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


# ----------------------------------------------------------------------------
# bf16 rows
# ----------------------------------------------------------------------------

def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> the fp32 values they denote, exactly: a
    bf16 number is the fp32 number whose low 16 bits are zero."""
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise ValueError("bf16 rows are passed as their uint16 bit patterns")
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def topk_bf16(bits: np.ndarray, lengths, k: int, *, n_cols: int | None = None,
              page_table: np.ndarray | None = None, page_size: int = 0,
              threads: int = 0) -> np.ndarray:
    """Exact top-k of bf16 rows ("dsv4.1: Top-k kernels and candidate
    selection", code excerpts, docstring of the bf16 small-row entry: the k
    best of the first lengths[b] scores, -1 past min(k, lengths[b]), page-table
    transform, at most 16384 scores per row and k at most 2048).

    ``bits`` is uint16 ``[batch, row_stride]``; the rows are widened exactly to
    fp32 and selected by ``topk``, so the order, the tie rule and the length
    clamp are the fp32 ones.
    """
    if n_cols is None:
        n_cols = bits.shape[1]
    if n_cols > 16384 or not 1 <= k <= 2048:
        raise ValueError("bf16 rows hold at most 16384 scores and k is at most 2048")
    return topk(bf16_to_f32(bits), lengths, k, n_cols=n_cols, page_table=page_table,
                page_size=page_size, threads=threads)


# ----------------------------------------------------------------------------
# the two-level indexer's neighbours
# ----------------------------------------------------------------------------

def _block_max(blocks: np.ndarray) -> np.ndarray:
    """Largest of each row of ``blocks`` (float32 [n, 8]): NaN ignored, +0
    above -0; NaN for a block of NaN only."""
    nan = np.isnan(blocks)
    top = np.where(nan, np.float32(-np.inf), blocks).max(axis=1)
    pos_zero = ((blocks == 0) & ~np.signbit(blocks)).any(axis=1)
    top = np.where(top == 0, np.where(pos_zero, np.float32(0.0), np.float32(-0.0)), top)
    return np.where(nan.all(axis=1), np.float32(np.nan), top).astype(np.float32)


def amax8(scores: np.ndarray, lengths, topk: int, out: np.ndarray, *, n_cols: int | None = None) -> np.ndarray:
    """Block keys for the first stage of the two-level indexer, as defined for
    the block-max kernel on "dsv4.1: Top-k kernels and candidate selection"
    (implementation section 2 and the ``amax8_varlen`` entry among the code
    excerpts). Written into ``out`` in place.

    Row b keeps L = clamp(lengths[b], 0, n_cols) scores (``lengths`` None:
    every row n_cols; n_cols defaults to the width of ``scores``), grouped
    into nb = ceil(L / 8) blocks of 8. Block i < nb - 1 gets the largest of
    its 8 scores, ranking +0 above -0 and skipping NaN (an all-NaN block
    gives NaN). Block nb - 1, the most recent one, is set to +inf so that a
    later top-k always keeps it. Columns from nb on are not touched, and
    neither is any row whose nb is at most ``topk`` when ``topk > 0``,
    since such a row keeps every block. ``out`` needs at least
    ceil(n_cols / 8) columns.
    """
    scores = np.asarray(scores, dtype=np.float32)
    n_cols = scores.shape[1] if n_cols is None else n_cols
    for b in range(scores.shape[0]):
        L = n_cols if lengths is None else min(max(int(lengths[b]), 0), n_cols)
        nb = -(-L // 8)
        if nb > out.shape[1] or L > scores.shape[1]:
            raise ValueError("a row's blocks do not fit the output or its scores")
        if nb == 0 or (topk > 0 and nb <= topk):
            continue
        if nb > 1:
            out[b, :nb - 1] = _block_max(scores[b, :8 * (nb - 1)].reshape(nb - 1, 8))
        out[b, nb - 1] = np.inf
    return out


INT32_MAX = 2**31 - 1


def sort_candidate_blocks(blocks: np.ndarray, lengths, page_table: np.ndarray,
                          page_size: int, *, n_cols: int):
    """Candidate block table of the two-level indexer, as defined for the
    block-table kernel on "dsv4.1: Top-k kernels and candidate selection"
    (implementation section 2 and the ``sort_candidate_blocks`` entry among
    the code excerpts).

    Row b holds k = blocks.shape[1] block ids. Its length is clamped like
    every other length on the path, L = clamp(lengths[b], 0, n_cols)
    (``lengths`` None: every row n_cols), and it spans nb = ceil(L / 8)
    blocks. With nb <= k the result is 0 .. nb-1 and the ids given are
    ignored; with nb > k it is the distinct given ids inside [0, nb), in
    increasing order (all k of them when the ids come from a top-k
    selection). INT32_MAX pads the rest of the row. The page output maps id
    to ``page_table[b, id // bpp] * bpp + id % bpp`` with
    ``bpp = page_size // 8`` and carries the same padding.
    Returns ``(table, pages)``, both int32 ``[batch, k]``.
    """
    if page_size < 8 or page_size & (page_size - 1):
        raise ValueError("page_size must be a power of two, at least 8")
    if n_cols < 0:
        raise ValueError("n_cols must be non-negative")
    bpp = page_size // 8
    B, k = blocks.shape
    table = np.full((B, k), INT32_MAX, dtype=np.int32)
    pages = np.full((B, k), INT32_MAX, dtype=np.int32)
    for b in range(B):
        L = n_cols if lengths is None else min(max(int(lengths[b]), 0), n_cols)
        nb = -(-L // 8)
        if nb <= k:
            ids = np.arange(nb, dtype=np.int64)
        else:
            row = blocks[b].astype(np.int64)
            ids = np.unique(row[(row >= 0) & (row < nb)])
        table[b, :ids.size] = ids
        slot = page_table[b, ids // bpp].astype(np.int64) * bpp + ids % bpp
        pages[b, :ids.size] = slot
    return table, pages
