"""Exact per-row top-k over long, ragged fp32 rows on MI355X (gfx950).

A thin ctypes binding of ``libexact_topk.so`` (C ABI in ``include/exact_topk.h``).
The functions keep the C names and only marshal torch tensors into pointers,
sizes and the current HIP stream; every step of the selection runs in the HIP
kernels. There is no fallback: if the library is not built, or the tensors do
not live on a GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "topk_select", "topk_select_ex", "topk_select_split", "topk_split_workspace_bytes",
    "topk_split_capacity", "topk_select_split_noalloc", "SPLIT_NOALLOC_MAX_BATCH", "topk_select_bf16",
    "amax8_varlen", "sort_candidate_blocks",
    "topk_select_bf16_ex", "topk_status_string", "topk_max_capacity", "topk_short_capacity",
    "topk_watchdog_trips", "KERNEL_AUTO", "KERNEL_PERSISTENT", "KERNEL_SHORT",
    "TopKError", "library_path", "PATH_AUTO", "PATH_LDS", "PATH_SAMPLED", "PATH_FULLROW",
    "ROW_EMPTY", "ROW_ALL", "ROW_LDS", "ROW_SAMPLED", "ROW_FULL_OVERFLOW",
    "ROW_FULL_UNDERFLOW", "ROW_FULL_FORCED", "MAX_K",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_PKG, "libexact_topk.so")

MAX_K = 2048
PATH_AUTO, PATH_LDS, PATH_SAMPLED, PATH_FULLROW = 0, 1, 2, 3
KERNEL_AUTO, KERNEL_PERSISTENT, KERNEL_SHORT = 0, 1, 2
SPLIT_NOALLOC_MAX_BATCH = 256
(ROW_EMPTY, ROW_ALL, ROW_LDS, ROW_SAMPLED, ROW_FULL_OVERFLOW, ROW_FULL_UNDERFLOW,
 ROW_FULL_FORCED) = range(7)


class TopKError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


class _Options(ctypes.Structure):
    _fields_ = [("force_path", ctypes.c_int32), ("capacity", ctypes.c_int32),
                ("row_stats", ctypes.c_void_p), ("kernel", ctypes.c_int32)]


_lib = None
_ARGS = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
         ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
         ctypes.c_void_p]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise ImportError(
                f"{library_path} is missing: build it with `python -m exact_row_top_fp32_amd.build`")
        lib = ctypes.CDLL(library_path)
        lib.topk_select.restype = ctypes.c_int
        lib.topk_select.argtypes = _ARGS
        lib.topk_select_ex.restype = ctypes.c_int
        lib.topk_select_ex.argtypes = _ARGS + [ctypes.POINTER(_Options)]
        lib.topk_status_string.restype = ctypes.c_char_p
        lib.topk_status_string.argtypes = [ctypes.c_int]
        lib.topk_max_capacity.restype = ctypes.c_int32
        lib.topk_max_capacity.argtypes = []
        lib.topk_short_capacity.restype = ctypes.c_int32
        lib.topk_short_capacity.argtypes = []
        lib.topk_watchdog_trips.restype = ctypes.c_uint32
        lib.topk_watchdog_trips.argtypes = []
        lib.topk_select_split.restype = ctypes.c_int
        lib.topk_select_split.argtypes = (_ARGS[:-1] + [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                                         ctypes.c_void_p, ctypes.POINTER(_Options)])
        lib.topk_select_split_noalloc.restype = ctypes.c_int
        lib.topk_select_split_noalloc.argtypes = (_ARGS[:-1] + [ctypes.c_int32, ctypes.c_void_p,
                                                                 ctypes.POINTER(_Options)])
        lib.topk_split_workspace_bytes.restype = ctypes.c_int64
        lib.topk_split_workspace_bytes.argtypes = [ctypes.c_int64]
        lib.topk_split_capacity.restype = ctypes.c_int32
        lib.topk_split_capacity.argtypes = []
        lib.topk_select_bf16.restype = ctypes.c_int
        lib.topk_select_bf16.argtypes = _ARGS
        lib.topk_select_bf16_ex.restype = ctypes.c_int
        lib.topk_select_bf16_ex.argtypes = _ARGS + [ctypes.POINTER(_Options)]
        lib.amax8_varlen.restype = ctypes.c_int
        lib.amax8_varlen.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                     ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64,
                                     ctypes.c_void_p]
        lib.sort_candidate_blocks.restype = ctypes.c_int
        lib.sort_candidate_blocks.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                              ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                              ctypes.c_void_p, ctypes.c_void_p]
        _lib = lib
    return _lib


def topk_status_string(status: int) -> str:
    return _load().topk_status_string(status).decode()


def topk_max_capacity() -> int:
    return int(_load().topk_max_capacity())


def topk_short_capacity() -> int:
    return int(_load().topk_short_capacity())


def topk_watchdog_trips() -> int:
    """Workgroups that gave up a bounded wait since load (nonzero means a defect)."""
    return int(_load().topk_watchdog_trips())


def _device_ptr(t: torch.Tensor | None, name: str, dtype: torch.dtype):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _same_device(device, **tensors):
    for name, t in tensors.items():
        if t is not None and isinstance(t, torch.Tensor) and t.device != device:
            raise ValueError(f"{name} is on {t.device}, scores on {device}")


def _stream_handle(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _marshal(scores, lengths, k, out, page_table, page_size, n_cols, stream, dtype=torch.float32):
    if scores.dim() != 2 or (scores.size(1) > 1 and scores.stride(1) != 1):
        raise ValueError("scores must be 2-D with unit column stride")
    batch = scores.size(0)
    row_stride = scores.stride(0) if batch > 1 else max(scores.size(1), 1)
    if n_cols is None:
        n_cols = scores.size(1)
    if n_cols > scores.size(1):
        raise ValueError("n_cols exceeds the width of scores")
    if lengths is not None:
        if lengths.dim() != 1 or lengths.size(0) != batch or not lengths.is_contiguous():
            raise ValueError("lengths must be a contiguous [batch] tensor")
    if out is None:
        out = torch.empty((batch, k), dtype=torch.int32, device=scores.device)
    elif out.shape != (batch, k) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [batch, k] tensor")
    pt_stride = 0
    if page_table is not None:
        if page_table.dim() != 2 or page_table.size(0) != batch or (
                page_table.size(1) > 1 and page_table.stride(1) != 1):
            raise ValueError("page_table must be [batch, pages] with unit column stride")
        if page_size >= 1 and page_table.size(1) < -(-n_cols // page_size):
            raise ValueError(f"page_table has {page_table.size(1)} columns; rows of {n_cols} scores "
                             f"span {-(-n_cols // page_size)} pages of {page_size}")
        pt_stride = page_table.stride(0) if batch > 1 else page_table.size(1)
    _same_device(scores.device, lengths=lengths, out=out, page_table=page_table)
    handle = _stream_handle(stream, scores.device)
    args = (
        _device_ptr(scores, "scores", dtype), batch, row_stride, n_cols,
        _device_ptr(lengths, "lengths", torch.int32), int(k),
        _device_ptr(out, "out", torch.int32), _device_ptr(page_table, "page_table", torch.int32),
        pt_stride, int(page_size), handle,
    )
    return args, out


def _check(status: int):
    if status != 0:
        raise TopKError(status, topk_status_string(status))


def topk_select(scores: torch.Tensor, lengths: torch.Tensor | None, k: int,
                out: torch.Tensor | None = None, page_table: torch.Tensor | None = None,
                page_size: int = 0, *, n_cols: int | None = None, stream=None) -> torch.Tensor:
    """Exact top-k of every row of ``scores`` (fp32 ``[batch, >= n_cols]``).

    Returns ``out`` (int32 ``[batch, k]``): positions (or page-table slots) of
    each row's k best scores in no particular order, ``-1`` past
    ``min(k, lengths[b])``. Asynchronous on ``stream`` (default: the current
    torch stream).
    """
    args, out = _marshal(scores, lengths, k, out, page_table, page_size, n_cols, stream)
    _check(_load().topk_select(*args))
    return out


def _options(scores, force_path, capacity, row_stats, kernel):
    if row_stats is not None and (row_stats.shape != (scores.size(0), 2) or not row_stats.is_contiguous()):
        raise ValueError("row_stats must be a contiguous [batch, 2] tensor")
    _same_device(scores.device, row_stats=row_stats)
    return _Options(int(force_path), int(capacity), _device_ptr(row_stats, "row_stats", torch.int32), int(kernel))


def topk_select_ex(scores: torch.Tensor, lengths: torch.Tensor | None, k: int,
                   out: torch.Tensor | None = None, page_table: torch.Tensor | None = None,
                   page_size: int = 0, *, n_cols: int | None = None, stream=None,
                   force_path: int = PATH_AUTO, capacity: int = 0,
                   row_stats: torch.Tensor | None = None, kernel: int = KERNEL_AUTO) -> torch.Tensor:
    """``topk_select`` with path forcing, a capacity override, row statistics
    and a kernel choice.

    ``row_stats`` (int32 ``[batch, 2]``, contiguous) receives the path code
    and the sampled survivor count (or the length) of every row.
    """
    args, out = _marshal(scores, lengths, k, out, page_table, page_size, n_cols, stream)
    opt = _options(scores, force_path, capacity, row_stats, kernel)
    _check(_load().topk_select_ex(*args, ctypes.byref(opt)))
    return out


def topk_split_workspace_bytes(batch: int) -> int:
    """Bytes of device workspace ``topk_select_split`` needs for ``batch`` rows."""
    return int(_load().topk_split_workspace_bytes(int(batch)))


def topk_split_capacity() -> int:
    """Survivor entries per row in the split-row workspace."""
    return int(_load().topk_split_capacity())


def topk_select_split(scores: torch.Tensor, lengths: torch.Tensor | None, k: int,
                      out: torch.Tensor | None = None, page_table: torch.Tensor | None = None,
                      page_size: int = 0, *, workspace: torch.Tensor | None = None, pieces: int = 0,
                      n_cols: int | None = None, stream=None, force_path: int = PATH_AUTO,
                      capacity: int = 0, row_stats: torch.Tensor | None = None) -> torch.Tensor:
    """``topk_select`` with every row split over several workgroups (small batches).

    Same result as ``topk_select``. ``workspace`` is a uint8 GPU tensor of at
    least ``topk_split_workspace_bytes(batch)`` bytes (allocated here when
    omitted); ``pieces`` is the number of workgroups per row (0 = automatic).
    """
    args, out = _marshal(scores, lengths, k, out, page_table, page_size, n_cols, stream)
    opt = _options(scores, force_path, capacity, row_stats, KERNEL_AUTO)
    need = topk_split_workspace_bytes(scores.size(0))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=scores.device)
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    _same_device(scores.device, workspace=workspace)
    status = _load().topk_select_split(*args[:-1], _device_ptr(workspace, "workspace", torch.uint8),
                                       workspace.numel(), int(pieces), args[-1], ctypes.byref(opt))
    _check(status)
    return out


def topk_select_split_noalloc(scores: torch.Tensor, lengths: torch.Tensor | None, k: int,
                              out: torch.Tensor, page_table: torch.Tensor | None = None,
                              page_size: int = 0, *, pieces: int = 0, n_cols: int | None = None,
                              stream=None, force_path: int = PATH_AUTO, capacity: int = 0,
                              row_stats: torch.Tensor | None = None) -> torch.Tensor:
    """``topk_select_split`` with its workspace in a fixed device array inside
    the library (at most ``SPLIT_NOALLOC_MAX_BATCH`` rows): neither the
    library nor this binding allocates device memory, so ``out`` must be
    given. Calls that can overlap in time on one GPU share the array and race.
    """
    if out is None:
        raise ValueError("out must be given: this entry allocates nothing")
    args, out = _marshal(scores, lengths, k, out, page_table, page_size, n_cols, stream)
    opt = _options(scores, force_path, capacity, row_stats, KERNEL_AUTO)
    _check(_load().topk_select_split_noalloc(*args[:-1], int(pieces), args[-1], ctypes.byref(opt)))
    return out


def topk_select_bf16(scores: torch.Tensor, lengths: torch.Tensor | None, k: int,
                     out: torch.Tensor | None = None, page_table: torch.Tensor | None = None,
                     page_size: int = 0, *, n_cols: int | None = None, stream=None) -> torch.Tensor:
    """Exact top-k of bf16 rows of at most 16384 scores (``scores`` bfloat16
    ``[batch, >= n_cols]``); same result as ``topk_select`` on the rows
    widened to fp32."""
    if scores.dtype != torch.bfloat16:
        raise TypeError(f"scores must be torch.bfloat16, got {scores.dtype}")
    args, out = _marshal(scores, lengths, k, out, page_table, page_size, n_cols, stream,
                         dtype=torch.bfloat16)
    _check(_load().topk_select_bf16(*args))
    return out


def topk_select_bf16_ex(scores: torch.Tensor, lengths: torch.Tensor | None, k: int,
                        out: torch.Tensor | None = None, page_table: torch.Tensor | None = None,
                        page_size: int = 0, *, n_cols: int | None = None, stream=None,
                        force_path: int = PATH_AUTO, capacity: int = 0,
                        row_stats: torch.Tensor | None = None) -> torch.Tensor:
    """``topk_select_bf16`` with path forcing, a capacity override (at most
    ``topk_short_capacity()``) and row statistics, as ``topk_select_ex``."""
    if scores.dtype != torch.bfloat16:
        raise TypeError(f"scores must be torch.bfloat16, got {scores.dtype}")
    args, out = _marshal(scores, lengths, k, out, page_table, page_size, n_cols, stream,
                         dtype=torch.bfloat16)
    opt = _options(scores, force_path, capacity, row_stats, KERNEL_AUTO)
    _check(_load().topk_select_bf16_ex(*args, ctypes.byref(opt)))
    return out


def amax8_varlen(scores: torch.Tensor, lengths: torch.Tensor | None, topk: int = 0, *,
                 max_seqlen: int = 0, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Block keys for the indexer's first stage (the block-max kernel of
    "dsv4.1: Top-k kernels and candidate selection", implementation section 2;
    signature kept from that page's entry so callers can switch). Row b's
    first L = clamp(lengths[b], 0, max_seqlen) scores form ceil(L / 8) blocks
    of 8; each block but the last gets its largest score (NaN skipped, +0
    ranked above -0), the last gets +inf, and later columns are not written.
    With ``topk > 0`` a row of at most ``topk`` blocks is not written at all;
    ``topk = 0`` writes every row. ``out`` is fp32 ``[batch, >= ceil(max_seqlen
    / 8)]``, allocated uninitialised when omitted; ``max_seqlen`` = 0 means
    the width of ``scores``."""
    if scores.dim() != 2 or (scores.size(1) > 1 and scores.stride(1) != 1):
        raise ValueError("scores must be 2-D with unit column stride")
    batch = scores.size(0)
    n_cols = max_seqlen if max_seqlen > 0 else scores.size(1)
    if n_cols > scores.size(1):
        raise ValueError("max_seqlen exceeds the width of scores")
    if out is None:
        out = torch.empty((batch, (n_cols + 7) // 8), dtype=torch.float32, device=scores.device)
    if out.dim() != 2 or out.size(0) != batch or (out.size(1) > 1 and out.stride(1) != 1):
        raise ValueError("out must be [batch, blocks] with unit column stride")
    if lengths is not None and (lengths.dim() != 1 or lengths.size(0) != batch or not lengths.is_contiguous()):
        raise ValueError("lengths must be a contiguous [batch] tensor")
    _same_device(scores.device, lengths=lengths, out=out)
    row_stride = scores.stride(0) if batch > 1 else max(scores.size(1), 1)
    out_stride = out.stride(0) if batch > 1 else out.size(1)
    _check(_load().amax8_varlen(_device_ptr(scores, "scores", torch.float32), batch, row_stride, n_cols,
                                _device_ptr(lengths, "lengths", torch.int32), int(topk),
                                _device_ptr(out, "out", torch.float32), out_stride,
                                _stream_handle(stream, scores.device)))
    return out


def sort_candidate_blocks(blocks: torch.Tensor, lengths: torch.Tensor | None, page_table: torch.Tensor,
                          page_size: int, *, out_pages: torch.Tensor | None = None,
                          n_cols: int | None = None, stream=None) -> torch.Tensor:
    """The two-level indexer's block table, in place: ``blocks`` (int32
    ``[batch, k]``, selected block ids in any order) becomes the ids ascending,
    ``INT32_MAX`` padded (the identity table for rows with at most k blocks);
    ``out_pages`` receives ``page_table[b, id // bpp] * bpp + id % bpp``,
    ``bpp = page_size // 8``. ``n_cols`` (the largest length, in positions)
    defaults to ``8 * page_table.size(1) * bpp``. Returns ``out_pages``."""
    if blocks.dim() != 2 or not blocks.is_contiguous():
        raise ValueError("blocks must be a contiguous [batch, k] tensor")
    batch, k = blocks.shape
    if out_pages is None:
        out_pages = torch.empty_like(blocks)
    if out_pages.shape != blocks.shape or not out_pages.is_contiguous():
        raise ValueError("out_pages must be a contiguous tensor shaped like blocks")
    if page_table.dim() != 2 or page_table.size(0) != batch or (
            page_table.size(1) > 1 and page_table.stride(1) != 1):
        raise ValueError("page_table must be [batch, pages] with unit column stride")
    if lengths is not None and (lengths.dim() != 1 or lengths.size(0) != batch or not lengths.is_contiguous()):
        raise ValueError("lengths must be a contiguous [batch] tensor")
    bpp = max(page_size // 8, 1)
    if n_cols is None:
        n_cols = 8 * page_table.size(1) * bpp
    if page_table.size(1) < -(-(-(-n_cols // 8)) // bpp):
        raise ValueError(f"page_table has {page_table.size(1)} columns; rows of {n_cols} positions "
                         f"span {-(-(-(-n_cols // 8)) // bpp)} pages of {bpp} blocks")
    _same_device(blocks.device, lengths=lengths, page_table=page_table, out_pages=out_pages)
    pt_stride = page_table.stride(0) if batch > 1 else page_table.size(1)
    _check(_load().sort_candidate_blocks(_device_ptr(blocks, "blocks", torch.int32), batch, int(k),
                                         _device_ptr(lengths, "lengths", torch.int32), int(n_cols),
                                         _device_ptr(page_table, "page_table", torch.int32), pt_stride,
                                         int(page_size), _device_ptr(out_pages, "out_pages", torch.int32),
                                         _stream_handle(stream, blocks.device)))
    return out_pages
