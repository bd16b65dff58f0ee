"""The C ABI without a GPU: exported symbols and host-side argument checks.

Every function declared in include/*.h must be exported by the built library.
Argument errors are decided on the host before any HIP call, so they are
checked here with pointers that are never dereferenced.
"""
from __future__ import annotations

import ctypes
import glob
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "exact_row_top_fp32_amd", "libexact_topk.so")

ARGS = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
        ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
        ctypes.c_void_p]


class Options(ctypes.Structure):
    _fields_ = [("force_path", ctypes.c_int32), ("capacity", ctypes.c_int32),
                ("row_stats", ctypes.c_void_p), ("kernel", ctypes.c_int32)]


def header_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^(?:const\s+)?(?:int|int32_t|int64_t|uint32_t|char)\s*\*?\s*(\w+)\s*\(",
                            text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from exact_row_top_fp32_amd import build
        build.build()
    lib = ctypes.CDLL(LIB)
    lib.topk_select.argtypes = ARGS
    lib.topk_select.restype = ctypes.c_int
    lib.topk_select_ex.argtypes = ARGS + [ctypes.POINTER(Options)]
    lib.topk_select_ex.restype = ctypes.c_int
    lib.topk_status_string.restype = ctypes.c_char_p
    lib.topk_max_capacity.restype = ctypes.c_int32
    lib.topk_select_split.argtypes = ARGS[:-1] + [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                                   ctypes.c_void_p, ctypes.POINTER(Options)]
    lib.topk_select_split.restype = ctypes.c_int
    lib.topk_split_workspace_bytes.argtypes = [ctypes.c_int64]
    lib.topk_split_workspace_bytes.restype = ctypes.c_int64
    lib.topk_split_capacity.restype = ctypes.c_int32
    return lib


def test_header_declares_the_entry_points():
    assert header_functions() == sorted(
        ["topk_select", "topk_select_ex", "topk_status_string", "topk_max_capacity",
         "topk_short_capacity", "topk_watchdog_trips", "topk_select_split", "topk_split_workspace_bytes",
         "topk_split_capacity", "topk_select_split_noalloc", "topk_select_bf16", "topk_select_bf16_ex",
         "amax8_varlen", "sort_candidate_blocks"])


def test_every_declared_symbol_is_exported(lib):
    for name in header_functions():
        assert hasattr(lib, name), name
    dyn = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    for name in header_functions():
        assert re.search(rf"\bT {name}\b", dyn), name


def test_library_targets_gfx950():
    out = subprocess.run(["strings", LIB], capture_output=True, text=True).stdout
    assert "gfx950" in out


FAKE = 0x10000  # 16-byte aligned, never dereferenced


def call(lib, scores=FAKE, batch=4, row_stride=1024, n_cols=1024, lengths=None, k=16,
         out=FAKE, page_table=None, pt_stride=0, page_size=0, opt=None):
    a = (scores, batch, row_stride, n_cols, lengths, k, out, page_table, pt_stride, page_size, None)
    if opt is None:
        return lib.topk_select(*a)
    return lib.topk_select_ex(*a, ctypes.byref(opt))


def test_host_argument_checks(lib):
    assert call(lib, k=0) == 2 and call(lib, k=2049) == 2 and call(lib, k=-5) == 2
    assert call(lib, batch=-1) == 1
    assert call(lib, batch=2**31) == 1
    assert call(lib, row_stride=1000, n_cols=1024) == 1
    assert call(lib, n_cols=-1) == 1
    assert call(lib, scores=None) == 1 and call(lib, out=None) == 1
    assert call(lib, scores=FAKE + 4) == 3
    assert call(lib, row_stride=1026, n_cols=1024) == 3
    assert call(lib, page_table=FAKE, page_size=0, pt_stride=64) == 1
    assert call(lib, page_table=FAKE, page_size=64, pt_stride=15) == 1
    assert call(lib, opt=Options(7, 0, None)) == 1
    assert call(lib, opt=Options(0, lib.topk_max_capacity() + 1, None)) == 1
    assert call(lib, opt=Options(0, -1, None)) == 1
    # kernel choice: values, and a capacity the short-row kernel cannot hold
    lib.topk_short_capacity.restype = ctypes.c_int32
    short_cap = lib.topk_short_capacity()
    assert 0 < short_cap < lib.topk_max_capacity()
    assert call(lib, opt=Options(0, 0, None, 3)) == 1 and call(lib, opt=Options(0, 0, None, -1)) == 1
    assert call(lib, opt=Options(0, short_cap + 1, None, 2)) == 1


def test_empty_batch_is_a_no_op(lib):
    assert call(lib, batch=0, scores=None, out=None) == 0
    assert call(lib, batch=0, scores=None, out=None, opt=Options(3, 5, None)) == 0


def test_status_strings(lib):
    for code in (0, 1, 2, 3, 4, 5, 99):
        assert lib.topk_status_string(code)
    assert lib.topk_max_capacity() >= 4096


WS = 0x100000  # 256-byte aligned, never dereferenced


def split_call(lib, scores=FAKE, batch=4, row_stride=1024, n_cols=1024, lengths=None, k=16,
               out=FAKE, page_table=None, pt_stride=0, page_size=0, ws=WS, ws_bytes=None,
               pieces=0, opt=None):
    if ws_bytes is None:
        ws_bytes = lib.topk_split_workspace_bytes(batch) if batch >= 0 else 0
    a = (scores, batch, row_stride, n_cols, lengths, k, out, page_table, pt_stride, page_size,
         ws, ws_bytes, pieces, None)
    return lib.topk_select_split(*a, ctypes.byref(opt) if opt is not None else None)


def test_split_workspace_size(lib):
    cap = lib.topk_split_capacity()
    assert cap >= lib.topk_max_capacity()
    assert lib.topk_split_workspace_bytes(0) == 0
    assert lib.topk_split_workspace_bytes(1) == 256 + 8 * cap
    assert lib.topk_split_workspace_bytes(40) == 768 + 40 * 8 * cap
    assert lib.topk_split_workspace_bytes(-1) == -1 and lib.topk_split_workspace_bytes(2**31) == -1


def test_split_host_argument_checks(lib):
    assert split_call(lib, k=0) == 2 and split_call(lib, k=2049) == 2
    assert split_call(lib, batch=-1) == 1 and split_call(lib, batch=2**31) == 1
    assert split_call(lib, row_stride=1000, n_cols=1024) == 1
    assert split_call(lib, scores=None) == 1 and split_call(lib, out=None) == 1
    assert split_call(lib, ws=None) == 1
    need = lib.topk_split_workspace_bytes(4)
    assert split_call(lib, ws_bytes=need - 1) == 1
    assert split_call(lib, ws=WS + 8) == 3
    assert split_call(lib, scores=FAKE + 4) == 3
    assert split_call(lib, row_stride=1026, n_cols=1024) == 3
    assert split_call(lib, pieces=-1) == 1 and split_call(lib, pieces=257) == 1
    assert split_call(lib, page_table=FAKE, page_size=0, pt_stride=64) == 1
    assert split_call(lib, opt=Options(4, 0, None)) == 1
    assert split_call(lib, opt=Options(0, lib.topk_split_capacity() + 1, None)) == 1
    assert split_call(lib, opt=Options(0, 0, None, 1)) == 1  # the split entry has its own kernels
    # a grid past 2^32 work-items
    assert split_call(lib, batch=2**24, n_cols=2**31 - 1, row_stride=2**31, ws_bytes=2**62,
                      pieces=256) == 1


def test_noalloc_split_host_argument_checks(lib):
    lib.topk_select_split_noalloc.argtypes = ARGS[:-1] + [ctypes.c_int32, ctypes.c_void_p,
                                                           ctypes.POINTER(Options)]
    na = lambda batch=4, k=16, scores=FAKE, opt=None: lib.topk_select_split_noalloc(
        scores, batch, 1024, 1024, None, k, FAKE, None, 0, 0, 0, None, ctypes.byref(opt) if opt else None)
    assert na(batch=257) == 1 and na(batch=-1) == 1  # TOPK_SPLIT_NOALLOC_MAX_BATCH rows at most
    assert na(batch=0, scores=None) == 0
    assert na(k=0) == 2 and na(k=2049) == 2


def test_split_empty_batch_is_a_no_op(lib):
    assert split_call(lib, batch=0, scores=None, out=None, ws=None, ws_bytes=0) == 0


def test_indexer_host_argument_checks(lib):
    lib.topk_select_bf16.argtypes = ARGS
    bf = lambda **kw: lib.topk_select_bf16(*{**dict(zip(
        ["s", "batch", "stride", "n_cols", "len", "k", "out", "pt", "pts", "ps", "st"],
        [FAKE, 4, 1024, 1024, None, 16, FAKE, None, 0, 0, None])), **kw}.values())
    assert bf(n_cols=16385, stride=16392) == 1 and bf(k=2049) == 2 and bf(k=0) == 2
    assert bf(s=FAKE + 2) == 3 and bf(stride=1028) == 3 and bf(out=None) == 1
    assert bf(batch=0, s=None, out=None) == 0
    assert bf(batch=2**24) == 1  # past one 256-thread workgroup per row

    lib.amax8_varlen.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                 ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64,
                                 ctypes.c_void_p]
    am = lambda s=FAKE, batch=4, stride=1024, n=1024, topk=0, out=FAKE, ostride=128: lib.amax8_varlen(
        s, batch, stride, n, None, topk, out, ostride, None)
    assert am(ostride=127) == 1 and am(topk=-1) == 1 and am(s=None) == 1
    assert am(s=FAKE + 16) == 3 and am(stride=1028, n=1020) == 3
    assert am(batch=0, s=None, out=None) == 0

    lib.sort_candidate_blocks.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                          ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                          ctypes.c_void_p, ctypes.c_void_p]
    sb = lambda blocks=FAKE, batch=4, k=64, n=8192, pt=FAKE, pts=128, ps=64, out=FAKE: \
        lib.sort_candidate_blocks(blocks, batch, k, None, n, pt, pts, ps, out, None)
    assert sb(ps=48) == 1 and sb(ps=4) == 1 and sb(pts=127) == 1 and sb(k=0) == 1
    assert sb(n=2**21 + 1, pts=2**20) == 1 and sb(pt=None) == 1 and sb(out=None) == 1
    assert sb(batch=0, blocks=None, pt=None, out=None) == 0


def test_binding_rejects_narrow_page_tables():
    # the binding checks page-table widths before taking any pointer, so CPU
    # tensors reach the check; a column slice keeps its row stride, so the C
    # side's stride check alone would accept it
    import torch

    import exact_row_top_fp32_amd as topk

    scores = torch.zeros((4, 1000))
    pt = torch.zeros((4, 40), dtype=torch.int32)[:, :15]  # 1000 scores span 16 pages of 64
    with pytest.raises(ValueError, match="page_table"):
        topk.topk_select(scores, None, 8, page_table=pt, page_size=64)
    blocks = torch.zeros((4, 8), dtype=torch.int32)
    with pytest.raises(ValueError, match="page_table"):  # 1000 positions: 125 blocks, 16 pages of 8
        topk.sort_candidate_blocks(blocks, None, pt, 64, n_cols=1000)


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="a GPU driver is present: the call would launch")
def test_valid_calls_without_a_device_return_device_error(lib):
    # every argument valid, but no gfx950 device is current: TOPK_ERR_DEVICE
    # before any launch (the pointers are never used)
    assert call(lib) == 4
    assert call(lib, opt=Options(2, 100, None, 1)) == 4
    assert call(lib, n_cols=40000, row_stride=40000) == 4
    assert split_call(lib) == 4
    lib.topk_select_split_noalloc.argtypes = ARGS[:-1] + [ctypes.c_int32, ctypes.c_void_p,
                                                           ctypes.POINTER(Options)]
    assert lib.topk_select_split_noalloc(FAKE, 4, 1024, 1024, None, 16, FAKE, None, 0, 0, 0, None, None) == 4
    lib.topk_select_bf16.argtypes = ARGS
    assert lib.topk_select_bf16(FAKE, 4, 1024, 1024, None, 16, FAKE, None, 0, 0, None) == 4
    lib.topk_select_bf16_ex.argtypes = ARGS + [ctypes.POINTER(Options)]
    assert lib.topk_select_bf16_ex(FAKE, 4, 1024, 1024, None, 16, FAKE, None, 0, 0, None,
                                   ctypes.byref(Options(1, 0, None, 1))) == 1  # no persistent bf16 kernel
    assert lib.topk_select_bf16_ex(FAKE, 4, 1024, 1024, None, 16, FAKE, None, 0, 0, None,
                                   ctypes.byref(Options(3, 0, None, 2))) == 4
