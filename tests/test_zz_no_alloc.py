"""GPU test of topk_select_split_noalloc: the split-row selection with its
workspace in the library's fixed device array instead of the caller's.

Called through the C ABI (ctypes, plain pointers) and checked index for index
against topk_select_split with a caller workspace, and against the oracle, on
two calls in a row, the second smaller than the first (the array then still
holds the first call's survivors and headers), with the output between guard
regions. Batches up to TOPK_SPLIT_NOALLOC_MAX_BATCH rows run; one more row is
an argument error, with nothing launched.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from topk_check import check

pytestmark = pytest.mark.gpu

GUARD = 4096
CANARY = 0x5A5A5A5A
MAX_BATCH = 256  # TOPK_SPLIT_NOALLOC_MAX_BATCH in include/exact_topk.h


class Options(ctypes.Structure):
    _fields_ = [("force_path", ctypes.c_int32), ("capacity", ctypes.c_int32),
                ("row_stats", ctypes.c_void_p), ("kernel", ctypes.c_int32)]


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_row_top_fp32_amd as topk_mod
    topk_mod._load()
    l = ctypes.CDLL(topk_mod.library_path)
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    l.topk_select_split_noalloc.argtypes = [p, i64, i64, i64, p, i32, p, p, i64, i32, i32, p,
                                            ctypes.POINTER(Options)]
    l.topk_select_split_noalloc.restype = ctypes.c_int
    l.topk_select_split.argtypes = [p, i64, i64, i64, p, i32, p, p, i64, i32, p, i64, i32, p,
                                    ctypes.POINTER(Options)]
    l.topk_select_split.restype = ctypes.c_int
    l.topk_split_workspace_bytes.argtypes = [i64]
    l.topk_split_workspace_bytes.restype = i64
    return l


def say(*msg):
    print(*msg, flush=True)


def run_both(lib, wl, pieces=0):
    """The no-alloc entry and the workspace entry on the same rows; returns
    both outputs (guards checked)."""
    B, k = wl.batch, wl.k
    s = torch.from_numpy(np.ascontiguousarray(wl.scores)).cuda()
    ln = torch.from_numpy(wl.lengths).cuda()
    pt = torch.from_numpy(wl.page_table).cuda() if wl.page_table is not None else None
    stream = torch.cuda.current_stream().cuda_stream
    stride = s.stride(0) if B > 1 else s.size(1)
    pt_ptr, pt_stride = (pt.data_ptr(), pt.stride(0) if B > 1 else pt.size(1)) if pt is not None else (None, 0)
    bufs = []
    for entry in ("noalloc", "workspace"):
        buf = torch.full((B * k + 2 * GUARD,), CANARY, dtype=torch.int32, device="cuda")
        out = buf[GUARD:GUARD + B * k]
        say(f"  gpu {entry} split call: {wl.name} B={B} k={k} pieces={pieces}")
        if entry == "noalloc":
            rc = lib.topk_select_split_noalloc(s.data_ptr(), B, stride, wl.n_cols, ln.data_ptr(), k,
                                               out.data_ptr(), pt_ptr, pt_stride, wl.page_size, pieces,
                                               stream, None)
        else:
            ws = torch.empty(lib.topk_split_workspace_bytes(B), dtype=torch.uint8, device="cuda")
            rc = lib.topk_select_split(s.data_ptr(), B, stride, wl.n_cols, ln.data_ptr(), k, out.data_ptr(),
                                       pt_ptr, pt_stride, wl.page_size, ws.data_ptr(), ws.numel(), pieces,
                                       stream, None)
        assert rc == 0, (entry, rc)
        bufs.append(buf)
    torch.cuda.synchronize()
    outs = []
    for buf in bufs:
        h = buf.cpu().numpy()
        assert np.all(h[:GUARD] == CANARY) and np.all(h[GUARD + B * k:] == CANARY), "write outside out"
        outs.append(h[GUARD:GUARD + B * k].reshape(B, k))
    return outs


def assert_same(wl, got, ref):
    assert np.array_equal(np.sort(got, 1), np.sort(ref, 1)), "differs from the workspace entry"
    want = oracle.topk(wl.scores, wl.lengths, wl.k, n_cols=wl.n_cols, page_table=wl.page_table,
                       page_size=wl.page_size)
    fails = check(wl.scores, wl.lengths, wl.n_cols, wl.k, got, want, page_table=wl.page_table,
                  page_size=wl.page_size)
    assert not fails, "\n".join(fails)


def test_noalloc_split_two_calls_second_smaller(lib):
    # first: the full array, 256 ragged rows of 65536 (k = 1024, paged, every
    # length category); then 40 rows of the 128K decode batch (k = 2048); then
    # 7 adversarial rows of 32768 (k = 512): each call smaller than the one
    # before, over what that call left in the array
    first = synth.c5(batch=MAX_BATCH)
    c3 = synth.c3(batch=40)
    second = synth.Workload("c3_first40", 3, c3.scores, c3.lengths, c3.n_cols, c3.k)
    third = synth.mixed_rows(["onebin", "crowd4096", "crowd16385", "above_fp16", "signed_zero", "constant",
                              "normal"], 32768, 512, seed=46, lengths=[32768, 32767, 30000, 513, 512, 0, 32768])
    for wl in (first, second, third):
        got, ref = run_both(lib, wl)
        assert_same(wl, got, ref)


def test_noalloc_split_piece_counts(lib):
    wl = synth.mixed_rows(["normal", "heavy_ties", "clustered_peaks"], 100000, 700, seed=47,
                          lengths=[100000, 99999, 65537])
    for pieces in (1, 5, 0):
        got, ref = run_both(lib, wl, pieces)
        assert_same(wl, got, ref)


def test_noalloc_split_rejects_more_rows_than_the_array_holds(lib):
    B, W, k = MAX_BATCH + 1, 1024, 16
    s = torch.zeros((B, W), dtype=torch.float32, device="cuda")
    out = torch.full((B, k), CANARY, dtype=torch.int32, device="cuda")
    rc = lib.topk_select_split_noalloc(s.data_ptr(), B, W, W, None, k, out.data_ptr(), None, 0, 0, 0,
                                       torch.cuda.current_stream().cuda_stream, None)
    torch.cuda.synchronize()
    assert rc == 1
    assert torch.all(out == CANARY), "nothing may be launched on an argument error"
