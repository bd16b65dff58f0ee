"""Captured launches: topk_select, topk_select_ex and topk_select_split in a
HIP graph, replayed with new lengths and scores written in place.

The vLLM PR #56346 report (implementation items 4-5) tests its top-k under
graph replay with a fixed capacity and lengths that change between replays;
the launches here take everything from device memory and allocate and clear
nothing, so one capture serves every replay. Each replay follows eager work
on the same buffers and a synchronisation, and is checked against the oracle
on the inputs of that replay.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from topk_check import check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def topk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_row_top_fp32_amd as topk_mod
    topk_mod._load()
    return topk_mod


def say(*msg):
    print(*msg, flush=True)


def expect(scores, lengths, n_cols, k):
    return oracle.topk(scores, lengths, k, n_cols=n_cols)


def parity(scores, lengths, n_cols, k, got, want):
    fails = check(scores, lengths, n_cols, k, got, want)
    assert not fails, "\n".join(fails)


LENGTH_SETS = [
    None,                                              # the capture's own lengths
    [0, 1, 511, 512, 513, 7168, 7169, 9000, 30000, 60000, 60000, 45000],
    [60000] * 12,
    [-1, 60017, 513, 100, 0, 59999, 20001, 8192, 8193, 16385, 3, 40000],
]


@pytest.mark.parametrize("entry", ["topk_select", "topk_select_short_rows", "topk_select_ex_small_capacity",
                                   "topk_select_split"])
def test_graph_replay_with_new_lengths_and_scores(topk, entry):
    k, W = 512, 60000
    kinds = ["normal", "clustered_peaks", "onebin", "neginf_half", "heavy_ties", "crowd4096",
             "normal", "signed_zero", "ascending", "normal", "above_fp16", "lowbits10"]
    wl = synth.mixed_rows(kinds, W, k, seed=51)
    B = wl.batch
    host = wl.scores.copy()
    s = torch.from_numpy(host).cuda()
    ln = torch.from_numpy(wl.lengths.copy()).cuda()
    out = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(topk.topk_split_workspace_bytes(B), dtype=torch.uint8, device="cuda")

    n_cols = 30000 if entry == "topk_select_short_rows" else W  # rows of at most 32768: the short-row kernel

    def call():
        if entry == "topk_select":
            topk.topk_select(s, ln, k, out)
        elif entry == "topk_select_short_rows":
            topk.topk_select(s[:, :n_cols], ln, k, out)
        elif entry == "topk_select_ex_small_capacity":
            topk.topk_select_ex(s, ln, k, out, capacity=700)  # every sampled row overflows
        else:
            topk.topk_select_split(s, ln, k, out, workspace=ws, capacity=700)

    say(f"  eager {entry}")
    call()
    torch.cuda.synchronize()
    parity(host, wl.lengths, n_cols, k, out.cpu().numpy(), expect(host, wl.lengths, n_cols, k))

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()  # warm-up on the capturing stream's side, as torch asks
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    say(f"  capture {entry}")
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()

    rng = np.random.default_rng(52)
    for rep in range(8):
        lens = LENGTH_SETS[rep % len(LENGTH_SETS)]
        lens = wl.lengths.copy() if lens is None else np.array(lens, np.int32)
        if rep >= 4:  # new scores as well: a sign flip of some rows, a shuffle of others
            flip = rng.random(B) < 0.5
            host[flip] = -host[flip]
            for b in np.flatnonzero(~flip)[:3]:
                host[b, :W] = rng.permutation(host[b, :W])
            s.copy_(torch.from_numpy(host))
        ln.copy_(torch.from_numpy(lens))
        out.fill_(-7)                      # eager work between replays
        torch.cuda.synchronize()
        say(f"  replay {rep} of {entry}")
        g.replay()
        torch.cuda.synchronize()
        parity(host, lens, n_cols, k, out.cpu().numpy(), expect(host, lens, n_cols, k))
    assert topk.topk_watchdog_trips() == 0
