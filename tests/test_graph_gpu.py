"""Captured launches: topk_select, topk_select_ex and topk_select_split in a
HIP graph, and the two-level indexer's chain (amax8_varlen, topk_select over
the block keys, sort_candidate_blocks) with topk_select_bf16, replayed with
new lengths and scores written in place.

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


def test_graph_replay_of_the_indexer_chain_and_bf16_topk(topk):
    # the two-level indexer's three calls (block max, top-k over the block
    # keys, block table) and a bf16 top-k captured in one graph, replayed
    # with new lengths and scores; every output checked against the oracle
    B, W, k, ps, Wb, kb = 64, 32768, 256, 64, 16384, 512
    nblk = W // 8
    rng = np.random.default_rng(53)
    x = rng.standard_normal((B, W)).astype(np.float32)
    lens = rng.integers(W // 2, W + 1, B).astype(np.int32)
    lens[:6] = [0, 1, 7, 8 * k, 8 * k + 1, W]
    pt_h = np.stack([rng.permutation(nblk // (ps // 8)) for _ in range(B)]).astype(np.int32)
    s = torch.from_numpy(x).cuda()
    ln = torch.from_numpy(lens).cuda()
    pt = torch.from_numpy(pt_h).cuda()
    nb = torch.empty(B, dtype=torch.int32, device="cuda")
    keys = torch.empty((B, nblk), dtype=torch.float32, device="cuda")
    blocks = torch.empty((B, k), dtype=torch.int32, device="cuda")
    pages = torch.empty((B, k), dtype=torch.int32, device="cuda")
    bits = synth.to_bf16_bits(x[:, :Wb])
    lens_b = np.minimum(lens, Wb).astype(np.int32)
    sb = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    lnb = torch.from_numpy(lens_b).cuda()
    out_b = torch.empty((B, kb), dtype=torch.int32, device="cuda")

    def call():
        topk.amax8_varlen(s, ln, k, out=keys)
        torch.div(ln.clamp(min=0) + 7, 8, rounding_mode="floor", out=nb)
        topk.topk_select(keys, nb, k, blocks)
        topk.sort_candidate_blocks(blocks, ln, pt, ps, out_pages=pages, n_cols=W)
        topk.topk_select_bf16(sb, lnb, kb, out_b)

    def verify(x, lens, bits, lens_b):
        want_keys = np.full((B, nblk), 7.0, np.float32)
        oracle.amax8(x, lens, k, want_keys)
        assert np.array_equal(keys.cpu().numpy().view(np.uint32), want_keys.view(np.uint32))
        nb_h = ((np.maximum(lens, 0).astype(np.int64) + 7) // 8).astype(np.int32)
        table, slots = oracle.sort_candidate_blocks(oracle.topk(want_keys, nb_h, k), lens, pt_h, ps, n_cols=W)
        assert np.array_equal(blocks.cpu().numpy(), table)
        assert np.array_equal(pages.cpu().numpy(), slots)
        want_b = oracle.topk_bf16(bits, lens_b, kb)
        fails = check(oracle.bf16_to_f32(bits), lens_b, Wb, kb, out_b.cpu().numpy(), want_b)
        assert not fails, "\n".join(fails)

    keys.fill_(7.0)
    say("  eager indexer chain")
    call()
    torch.cuda.synchronize()
    verify(x, lens, bits, lens_b)

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    say("  capture indexer chain")
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()

    for rep in range(4):
        lens = rng.integers(0, W + 1, B).astype(np.int32)
        lens[rep] = 8 * k  # a row with exactly k blocks: the identity table
        if rep >= 2:
            x = -x
            x[rep + 10] = rng.permutation(x[rep + 10])
        bits = synth.to_bf16_bits(x[:, :Wb])
        lens_b = np.minimum(lens, Wb).astype(np.int32)
        s.copy_(torch.from_numpy(x))
        ln.copy_(torch.from_numpy(lens))
        sb.copy_(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16))
        lnb.copy_(torch.from_numpy(lens_b))
        keys.fill_(7.0)                    # eager work between replays
        torch.cuda.synchronize()
        say(f"  replay {rep} of the indexer chain")
        g.replay()
        torch.cuda.synchronize()
        verify(x, lens, bits, lens_b)
