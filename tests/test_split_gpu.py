"""GPU parity of the split-row mode (topk_select_split) against the CPU oracle.

Each row is cut into pieces, one workgroup each; a third launch, one
workgroup per row, selects from the survivors every piece appended to the
row's area of the workspace (a full batch with the automatic piece count runs
one workgroup per row in a single launch instead). The result must be the oracle's, index for index, whatever the
number of pieces, the row's length (tails of 1-3 scores, pieces with nothing
to read), the path (sampled, keep-all, full-row, overflow), or what an
earlier call left in the workspace. Output and workspace sit between guard
regions that must come back untouched.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from topk_check import check, check_fast_raw

pytestmark = pytest.mark.gpu

GUARD = 4096
CANARY = 0x5A5A5A5A


@pytest.fixture(scope="session")
def topk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_row_top_fp32_amd as topk_mod
    topk_mod._load()
    return topk_mod


def say(*msg):
    print(*msg, flush=True)


_workspaces = {}


def guarded_workspace(topk, batch, fill):
    """A workspace between canaries, pre-filled with `fill` bytes (what an earlier call may leave)."""
    need = topk.topk_split_workspace_bytes(batch)
    pad = 256 * ((GUARD + 255) // 256)
    buf = torch.full((need + 2 * pad,), fill, dtype=torch.uint8, device="cuda")
    buf[:pad] = 0x5A
    buf[pad + need:] = 0x5A
    return buf, buf[pad:pad + need], pad, need


def run_split(topk, wl, *, k=None, force=0, capacity=0, pieces=0, lengths=None, scores_dev=None,
              n_cols=None, want_stats=False, fill=0xFF, workspace=None):
    k = wl.k if k is None else k
    B = wl.batch
    s = torch.from_numpy(np.ascontiguousarray(wl.scores)).cuda() if scores_dev is None else scores_dev
    ln = torch.from_numpy(np.ascontiguousarray(wl.lengths if lengths is None else lengths)).cuda()
    pt = torch.from_numpy(wl.page_table).cuda() if wl.page_table is not None else None
    out_buf = torch.full((B * k + 2 * GUARD,), CANARY, dtype=torch.int32, device="cuda")
    out = out_buf[GUARD:GUARD + B * k].view(B, k)
    stats = torch.full((B, 2), -7, dtype=torch.int32, device="cuda") if want_stats else None
    if workspace is None:
        ws_buf, ws, pad, need = guarded_workspace(topk, B, fill)
    else:
        ws_buf, ws, pad, need = workspace
    say(f"  gpu split call: {wl.name} B={B} k={k} force={force} cap={capacity} pieces={pieces}")
    topk.topk_select_split(s, ln, k, out, pt, wl.page_size, workspace=ws, pieces=pieces,
                           n_cols=n_cols or wl.n_cols, force_path=force, capacity=capacity,
                           row_stats=stats)
    torch.cuda.synchronize()
    h = out_buf.cpu().numpy()
    assert np.all(h[:GUARD] == CANARY) and np.all(h[GUARD + B * k:] == CANARY), "write outside out"
    w = ws_buf.cpu().numpy()
    assert np.all(w[:pad] == 0x5A) and np.all(w[pad + need:] == 0x5A), "write outside the workspace"
    return h[GUARD:GUARD + B * k].reshape(B, k), (stats.cpu().numpy() if want_stats else None)


def expect(wl, k=None, lengths=None, n_cols=None):
    return oracle.topk(wl.scores, wl.lengths if lengths is None else lengths,
                       wl.k if k is None else k, n_cols=n_cols or wl.n_cols,
                       page_table=wl.page_table, page_size=wl.page_size)


def assert_parity(wl, got, want, k=None, lengths=None, n_cols=None):
    fails = check(wl.scores, wl.lengths if lengths is None else lengths, n_cols or wl.n_cols,
                  wl.k if k is None else k, got, want, page_table=wl.page_table,
                  page_size=wl.page_size)
    assert not fails, "\n".join(fails)


PATHS = [0, 1, 2, 3]
PATH_IDS = ["auto", "keepall", "sampled", "fullrow"]


@pytest.mark.parametrize("force", PATHS, ids=PATH_IDS)
def test_split_c1(topk, force):
    wl = synth.c1()
    for pieces in (0, 1):
        got, _ = run_split(topk, wl, force=force, pieces=pieces)
        assert_parity(wl, got, expect(wl))


@pytest.mark.parametrize("k", [512, 1024, 2048])
@pytest.mark.parametrize("force", PATHS, ids=PATH_IDS)
def test_split_c2_adversarial(topk, k, force):
    wl = synth.c2(k)
    want = expect(wl)
    for pieces in (0, 1, 3):  # 32768-wide rows: at most 4 pieces of 8192 scores
        got, stats = run_split(topk, wl, force=force, pieces=pieces, want_stats=True)
        assert_parity(wl, got, want)
        if force == 0 and pieces == 0:
            say("  row paths:", dict(zip(*np.unique(stats[:, 0], return_counts=True))))


def test_split_c2_small_capacity_overflows(topk):
    wl = synth.c2(1024)
    got, stats = run_split(topk, wl, force=2, capacity=300, want_stats=True)
    assert_parity(wl, got, expect(wl))
    assert np.all(stats[:, 0] >= 4)


@pytest.mark.parametrize("batch", [1, 7, 40, 128])
def test_split_small_batches_of_the_decode_rows(topk, c3, c4, batch):
    for big in (c3, c4):
        sub = synth.Workload(f"{big.name}_first{batch}", big.seed, big.scores[:batch],
                             big.lengths[:batch], big.n_cols, big.k)
        want = expect(sub)
        for pieces in (0, 5, 256):
            got, stats = run_split(topk, sub, pieces=pieces, want_stats=True)
            assert not check_fast_raw(got, want, sub.lengths, sub.n_cols, sub.k)
            assert np.all(stats[:, 0] == 3), "decode rows take the sampled path"


def test_split_full_decode_batches(topk, c3, c4):
    # one piece per row through the split kernels; then the automatic piece
    # count, which on batches of four rows per compute unit runs one
    # workgroup per row in one launch and leaves the workspace untouched
    for wl in (c3, c4):
        want = expect(wl)
        got, stats = run_split(topk, wl, pieces=1, want_stats=True)
        bad = check_fast_raw(got, want, wl.lengths, wl.n_cols, wl.k)
        assert not bad, f"rows differing from the oracle: {bad[:10]}"
        say(f"  {wl.name} split paths:", dict(zip(*np.unique(stats[:, 0], return_counts=True))),
            "survivors mean/max:", stats[:, 1].mean(), stats[:, 1].max())
        ws = guarded_workspace(topk, wl.batch, 0xA7)
        got, _ = run_split(topk, wl, pieces=0, workspace=ws)
        bad = check_fast_raw(got, want, wl.lengths, wl.n_cols, wl.k)
        assert not bad, f"rows differing from the oracle: {bad[:10]}"
        if wl.batch >= 4 * torch.cuda.get_device_properties(0).multi_processor_count:
            assert bool((ws[1] == 0xA7).all()), "the one-workgroup-per-row launch wrote to the workspace"


@pytest.mark.parametrize("global_pool", [False, True], ids=["row_perm", "global_pool"])
def test_split_c5_paged(topk, global_pool):
    wl = synth.c5(global_pool=global_pool)
    for force in PATHS:
        got, _ = run_split(topk, wl, force=force)
        assert_parity(wl, got, expect(wl))


def test_split_length_boundaries_and_tails(topk):
    # lengths around k, the capacity and piece edges (8192 scores per round),
    # with 1-3 scores past the last full group
    k, W = 512, 40000
    cap = topk.topk_split_capacity()
    lens = [-1, 0, 1, k - 1, k, k + 1, k + 3, cap - 1, cap, cap + 1, cap + 2, 8192 * 2 + 1,
            8192 * 3 - 1, 8192 * 4 + 3, W - 1, W, W + 17]
    wl = synth.mixed_rows(["normal", "ascending", "heavy_ties"] * 6, W, k, seed=41)
    wl.scores, wl.lengths = wl.scores[:len(lens)], np.array(lens, np.int32)
    synth.poison_tails(wl.scores, np.clip(wl.lengths, 0, W))
    want = expect(wl)
    for force in PATHS:
        for pieces in (0, 1, 2, 5):
            got, _ = run_split(topk, wl, force=force, pieces=pieces)
            assert_parity(wl, got, want)


def test_split_width_not_a_multiple_of_four(topk):
    # a single row (no stride constraint): widths 1-3 past a group, every piece count
    rng = np.random.default_rng(42)
    for W in (9001, 16386, 24579):
        scores = rng.standard_normal((1, W)).astype(np.float32)
        scores[0, -1] = 50.0  # the very last score must be found
        wl = synth.Workload(f"w{W}", 42, scores, np.array([W], np.int32), W, 300)
        for pieces in (0, 1, 2, 3):
            got, _ = run_split(topk, wl, pieces=pieces)
            assert_parity(wl, got, expect(wl))


@pytest.mark.parametrize("k", [1, 2, 64, 2047, 2048])
def test_split_k_range(topk, k):
    wl = synth.mixed_rows(["normal", "heavy_ties", "constant", "signed_zero", "onebin"], 30000, k,
                          seed=43)
    for force in PATHS:
        got, _ = run_split(topk, wl, k=k, force=force)
        assert_parity(wl, got, expect(wl, k=k), k=k)


@pytest.mark.parametrize("width", [131072, 262144])
def test_split_long_adversarial_rows(topk, width):
    kinds = ["onebin", "crowd16385", "crowd16385_top", "above_fp16", "neginf_few_finite",
             "signed_zero", "constant", "clustered_peaks", "periodic_peaks", "lowbits10"]
    for k in (512, 2048):
        wl = synth.mixed_rows(kinds, width, k, seed=44)
        want = expect(wl)
        for force in (0, 3):
            got, _ = run_split(topk, wl, force=force)
            assert_parity(wl, got, want)


def test_split_matches_topk_select_and_reuses_a_workspace(topk, c4):
    # one workspace, calls with different batches and lengths, no clearing in
    # between: every result equals topk_select's
    ws = guarded_workspace(topk, 64, 0x00)
    s = torch.from_numpy(np.ascontiguousarray(c4.scores[:64])).cuda()
    for B, lens in ((64, c4.lengths[:64]), (17, c4.lengths[:17] // 3), (64, c4.lengths[:64] // 7)):
        sub = synth.Workload("c4_sub", 4, c4.scores[:B], lens.astype(np.int32), c4.n_cols, c4.k)
        got, _ = run_split(topk, sub, scores_dev=s[:B], workspace=ws)
        ref = topk.topk_select(s[:B], torch.from_numpy(sub.lengths).cuda(), sub.k)
        torch.cuda.synchronize()
        assert np.array_equal(np.sort(got, 1), np.sort(ref.cpu().numpy(), 1))
        assert not check_fast_raw(got, expect(sub), sub.lengths, sub.n_cols, sub.k)
