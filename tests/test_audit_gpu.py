"""GPU audit of every kernel's exact boundaries, through the C ABI.

The pages trace their selection bugs to off-by-one limits: a threshold bin
holding exactly 4096 candidates ("Fix incorrect sparse-attention top-k
selection when candidate bins overflow", comment thread; the vLLM
persistent_topk issue, cause analysis), and they base the fix's correctness
on forcing every backend on chosen rows (vLLM PR #56346 report, discussion).
Here each limit is hit on each kernel that has it:

* survivor buffers: exactly at the capacity (the row stays on the sampled
  path) and one entry short of it (the overflow fallback), on the short-row
  kernel and the split-row entry (the persistent kernel's own case is in
  test_parity_gpu);
* the direct ranking of a cutoff bin (at most 64 entries ranked by one
  wave, more by radix passes): rows whose cutoff falls in a group of 63, 64
  or 65 equal scores, or of 63, 64 or 65 distinct scores closer together than
  any bin, through the persistent kernel's wave finisher, its whole-workgroup
  finish of a workgroup's last row, the short-row kernel and the split-row
  finisher;
* NaN inside a row's length, outside the contract: every kernel stays inside
  its buffers and every wait ends.

Every selection is checked against the oracle element by element, and the
row statistics name the path each row took.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from topk_check import check

pytestmark = pytest.mark.gpu

GUARD = 4096
CANARY = 0x5A5A5A5A


@pytest.fixture(scope="module")
def topk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_row_top_fp32_amd as topk_mod
    topk_mod._load()
    return topk_mod


def say(*msg):
    print(*msg, flush=True)


def guarded_out(B, k):
    buf = torch.full((B * k + 2 * GUARD,), CANARY, dtype=torch.int32, device="cuda")
    return buf, buf[GUARD:GUARD + B * k].view(B, k)


def unguard(buf, B, k):
    h = buf.cpu().numpy()
    assert np.all(h[:GUARD] == CANARY) and np.all(h[GUARD + B * k:] == CANARY), "write outside out"
    return h[GUARD:GUARD + B * k].reshape(B, k)


def select(topk, entry, wl, *, force=0, capacity=0, kernel=0, k=None):
    """One call of `entry` ("ex": topk_select_ex, "split": topk_select_split)
    with guarded output and row statistics; returns (out, stats)."""
    k = wl.k if k is None else k
    B = wl.batch
    s = torch.from_numpy(np.ascontiguousarray(wl.scores)).cuda()
    ln = torch.from_numpy(wl.lengths).cuda()
    buf, out = guarded_out(B, k)
    stats = torch.full((B, 2), -7, dtype=torch.int32, device="cuda")
    say(f"  gpu {entry} call: {wl.name} B={B} k={k} force={force} cap={capacity} kernel={kernel}")
    if entry == "ex":
        topk.topk_select_ex(s, ln, k, out, n_cols=wl.n_cols, force_path=force, capacity=capacity,
                            row_stats=stats, kernel=kernel)
    else:
        topk.topk_select_split(s, ln, k, out, n_cols=wl.n_cols, force_path=force, capacity=capacity,
                               row_stats=stats)
    torch.cuda.synchronize()
    assert topk.topk_watchdog_trips() == 0, "a workgroup gave up waiting"
    return unguard(buf, B, k), stats.cpu().numpy()


def assert_parity(wl, got, want=None, k=None):
    k = wl.k if k is None else k
    if want is None:
        want = oracle.topk(wl.scores, wl.lengths, k, n_cols=wl.n_cols)
    fails = check(wl.scores, wl.lengths, wl.n_cols, k, got, want)
    assert not fails, "\n".join(fails)


# ----------------------------------------------------------------------------
# survivors exactly at the capacity, and one over
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("entry", ["short_rows", "split"])
def test_survivors_at_the_capacity(topk, entry):
    # each sampled row is run again with the capacity set to its own survivor
    # count n (kept: code 3) and to n - 1 (one entry over: code 4, full row)
    wl = synth.mixed_rows(["normal", "crowd4096", "heavy_ties", "clustered_peaks"] * 2, 20000, 1024, seed=44)
    wl.lengths = np.array([20000, 19999, 20000, 17001, 12000, 20000, 9000, 20000], np.int32)
    synth.poison_tails(wl.scores, wl.lengths)
    name, kernel = ("ex", 2) if entry == "short_rows" else ("split", 0)
    limit = topk.topk_short_capacity() if entry == "short_rows" else topk.topk_split_capacity()
    _, stats = select(topk, name, wl, force=2, kernel=kernel)
    want = oracle.topk(wl.scores, wl.lengths, wl.k, n_cols=wl.n_cols)
    tried = 0
    for b in range(wl.batch):
        if stats[b, 0] != 3:
            continue
        n = int(stats[b, 1])
        row = synth.Workload(f"row{b}", 44, wl.scores[b:b + 1], wl.lengths[b:b + 1], wl.n_cols, wl.k)
        for cap, code in ((n, 3), (n - 1, 4)):
            if not 1 <= cap <= limit:
                continue
            got, st = select(topk, name, row, force=2, capacity=cap, kernel=kernel)
            assert st[0, 0] == code and (code != 3 or st[0, 1] == n), (b, n, cap, st[0])
            assert_parity(row, got, want[b:b + 1])
            tried += 1
    assert tried >= 8, f"only {tried} capacity cases ran"


# ----------------------------------------------------------------------------
# the cutoff bin's direct ranking limit (64 entries) in every finisher
# ----------------------------------------------------------------------------

FINISHERS = {
    # (entry, kernel, batch): 600 rows over at most 256 workgroups leave every
    # persistent workgroup two or three rows, all but its last finished by its
    # finisher wave; 4 rows give each workgroup one row, finished by all waves
    "persistent_wave": ("ex", 1, 600),
    "persistent_workgroup": ("ex", 1, 4),
    "short_rows": ("ex", 2, 8),
    "split": ("split", 0, 8),
}


@pytest.mark.parametrize("kind", ["ties", "cluster"])
@pytest.mark.parametrize("group", [63, 64, 65])
@pytest.mark.parametrize("finisher", list(FINISHERS))
def test_cutoff_group_at_the_direct_ranking_limit(topk, finisher, group, kind):
    entry, kernel, batch = FINISHERS[finisher]
    wl = synth.cutoff_group_rows(group, kind, batch=batch)
    got, stats = select(topk, entry, wl, force=2, kernel=kernel)
    assert np.all(stats[:, 0] == 3), f"every row selects among its survivors: {np.unique(stats[:, 0])}"
    assert_parity(wl, got)


# ----------------------------------------------------------------------------
# NaN inside a row's length: outside the contract, but memory-safe
# ----------------------------------------------------------------------------

def nan_rows(width, k, seed=45):
    rng = np.random.default_rng(seed)
    B = 6
    x = rng.standard_normal((B, width)).astype(np.float32)
    lengths = np.array([width, width - 3, width, width // 2, width, k + 1], np.int32)
    x[0, rng.permutation(width)[:width // 100]] = np.nan        # scattered NaN
    x[1, :] = np.nan                                             # all NaN
    x[2, rng.permutation(width)[:3 * k]] = np.nan                # more NaN than k
    x.view(np.uint32)[3, ::2] = 0xFFC00000                       # negative NaN patterns
    x[4, rng.permutation(width)[:k // 2]] = np.nan               # NaN among peaks
    x[4, rng.permutation(width)[:k // 2]] += 50.0
    x[5, :k + 1] = np.nan
    synth.poison_tails(x, lengths)
    return synth.Workload(f"nan_rows_{width}", seed, x, lengths, width, k)


def assert_safe_output(got, lengths, n_cols, k):
    """Outside the contract the choice is unspecified, but every slot holds -1
    exactly past m and a distinct in-range position before it."""
    L = np.clip(lengths, 0, n_cols)
    for b in range(got.shape[0]):
        m = min(k, int(L[b]))
        assert np.all(got[b, m:] == -1)
        head = got[b, :m]
        assert np.all((head >= 0) & (head < L[b])) and np.unique(head).size == m, b


@pytest.mark.parametrize("width", [16384, 131072])
def test_nan_inside_the_length_stays_memory_safe(topk, width):
    k = 512
    wl = nan_rows(width, k)
    runs = [("ex", 0, 0), ("ex", 1, 0), ("ex", 2, 0), ("ex", 1, 3), ("ex", 2, 3), ("split", 0, 0)]
    for entry, kernel, force in runs:
        got, stats = select(topk, entry, wl, force=force, kernel=kernel)
        assert_safe_output(got, wl.lengths, width, k)
    if width <= 16384:
        bits = synth.to_bf16_bits(wl.scores)
        s = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
        for force in (0, 1, 2, 3):
            buf, out = guarded_out(wl.batch, k)
            say(f"  gpu bf16 call: {wl.name} force={force}")
            topk.topk_select_bf16_ex(s, torch.from_numpy(wl.lengths).cuda(), k, out, force_path=force)
            torch.cuda.synchronize()
            assert_safe_output(unguard(buf, wl.batch, k), wl.lengths, width, k)
    assert topk.topk_watchdog_trips() == 0
