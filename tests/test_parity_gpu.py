"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every case compares the GPU's output with the oracle's on the same seeded
inputs: -1 slots, index range and uniqueness, the selected-value multiset bit
for bit, and the selected index set itself (both sides take the lowest indices
among ties at the cutoff, so the set is unique). Outputs sit between guard
regions that must come back untouched, and positions past each row's length
hold NaN, which would rank first if any kernel read it.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from topk_check import check, check_codes, check_fast_raw

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


_dev_cache = {}


def to_dev(a):
    key = id(a)
    if key not in _dev_cache:
        _dev_cache[key] = (a, torch.from_numpy(np.ascontiguousarray(a)).cuda())
    return _dev_cache[key][1]


def say(*msg):
    print(*msg, flush=True)


def run(topk, wl, *, k=None, force=0, capacity=0, lengths=None, scores_dev=None,
        n_cols=None, want_stats=False, kernel=0):
    """Launch through the C ABI with guarded output; returns (out, stats)."""
    k = wl.k if k is None else k
    B = wl.batch
    s = to_dev(wl.scores) if scores_dev is None else scores_dev
    ln = to_dev(wl.lengths if lengths is None else lengths)
    pt = to_dev(wl.page_table) if wl.page_table is not None else None
    buf = torch.full((B * k + 2 * GUARD,), CANARY, dtype=torch.int32, device="cuda")
    out = buf[GUARD:GUARD + B * k].view(B, k)
    stats = torch.full((B, 2), -7, dtype=torch.int32, device="cuda") if want_stats else None
    say(f"  gpu call: {wl.name} k={k} force={force} cap={capacity} kernel={kernel}")
    topk.topk_select_ex(s, ln, k, out, pt, wl.page_size, n_cols=n_cols or wl.n_cols,
                        force_path=force, capacity=capacity, row_stats=stats, kernel=kernel)
    torch.cuda.synchronize()
    assert topk.topk_watchdog_trips() == 0, "a workgroup gave up waiting"
    h = buf.cpu().numpy()
    assert np.all(h[:GUARD] == CANARY) and np.all(h[GUARD + B * k:] == CANARY), "write outside out"
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
PATH_IDS = ["auto", "lds", "sampled", "fullrow"]
# topk_options.kernel: the automatic choice (the short-row kernel for widths
# up to 32768), and the persistent kernel forced
KERNELS = [0, 1]
KERNEL_IDS = ["auto_kernel", "persistent"]


def kernel_capacity(topk, kernel, n_cols, capacity=0):
    """The survivor capacity the chosen kernel runs with."""
    if capacity:
        return capacity
    short = kernel == 2 or (kernel == 0 and n_cols <= 32768)
    return topk.topk_short_capacity() if short else topk.topk_max_capacity()


def assert_codes(stats, lengths, n_cols, k, force, cap):
    fails = check_codes(stats, lengths, n_cols, k, force, cap)
    assert not fails, "\n".join(fails[:10])


# ----------------------------------------------------------------------------
# the five workloads
# ----------------------------------------------------------------------------

@pytest.fixture(scope="session")
def c1():
    return synth.c1()


@pytest.mark.parametrize("kernel", KERNELS, ids=KERNEL_IDS)
@pytest.mark.parametrize("force", PATHS, ids=PATH_IDS)
def test_c1_every_path(topk, c1, force, kernel):
    got, stats = run(topk, c1, force=force, want_stats=True, kernel=kernel)
    assert_parity(c1, got, expect(c1))
    assert_codes(stats, c1.lengths, c1.n_cols, c1.k, force, kernel_capacity(topk, kernel, c1.n_cols))


@pytest.fixture(scope="session", params=[512, 1024, 2048])
def c2(request):
    return synth.c2(request.param)


@pytest.mark.parametrize("kernel", KERNELS, ids=KERNEL_IDS)
@pytest.mark.parametrize("force", PATHS, ids=PATH_IDS)
def test_c2_adversarial_every_path(topk, c2, force, kernel):
    got, stats = run(topk, c2, force=force, want_stats=True, kernel=kernel)
    want = expect(c2)
    assert_parity(c2, got, want)
    assert_codes(stats, c2.lengths, c2.n_cols, c2.k, force, kernel_capacity(topk, kernel, c2.n_cols))
    say("  row paths:", dict(zip(*np.unique(stats[:, 0], return_counts=True))))


@pytest.mark.parametrize("kernel", KERNELS, ids=KERNEL_IDS)
def test_c2_small_capacity_forces_overflow(topk, c2, kernel):
    got, stats = run(topk, c2, force=2, capacity=300, want_stats=True, kernel=kernel)
    assert_parity(c2, got, expect(c2))
    assert np.all(stats[:, 0] >= 4), "every row must fall back when m exceeds the capacity"


def test_c3_decode_batch_all_rows(topk, c3):
    got, stats = run(topk, c3, want_stats=True)
    want = expect(c3)
    bad = check_fast_raw(got, want, c3.lengths, c3.n_cols, c3.k)
    assert not bad, f"rows differing from the oracle: {bad[:10]}"
    assert_parity(c3, got, want)
    paths = dict(zip(*np.unique(stats[:, 0], return_counts=True)))
    say("  c3 row paths:", paths, "survivors min/mean/max:",
        stats[:, 1].min(), stats[:, 1].mean(), stats[:, 1].max())


def test_c4_decode_batch_all_rows(topk, c4):
    got, stats = run(topk, c4, want_stats=True)
    want = expect(c4)
    bad = check_fast_raw(got, want, c4.lengths, c4.n_cols, c4.k)
    assert not bad, f"rows differing from the oracle: {bad[:10]}"
    paths = dict(zip(*np.unique(stats[:, 0], return_counts=True)))
    say("  c4 row paths:", paths, "survivors min/mean/max:",
        stats[:, 1].min(), stats[:, 1].mean(), stats[:, 1].max())


@pytest.mark.parametrize("force", [1, 3], ids=["lds-forced", "fullrow"])
def test_c3_rows_forced_paths(topk, c3, force):
    # 64 rows of the decode batch through the fallback paths
    sub = synth.Workload("c3_first64", 3, c3.scores[:64], c3.lengths[:64], c3.n_cols, c3.k)
    got, _ = run(topk, sub, force=force)
    assert not check_fast_raw(got, expect(sub), sub.lengths, sub.n_cols, sub.k)


@pytest.mark.parametrize("kernel", [0, 2], ids=["auto_kernel", "short_rows"])
@pytest.mark.parametrize("global_pool", [False, True], ids=["row_perm", "global_pool"])
@pytest.mark.parametrize("force", PATHS, ids=PATH_IDS)
def test_c5_paged(topk, force, global_pool, kernel):
    wl = synth.c5(global_pool=global_pool)
    got, stats = run(topk, wl, force=force, want_stats=True, kernel=kernel)
    assert_parity(wl, got, expect(wl))
    assert_codes(stats, wl.lengths, wl.n_cols, wl.k, force, kernel_capacity(topk, kernel, wl.n_cols))


# ----------------------------------------------------------------------------
# boundaries and edge cases
# ----------------------------------------------------------------------------

def test_length_boundaries(topk):
    k, W = 512, 20000
    cap = topk.topk_max_capacity()
    lens = [-1, -100, 0, 1, k - 1, k, k + 1, cap - 1, cap, cap + 1, 2 * cap, W - 1, W, W + 17]
    wl = synth.mixed_rows(["normal"] * len(lens), W, k, seed=21)
    wl.lengths = np.array(lens, np.int32)
    synth.poison_tails(wl.scores, np.clip(wl.lengths, 0, W))
    for kernel in (0, 1):
        for force in PATHS:
            got, stats = run(topk, wl, force=force, want_stats=True, kernel=kernel)
            assert_parity(wl, got, expect(wl))
            assert_codes(stats, wl.lengths, W, k, force, kernel_capacity(topk, kernel, W))


@pytest.mark.parametrize("k", [1, 2, 63, 64, 65, 2047, 2048])
def test_k_range(topk, k):
    wl = synth.mixed_rows(["normal", "heavy_ties", "constant", "signed_zero", "ascending"], 9000, k, seed=22)
    wl.lengths = np.array([9000, 9000, 2048, 2049, 5000], np.int32)
    synth.poison_tails(wl.scores, wl.lengths)
    for kernel in (0, 1):
        for force in PATHS:
            got, stats = run(topk, wl, k=k, force=force, want_stats=True, kernel=kernel)
            assert_parity(wl, got, expect(wl, k=k), k=k)
            assert_codes(stats, wl.lengths, wl.n_cols, k, force, kernel_capacity(topk, kernel, wl.n_cols))


def test_offset_view_and_stride(topk):
    rng = np.random.default_rng(23)
    base = rng.standard_normal((10, 12000)).astype(np.float32)
    dev = torch.from_numpy(base).cuda()
    view = dev[2:8, 16:11016]   # base offset of 16 floats, row stride 12000 > n_cols 11000
    host = base[2:8, 16:11016]
    lengths = np.array([11000, 10000, 500, 0, 9001, 11000], np.int32)
    wl = synth.Workload("offset_view", 23, host, lengths, 11000, 700)
    for force in PATHS:
        got, _ = run(topk, wl, force=force, scores_dev=view)
        assert_parity(wl, got, expect(wl))


def test_lengths_null_means_full_rows(topk):
    wl = synth.mixed_rows(["normal", "lowbits10", "onebin"], 10000, 300, seed=24)
    s = to_dev(wl.scores)
    out = topk.topk_select(s, None, 300)
    torch.cuda.synchronize()
    assert_parity(wl, out.cpu().numpy(), expect(wl))


def test_exact_capacity_boundary(topk):
    # survivors exactly at the capacity are kept; one fewer slot forces the fallback
    wl = synth.mixed_rows(["normal"] * 8 + ["crowd4096"] * 8, 60000, 1024, seed=25)
    _, stats = run(topk, wl, force=2, want_stats=True)
    want = expect(wl)
    for b in range(wl.batch):
        if stats[b, 0] != 3:
            continue
        n = int(stats[b, 1])
        row = synth.Workload("row", 25, wl.scores[b:b + 1], wl.lengths[b:b + 1], wl.n_cols, wl.k)
        for cap, ok_code in ((n, 3), (n - 1, 4)):
            if not 1 <= cap <= topk.topk_max_capacity():
                continue
            got, st = run(topk, row, force=2, capacity=cap, want_stats=True)
            assert st[0, 0] == ok_code, (b, n, cap, st[0])
            assert_parity(row, got, want[b:b + 1])


@pytest.mark.parametrize("kernel", [1, 2], ids=["persistent", "short_rows"])
def test_lds_capacity_boundary(topk, kernel):
    cap = 3000
    wl = synth.mixed_rows(["normal", "heavy_ties", "normal", "heavy_ties"], 4000, 256, seed=26)
    wl.lengths = np.array([cap, cap, cap + 1, cap + 1], np.int32)
    synth.poison_tails(wl.scores, wl.lengths)
    got, stats = run(topk, wl, capacity=cap, want_stats=True, kernel=kernel)
    assert list(stats[:, 0]) == [2, 2, stats[2, 0], stats[3, 0]] and stats[2, 0] >= 3
    assert_parity(wl, got, expect(wl))


def test_repeated_calls_same_set_and_changed_inputs(topk):
    # the same device buffers reused with new lengths and flipped scores
    k = 512
    wl = synth.mixed_rows(["normal", "clustered_peaks", "onebin", "neginf_half"] * 2, 40000, k, seed=27)
    s = to_dev(wl.scores).clone()
    first, _ = run(topk, wl, scores_dev=s)
    again, _ = run(topk, wl, scores_dev=s)
    assert np.array_equal(np.sort(first, 1), np.sort(again, 1))
    for lens in ([-1, 0, 1, k - 1, k, 32769, 40000, 40017], [40000] * 8, [k + 1] * 8):
        lens = np.array(lens, np.int32)
        got, _ = run(topk, wl, scores_dev=s, lengths=lens)
        assert_parity(wl, got, expect(wl, lengths=lens), lengths=lens)
    flipped = -wl.scores
    s.copy_(torch.from_numpy(flipped))
    fw = synth.Workload("flipped", 27, flipped, wl.lengths, wl.n_cols, k)
    got, _ = run(topk, fw, scores_dev=s)
    assert_parity(fw, got, expect(fw))


@pytest.mark.parametrize("width", [131072, 262144])
@pytest.mark.parametrize("k", [512, 2048])
def test_long_adversarial_rows(topk, width, k):
    kinds = ["onebin", "crowd16385", "crowd16385_top", "above_fp16", "neginf_few_finite",
             "signed_zero", "constant", "clustered_peaks", "periodic_peaks", "lowbits10"]
    wl = synth.mixed_rows(kinds, width, k, seed=28)
    for force in (0, 3):
        got, _ = run(topk, wl, force=force)
        assert_parity(wl, got, expect(wl))


def test_plain_c_entry(topk):
    # topk_select through the C ABI directly, three calls on one stream
    wl = synth.mixed_rows(["normal", "onebin", "crowd4096", "signed_zero"], 50000, 777, seed=29)
    s = to_dev(wl.scores)
    ln = to_dev(wl.lengths)
    out = torch.full((wl.batch, wl.k), CANARY, dtype=torch.int32, device="cuda")
    lib = topk._load()
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(3):
        rc = lib.topk_select(s.data_ptr(), wl.batch, s.stride(0), wl.n_cols, ln.data_ptr(), wl.k,
                             out.data_ptr(), None, 0, 0, stream)
        assert rc == 0
    torch.cuda.synchronize()
    assert_parity(wl, out.cpu().numpy(), expect(wl))


def test_deferred_list_overflow(topk):
    # more rows forced to the full-row path than one workgroup can defer
    rng = np.random.default_rng(30)
    B, W, k = 256 * 80, 640, 9
    scores = rng.standard_normal((B, W)).astype(np.float32)
    lengths = rng.integers(k + 1, W + 1, B).astype(np.int32)
    synth.poison_tails(scores, lengths)
    wl = synth.Workload("many_fullrow", 30, scores, lengths, W, k)
    got, stats = run(topk, wl, force=3, want_stats=True)
    assert np.all(stats[:, 0] == 6)
    bad = check_fast_raw(got, expect(wl), wl.lengths, wl.n_cols, wl.k)
    assert not bad, bad[:10]


# ----------------------------------------------------------------------------
# sign of the cutoff, batches past the longest-first table, tiny batches
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("k", [512, 2048])
def test_negative_and_straddling_cutoffs(topk, k):
    # Rows shifted so the cutoff key falls below +0 (all-negative rows) or
    # right at it (about k positive scores per row): both filters then take
    # the signed compare rather than the non-negative one.
    rng = np.random.default_rng(31)
    B, W = 24, 131072
    shift = np.empty((B, 1), np.float32)
    shift[:8] = 10.0          # every score negative
    shift[8:16] = 2.15        # about 1.6 % positive: cutoff near zero for k = 2048
    shift[16:] = 2.88         # about 0.2 % positive: cutoff near zero for k = 512
    scores = (rng.standard_normal((B, W)).astype(np.float32) - shift).astype(np.float32)
    lengths = synth.ragged_lengths(rng, B, W)
    synth.poison_tails(scores, lengths)
    wl = synth.Workload("negative_cutoffs", 31, scores, lengths, W, k)
    want = expect(wl)
    for force in (0, 2):
        got, stats = run(topk, wl, force=force, want_stats=True)
        assert_parity(wl, got, want)
        say("  row paths:", dict(zip(*np.unique(stats[:, 0], return_counts=True))))
        assert np.all(stats[:8, 0] == 3), stats[:8]


@pytest.mark.parametrize("k", [512, 2048])
def test_short_rows_straddling_cutoffs(topk, k):
    # Short rows shifted so the cutoff falls below +0 (every score negative)
    # or near it (k = 2048: about 12.5 % positive at shift 1.15; k = 512:
    # about 3 % at 1.86): the sample's keys then straddle the sign, the
    # cutoff's first histogram is coarse and a second pass narrows it. Every
    # row must still take the sampled path (no overflow into the full row).
    rng = np.random.default_rng(33)
    B, W = 24, 16384
    shift = np.empty((B, 1), np.float32)
    shift[:8] = 10.0
    shift[8:16] = 1.15
    shift[16:] = 1.86
    scores = (rng.standard_normal((B, W)).astype(np.float32) - shift).astype(np.float32)
    lengths = synth.ragged_lengths(rng, B, W)
    synth.poison_tails(scores, lengths)
    wl = synth.Workload("short_negative_cutoffs", 33, scores, lengths, W, k)
    got, stats = run(topk, wl, want_stats=True)
    assert_parity(wl, got, expect(wl))
    say("  row paths:", dict(zip(*np.unique(stats[:, 0], return_counts=True))))
    assert np.all(stats[:, 0] == 3), stats[:, 0]


def test_batch_above_longest_first_table(topk):
    # 3000 rows of 8192 (above the LDS capacity): rows are claimed in batch
    # order once the batch no longer fits the longest-first table.
    rng = np.random.default_rng(32)
    B, W, k = 3000, 8192, 256
    scores = rng.standard_normal((B, W)).astype(np.float32)
    lengths = rng.integers(0, W + 1, B).astype(np.int32)
    lengths[::7] = W
    synth.poison_tails(scores, lengths)
    wl = synth.Workload("unordered_batch", 32, scores, lengths, W, k)
    want = expect(wl)
    for force in (0, 2):
        got, stats = run(topk, wl, force=force, want_stats=True)
        bad = check_fast_raw(got, want, wl.lengths, wl.n_cols, wl.k)
        assert not bad, f"rows differing from the oracle: {bad[:10]}"
        say("  row paths:", dict(zip(*np.unique(stats[:, 0], return_counts=True))))
    assert_parity(wl, got, want)


@pytest.mark.parametrize("batch", [1, 3, 255])
def test_batches_below_the_cu_count(topk, batch):
    # fewer rows than workgroups: most workgroups find no row to claim
    rng = np.random.default_rng(33 + batch)
    W, k = 262144, 2048
    scores = rng.standard_normal((batch, W)).astype(np.float32)
    lengths = synth.ragged_lengths(rng, batch, W)
    synth.poison_tails(scores, lengths)
    wl = synth.Workload(f"batch{batch}", 33, scores, lengths, W, k)
    want = expect(wl)
    for force in (0, 3):
        got, stats = run(topk, wl, force=force, want_stats=True)
        assert_parity(wl, got, want)
        if force == 0:
            assert np.all(stats[:, 0] == 3), stats


@pytest.mark.parametrize("layout", ["one_length", "two_lengths_and_ragged"])
def test_rows_sharing_a_length_bucket(topk, layout):
    # many rows of one length fall into one bucket of the longest-first sort,
    # whose index order then comes from a workgroup-wide scan
    rng = np.random.default_rng(34)
    B, W, k = 700, 9000, 300
    scores = rng.standard_normal((B, W)).astype(np.float32)
    if layout == "one_length":
        lengths = np.full(B, W, np.int32)
    else:
        lengths = rng.integers(k + 1, W + 1, B).astype(np.int32)
        lengths[rng.permutation(B)[:250]] = W
        lengths[rng.permutation(B)[:200]] = W // 2
    synth.poison_tails(scores, lengths)
    wl = synth.Workload(f"bucket_{layout}", 34, scores, lengths, W, k)
    want = expect(wl)
    for force in (0, 2):
        got, stats = run(topk, wl, force=force, want_stats=True)
        bad = check_fast_raw(got, want, wl.lengths, wl.n_cols, wl.k)
        assert not bad, f"rows differing from the oracle: {bad[:10]}"
    assert_parity(wl, got, want)


# ----------------------------------------------------------------------------
# short rows on the automatic path (n_cols <= 32768): one workgroup per row
# ----------------------------------------------------------------------------

SHORT_MAX_COLS = 32768
SHORT_CAP = 3840  # survivors the short-row kernel holds in LDS


@pytest.mark.parametrize("k", [512, 2048])
def test_short_rows_buffer_boundaries(topk, k):
    W = 20000
    lens = [SHORT_CAP - 1, SHORT_CAP, SHORT_CAP + 1, SHORT_CAP + 3, k + 1, 2 * SHORT_CAP, W - 3, W]
    wl = synth.mixed_rows(["normal", "heavy_ties", "ascending", "signed_zero"] * 2, W, k, seed=35)
    wl.lengths = np.array(lens, np.int32)
    synth.poison_tails(wl.scores, wl.lengths)
    got, stats = run(topk, wl, want_stats=True)
    assert_parity(wl, got, expect(wl))
    codes = stats[:, 0].tolist()
    assert codes[0] == 2 and codes[1] == 2, "rows up to the buffer keep every score"
    assert all(c in (3, 4, 5) for c in codes[2:4]) and codes[4] == (2 if k + 1 <= SHORT_CAP else 3)


@pytest.mark.parametrize("W", [SHORT_MAX_COLS, SHORT_MAX_COLS + 4])
def test_short_row_threshold_widths(topk, W):
    # the widest batch the short-row kernel takes, and one the persistent
    # kernel takes, both exact
    wl = synth.mixed_rows(["normal", "crowd4096", "onebin", "clustered_peaks"] * 2, W, 2048, seed=36)
    wl.lengths = np.array([W, W - 1, W - 2, W - 3, 5000, 4097, 2049, 1], np.int32)
    synth.poison_tails(wl.scores, wl.lengths)
    got, _ = run(topk, wl)
    assert_parity(wl, got, expect(wl))


def test_short_rows_past_16384_stay_sampled(topk):
    # rows of 16385..32768 scores take a sample of 64 runs: at k = 2048 their
    # survivors (about 1.4 m) stay well inside the 3840-entry buffer, so every
    # N(0,1) row keeps to the sampled path (with 32 runs, about one such row
    # in eleven overflowed into the full-row selection)
    rng = np.random.default_rng(57)
    B, W, k = 64, 32768, 2048
    scores = rng.standard_normal((B, W)).astype(np.float32)
    lengths = rng.integers(16385, W + 1, B).astype(np.int32)
    lengths[:3] = [16385, W, W - 1]
    synth.poison_tails(scores, lengths)
    wl = synth.Workload("short_past_16384", 57, scores, lengths, W, k)
    got, stats = run(topk, wl, want_stats=True)
    assert_parity(wl, got, expect(wl))
    assert np.all(stats[:, 0] == 3), f"rows off the sampled path: {np.unique(stats[:, 0], return_counts=True)}"
    assert stats[:, 1].max() <= SHORT_CAP and stats[:, 1].min() >= k


def test_short_rows_overflow_fallback(topk):
    # rows whose sample hides a crowd just above the cutoff: more survivors
    # than the LDS buffer holds, so the full-row selection runs
    wl = synth.c2(2048)
    got, stats = run(topk, wl, want_stats=True)
    assert_parity(wl, got, expect(wl))
    paths = dict(zip(*np.unique(stats[:, 0], return_counts=True)))
    say("  short-row paths on the adversarial rows:", paths)
    assert paths.get(4, 0) > 0, "some adversarial row overflows the buffer"


@pytest.mark.parametrize("W", [20000, 40000], ids=["short_rows", "persistent"])
@pytest.mark.parametrize("page_size", [1, 3, 100, 4096])
def test_page_sizes(topk, W, page_size):
    # page sizes that are not powers of two, one and larger than some rows;
    # page-table slots offset per row so a row-mixing mistake shows
    k = 777
    kinds = ["normal", "heavy_ties", "signed_zero", "neginf_few_finite", "ascending", "clustered_peaks"]
    wl = synth.mixed_rows(kinds, W, k, seed=37)
    wl.lengths = np.array([W, W - 1, 5000, k + 1, k - 1, 4099], np.int32)
    synth.poison_tails(wl.scores, wl.lengths)
    pages = -(-W // page_size)
    rng = np.random.default_rng(38)
    wl.page_table = np.stack([rng.permutation(pages) + 7 * pages * b for b in range(wl.batch)]).astype(np.int32)
    wl.page_size = page_size
    got, _ = run(topk, wl)
    assert_parity(wl, got, expect(wl))


@pytest.mark.parametrize("page_size", [1, 3, 100])
def test_bf16_page_sizes(topk, page_size):
    W, k = 16384, 500
    rng = np.random.default_rng(39)
    bits = synth.to_bf16_bits(rng.standard_normal((5, W)).astype(np.float32))
    lengths = np.array([W, 9000, k + 1, k, 3], np.int32)
    synth.poison_tails_bf16(bits, lengths)
    pages = -(-W // page_size)
    pt = np.stack([rng.permutation(pages) + 5 * pages * b for b in range(5)]).astype(np.int32)
    wl = synth.Bf16Workload("bf16_pages", 39, bits, lengths, W, k, pt, page_size)
    s = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    out = topk.topk_select_bf16(s, torch.from_numpy(lengths).cuda(), k, None, torch.from_numpy(pt).cuda(),
                                page_size)
    torch.cuda.synchronize()
    want = oracle.topk_bf16(bits, lengths, k, page_table=pt, page_size=page_size)
    fails = check(oracle.bf16_to_f32(bits), lengths, W, k, out.cpu().numpy(), want, page_table=pt,
                  page_size=page_size)
    assert not fails, "\n".join(fails)


def tie_rows(ties, W=16384, k=512, seed=41):
    """bf16 bit patterns of 4 rows whose cutoff falls inside a group of `ties`
    equal scores: k - 17 distinct scores above it (consecutive bf16 patterns),
    the rest below. Rows 0 and 2 tie at +32, rows 1 and 3 at -1 (the order key
    of a negative bf16 score has its low 16 bits set); rows 2 and 3 are
    ragged."""
    rng = np.random.default_rng(seed + ties)
    above = k - 17
    bits = np.empty((4, W), np.uint16)
    for b in range(4):
        if b % 2 == 0:   # background |N(0,1)| < 32, ties at +32, above from +64 up
            row = synth.to_bf16_bits(rng.standard_normal(W).astype(np.float32))
            tie, top = 0x4200, 0x4280 + np.arange(above)
        else:            # background below -2, ties at -1, above from +1 up
            row = synth.to_bf16_bits((-2.0 - np.abs(rng.standard_normal(W))).astype(np.float32))
            tie, top = 0xBF80, 0x3F80 + np.arange(above)
        pos = rng.permutation(W - 8)[:above + ties]
        row[pos[:above]] = top
        row[pos[above:]] = tie
        bits[b] = row
    lengths = np.array([W, W, W - 5, W - 7], np.int32)
    return bits, lengths


@pytest.mark.parametrize("ties", [18, 63, 64, 65, 300])
def test_short_rows_ties_at_the_cutoff(topk, ties):
    # 17 of the tied scores are taken, those at the lowest positions: up to 64
    # tied positions are ranked by one wave, more by radix passes; the same
    # rows as fp32 and as bf16
    W, k = 16384, 512
    bits, lengths = tie_rows(ties, W, k)
    synth.poison_tails_bf16(bits, lengths)
    scores = oracle.bf16_to_f32(bits)
    wl = synth.Workload(f"ties{ties}", 41, scores, lengths, W, k)
    got, _ = run(topk, wl)
    assert_parity(wl, got, expect(wl))
    s = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    say(f"  gpu bf16 call: ties{ties}")
    out = topk.topk_select_bf16(s, torch.from_numpy(lengths).cuda(), k)
    torch.cuda.synchronize()
    want = oracle.topk_bf16(bits, lengths, k)
    fails = check(scores, lengths, W, k, out.cpu().numpy(), want)
    assert not fails, "\n".join(fails)


@pytest.mark.parametrize("n_inf,k", [(1, 512), (100, 512), (512, 512), (600, 512), (50, 40), (5000, 512)])
def test_short_rows_infinities(topk, n_inf, k):
    # +inf scores in a short row: a finite cutoff (1, 100), every +inf taken
    # exactly (512), ties at +inf ranked by radix passes (600) or by one wave
    # (50 of k = 40), and more survivors than the buffer holds (5000); as
    # fp32 and as bf16 rows, the last row +inf at its last valid position only
    # (the block-max kernel's newest block); the fp32 rows also through the
    # split-row entry
    W = 16384
    rng = np.random.default_rng(42 + n_inf)
    x = (rng.standard_normal((4, W)) + 1.4).astype(np.float32)
    lengths = np.array([W, W - 3, 9000, 12001], np.int32)
    for b in range(3):
        x[b, rng.permutation(int(lengths[b]))[:n_inf]] = np.inf
    x[3, lengths[3] - 1] = np.inf
    bits = synth.to_bf16_bits(x)
    synth.poison_tails_bf16(bits, lengths)
    scores = oracle.bf16_to_f32(bits)
    wl = synth.Workload(f"inf{n_inf}", 42, scores, lengths, W, k)
    want32 = expect(wl)
    got, _ = run(topk, wl)
    assert_parity(wl, got, want32)
    say(f"  gpu split call: inf{n_inf} k={k}")
    out_s = topk.topk_select_split(to_dev(wl.scores), to_dev(wl.lengths), k)
    torch.cuda.synchronize()
    assert_parity(wl, out_s.cpu().numpy(), want32)
    s = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    say(f"  gpu bf16 call: inf{n_inf} k={k}")
    out = topk.topk_select_bf16(s, torch.from_numpy(lengths).cuda(), k)
    torch.cuda.synchronize()
    want = oracle.topk_bf16(bits, lengths, k)
    fails = check(scores, lengths, W, k, out.cpu().numpy(), want)
    assert not fails, "\n".join(fails)


# ----------------------------------------------------------------------------
# a sample that sees only the peaks: survivors fall short of m
# ----------------------------------------------------------------------------

def sample_positions(L, max_runs, align):
    """Where a sampling path reads a row of length L: runs of 64 scores at
    floor(r (L - 64) / (runs - 1)) rounded down to a multiple of `align`,
    runs = min(L // 128, max_runs). The persistent kernel takes 64 runs on
    16-byte loads (align 4); the short-row kernel 32 runs (64 for rows longer
    than 16384) on 128-byte lines (align 32 here, where every row starts on a
    line)."""
    runs = min(L // 128, max_runs)
    pos = []
    for r in range(runs):
        start = (r * (L - 64) // (runs - 1)) // align * align
        pos.extend(range(start, start + 64))
    return np.array(pos, np.int64)


@pytest.mark.parametrize("W,k", [(20000, 512), (131072, 2048), (131072, 512)],
                         ids=["short_rows", "persistent_k2048", "persistent_k512"])
def test_sample_that_sees_only_peaks_underflows(topk, W, k):
    # peaks planted on sampled positions only, fewer than m of them: the
    # sampled cutoff lands among the peaks, fewer than m scores survive, and
    # the full-row selection must take over (the pages' sampled-peaks case)
    rng = np.random.default_rng(40)
    B = 4
    scores = rng.standard_normal((B, W)).astype(np.float32)
    lengths = np.array([W, W - 3, W - 17, W], np.int32)
    # peaks where both this row's kernel and the split-row entry (64 runs on
    # 128-byte lines) sample; every row starts on a 128-byte line
    short = W <= 32768
    assert (W * 4) % 128 == 0
    for b in range(B):
        L = int(lengths[b])
        runs = (32 if L <= 16384 else 64) if short else 64
        pos = np.intersect1d(sample_positions(L, runs, 32 if short else 4), sample_positions(L, 64, 32))
        assert pos.size >= k // 2
        hit = rng.choice(pos, min(k // 2, pos.size), replace=False)
        scores[b, hit] = (50.0 + rng.standard_normal(hit.size)).astype(np.float32)
    synth.poison_tails(scores, lengths)
    wl = synth.Workload("sampled_peaks", 40, scores, lengths, W, k)
    want = expect(wl)
    got, stats = run(topk, wl, want_stats=True)
    assert_parity(wl, got, want)
    assert np.all(stats[:, 0] == 5), f"every row must take the underflow fallback: {stats[:, 0]}"
    if W > 16384:
        got, stats = run(topk, wl, force=2, want_stats=True)
        assert_parity(wl, got, want)
        assert np.all(stats[:, 0] == 5)
    # the split-row entry's sample sees the same peaks
    buf = torch.full((B, k), CANARY, dtype=torch.int32, device="cuda")
    sstats = torch.full((B, 2), -7, dtype=torch.int32, device="cuda")
    topk.topk_select_split(to_dev(wl.scores), to_dev(wl.lengths), k, buf, row_stats=sstats)
    torch.cuda.synchronize()
    assert_parity(wl, buf.cpu().numpy(), want)
    assert np.all(sstats.cpu().numpy()[:, 0] == 5)


@pytest.mark.parametrize("W", [20000, 131072])
def test_permuted_rows_select_the_same_values(topk, W):
    # the same multiset under a random permutation: the same selected values
    k = 1024
    wl = synth.mixed_rows(["heavy_ties", "onebin", "crowd4096", "signed_zero", "neginf_half", "normal"], W, k,
                          seed=41)
    rng = np.random.default_rng(42)
    perm = np.stack([rng.permutation(W) for _ in range(wl.batch)])
    pw = synth.Workload("permuted", 42, np.take_along_axis(wl.scores, perm, axis=1), wl.lengths, W, k)
    a, _ = run(topk, wl)
    b, _ = run(topk, pw)
    bits = wl.scores.view(np.uint32)
    pbits = pw.scores.view(np.uint32)
    for r in range(wl.batch):
        assert np.array_equal(np.sort(bits[r, a[r]]), np.sort(pbits[r, b[r]]))
    assert_parity(pw, b, expect(pw))
