"""GPU parity of the indexer's other kernels against the CPU oracle: bf16
top-k, the block max of every 8 scores and the candidate block table, each
through the C ABI, and the three chained as the two-level indexer runs them
(block max -> fp32 top-k over the block keys -> block table).

Selections are compared index for index (the oracle's lowest-index ties are
the kernels' too) with values bit for bit; block maxima bit for bit (NaN
ignored, +0 above -0); block tables and pool slots exactly. Outputs sit
between guard regions that must come back untouched.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from topk_check import check, check_codes

pytestmark = pytest.mark.gpu

GUARD = 4096
CANARY = 0x5A5A5A5A
INT32_MAX = 2**31 - 1


@pytest.fixture(scope="module")
def topk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_row_top_fp32_amd as topk_mod
    topk_mod._load()
    return topk_mod


def say(*msg):
    print(*msg, flush=True)


def guarded(shape, dtype, fill):
    n = int(np.prod(shape))
    buf = torch.full((n + 2 * GUARD,), fill, dtype=dtype, device="cuda")
    return buf, buf[GUARD:GUARD + n].view(*shape)


def guards_intact(buf, fill):
    h = buf.cpu()
    return bool(torch.all(h[:GUARD] == fill)) and bool(torch.all(h[-GUARD:] == fill))


# ----------------------------------------------------------------------------
# bf16 top-k
# ----------------------------------------------------------------------------

def run_bf16(topk, wl, k=None, lengths=None, n_cols=None):
    k = wl.k if k is None else k
    s = torch.from_numpy(wl.bits.view(np.int16)).cuda().view(torch.bfloat16)
    ln = torch.from_numpy(np.ascontiguousarray(wl.lengths if lengths is None else lengths)).cuda()
    pt = torch.from_numpy(wl.page_table).cuda() if wl.page_table is not None else None
    buf, out = guarded((wl.batch, k), torch.int32, CANARY)
    say(f"  gpu bf16 call: {wl.name} k={k}")
    topk.topk_select_bf16(s, ln, k, out, pt, wl.page_size, n_cols=n_cols or wl.n_cols)
    torch.cuda.synchronize()
    assert guards_intact(buf, CANARY), "write outside out"
    return out.cpu().numpy()


def bf16_parity(wl, got, k=None, lengths=None, n_cols=None, rows=None):
    k = wl.k if k is None else k
    lengths = wl.lengths if lengths is None else lengths
    n_cols = n_cols or wl.n_cols
    want = oracle.topk_bf16(wl.bits, lengths, k, n_cols=n_cols, page_table=wl.page_table,
                            page_size=wl.page_size)
    same = np.all(np.sort(got, 1) == np.sort(want, 1), axis=1)
    assert same.all(), f"rows differing from the oracle: {np.flatnonzero(~same)[:10]}"
    fails = check(oracle.bf16_to_f32(wl.bits), lengths, n_cols, k, got, want, page_table=wl.page_table,
                  page_size=wl.page_size, rows=rows)
    assert not fails, "\n".join(fails)


def test_bf16_consumer_rows_paged(topk):
    wl = synth.bf16_rows()  # 1024 x 16384, k=2048, page_size 64
    got = run_bf16(topk, wl)
    bf16_parity(wl, got, rows=range(0, wl.batch, 37))


@pytest.mark.parametrize("k", [1, 2, 64, 512, 2047, 2048])
def test_bf16_raw_k_range(topk, k):
    wl = synth.bf16_rows(64, 16384, k, seed=61, paged=False)
    bf16_parity(wl, run_bf16(topk, wl))


@pytest.mark.parametrize("k", [512, 1024, 2048])
def test_bf16_adversarial_rows(topk, k):
    wl = synth.bf16_adversarial(k)
    bf16_parity(wl, run_bf16(topk, wl))


def test_bf16_length_boundaries(topk):
    k, W, stride = 512, 16384, 16392
    lens = np.array([-1, 0, 1, k - 1, k, k + 1, 7, 9, 517, 8191, 16377, 16383, W, W + 17], np.int32)
    rng = np.random.default_rng(64)
    bits = synth.to_bf16_bits(rng.standard_normal((lens.size, stride)).astype(np.float32))
    synth.poison_tails_bf16(bits, np.clip(lens, 0, W))
    wl = synth.Bf16Workload("bf16_lengths", 64, bits, lens, W, k)
    bf16_parity(wl, run_bf16(topk, wl))


@pytest.mark.parametrize("k", [512, 2048])
@pytest.mark.parametrize("force", [0, 1, 2, 3], ids=["auto", "lds", "sampled", "fullrow"])
def test_bf16_forced_paths(topk, force, k):
    # every path of the bf16 kernel on the adversarial rows and on rows whose
    # lengths sit at k, the LDS capacity and the width, with the path code of
    # every row checked; the default capacity, then a small one
    cap = topk.topk_short_capacity()
    adv = synth.bf16_adversarial(k)
    W = 16384
    lens = np.array([-1, 0, 1, k - 1, k, k + 1, cap - 1, cap, cap + 1, 2 * cap, W - 1, W, W + 17], np.int32)
    rng = np.random.default_rng(72 + k)
    bits = synth.to_bf16_bits(rng.standard_normal((lens.size, W)).astype(np.float32))
    synth.poison_tails_bf16(bits, np.clip(lens, 0, W))
    edges = synth.Bf16Workload("bf16_length_edges", 72, bits, lens, W, k)
    for wl in (adv, edges):
        for capacity in (0, 700):
            ln = torch.from_numpy(np.ascontiguousarray(wl.lengths)).cuda()
            s = torch.from_numpy(wl.bits.view(np.int16)).cuda().view(torch.bfloat16)
            pt = torch.from_numpy(wl.page_table).cuda() if wl.page_table is not None else None
            buf, out = guarded((wl.batch, k), torch.int32, CANARY)
            stats = torch.full((wl.batch, 2), -7, dtype=torch.int32, device="cuda")
            say(f"  gpu bf16 call: {wl.name} k={k} force={force} cap={capacity}")
            topk.topk_select_bf16_ex(s, ln, k, out, pt, wl.page_size, n_cols=wl.n_cols, force_path=force,
                                     capacity=capacity, row_stats=stats)
            torch.cuda.synchronize()
            assert guards_intact(buf, CANARY), "write outside out"
            bf16_parity(wl, out.cpu().numpy(), k=k)
            fails = check_codes(stats.cpu().numpy(), wl.lengths, wl.n_cols, k, force, capacity or cap)
            assert not fails, "\n".join(fails[:10])


def test_bf16_single_row_odd_width(topk):
    rng = np.random.default_rng(65)
    for W in (5, 1001, 16383):
        bits = synth.to_bf16_bits(rng.standard_normal((1, W)).astype(np.float32))
        bits[0, -1] = 0x4480  # 1024.0: the very last score must be found
        wl = synth.Bf16Workload(f"bf16_w{W}", 65, bits, np.array([W], np.int32), W, 3)
        bf16_parity(wl, run_bf16(topk, wl))


# ----------------------------------------------------------------------------
# block max
# ----------------------------------------------------------------------------

def run_amax(topk, wl, lengths=None, topk_k=None, fill=12345.0):
    topk_k = wl.topk if topk_k is None else topk_k
    lengths = wl.lengths if lengths is None else lengths
    s = torch.from_numpy(wl.scores).cuda()
    ln = torch.from_numpy(np.ascontiguousarray(lengths)).cuda()
    buf, out = guarded((wl.batch, wl.out_blocks), torch.float32, fill)
    say(f"  gpu amax8 call: {wl.name} topk={topk_k}")
    topk.amax8_varlen(s, ln, topk_k, out=out)
    torch.cuda.synchronize()
    assert guards_intact(buf, fill), "write outside out"
    got = out.cpu().numpy()
    want = np.full((wl.batch, wl.out_blocks), fill, np.float32)
    oracle.amax8(wl.scores, lengths, topk_k, want)
    bad = np.flatnonzero(np.any(got.view(np.uint32) != want.view(np.uint32), axis=1))
    assert bad.size == 0, f"rows differing bit for bit: {bad[:10]}"
    return got


@pytest.mark.parametrize("topk_k", [0, 512])
def test_amax8_decode_rows(topk, topk_k):
    wl = synth.amax8_rows(256, 131072, topk_k, nan_rate=1e-4, zero_rate=1e-3)
    run_amax(topk, wl)


def test_amax8_lengths_and_skip_rule(topk):
    W, t = 16384, 64
    lens = np.array([-3, 0, 1, 7, 8, 9, 8 * t - 1, 8 * t, 8 * t + 1, 8 * 1000 + 5, W - 1, W, W + 40], np.int32)
    wl = synth.amax8_rows(lens.size, W, t, seed=66, nan_rate=0.02, zero_rate=0.05)
    run_amax(topk, wl, lengths=lens)
    run_amax(topk, wl, lengths=lens, topk_k=0)


def test_amax8_all_nan_and_signed_zero_blocks(topk):
    W = 4096
    x = np.random.default_rng(67).standard_normal((4, W)).astype(np.float32)
    x[0, 8:16] = np.nan                          # all NaN -> NaN
    x[0, 16:24] = [-0.0, 0.0, -1, -2, np.nan, -0.0, -3, -4]   # +0 wins over -0
    x[0, 24:32] = [-0.0] * 8                     # -0
    x[1, :] = -np.inf
    x[2, ::2] = np.nan                           # NaN ignored everywhere
    wl = synth.Amax8Workload("amax8_edges", 67, x, np.array([W, W, W, 100], np.int32), W // 8, 0)
    got = run_amax(topk, wl)
    assert np.isnan(got[0, 1]) and got[0, 2] == 0 and not np.signbit(got[0, 2]) and np.signbit(got[0, 3])


def test_amax8_lengths_past_n_cols(topk):
    # n_cols below the width of the storage, lengths past it: each row acts as
    # if its length were n_cols; the scores past n_cols are large, so reading
    # any of them would show in the keys
    W, stride = 4096 + 19 * 8 + 3, 4096 + 64 * 8
    lens = np.array([W, W + 1, W + 7, W + 8, W + 300, 2**31 - 1, W - 1, 0], np.int32)
    rng = np.random.default_rng(70)
    x = rng.standard_normal((lens.size, stride)).astype(np.float32)
    x[:, W:] = 1e30
    for topk_k in (0, 300, W // 8):
        s = torch.from_numpy(x).cuda()
        ln = torch.from_numpy(lens).cuda()
        cols = stride // 8
        buf, out = guarded((lens.size, cols), torch.float32, -7.0)
        say(f"  gpu amax8 call: lengths past n_cols={W}, topk={topk_k}")
        topk.amax8_varlen(s, ln, topk_k, max_seqlen=W, out=out)
        torch.cuda.synchronize()
        assert guards_intact(buf, -7.0), "write outside out"
        want = np.full((lens.size, cols), -7.0, np.float32)
        oracle.amax8(x, lens, topk_k, want, n_cols=W)
        got = out.cpu().numpy()
        bad = np.flatnonzero(np.any(got.view(np.uint32) != want.view(np.uint32), axis=1))
        assert bad.size == 0, f"rows differing bit for bit: {bad[:10]}"


# ----------------------------------------------------------------------------
# candidate block table
# ----------------------------------------------------------------------------

def run_table(topk, wl, n_cols):
    blocks = torch.from_numpy(wl.blocks.copy()).cuda()
    ln = torch.from_numpy(wl.lengths).cuda()
    pt = torch.from_numpy(wl.page_table).cuda()
    buf, pages = guarded(tuple(wl.blocks.shape), torch.int32, CANARY)
    say(f"  gpu block table call: {wl.name}")
    topk.sort_candidate_blocks(blocks, ln, pt, wl.page_size, out_pages=pages, n_cols=n_cols)
    torch.cuda.synchronize()
    assert guards_intact(buf, CANARY), "write outside out_pages"
    table, slots = oracle.sort_candidate_blocks(wl.blocks, wl.lengths, wl.page_table, wl.page_size, n_cols=n_cols)
    got_t, got_p = blocks.cpu().numpy(), pages.cpu().numpy()
    bad = np.flatnonzero(np.any(got_t != table, axis=1) | np.any(got_p != slots, axis=1))
    assert bad.size == 0, f"rows differing: {bad[:10]}"


@pytest.mark.parametrize("page_size", [8, 64, 256])
def test_block_table_decode_rows(topk, page_size):
    wl = synth.candidate_blocks(1024, 131072, 512, page_size=page_size)
    run_table(topk, wl, 131072)


def test_block_table_junk_entries_and_large_rows(topk):
    # entries outside [0, nb) and repeats are ignored; rows up to 2^21 positions
    rng = np.random.default_rng(68)
    W, k = 2 ** 21, 300
    lens = np.array([W, W - 5, 8 * k, 8 * k + 1, 0, -4, 12345], np.int32)
    blocks = np.full((lens.size, k), -1, np.int32)
    for b, L in enumerate(lens):
        nb = -(-max(int(L), 0) // 8)
        if nb > k:
            blocks[b] = rng.choice(nb, k, replace=False)
            junk = rng.random(k) < 0.2
            blocks[b, junk] = rng.choice([-1, nb, nb + 99, -7, int(blocks[b, 0])], int(junk.sum()))
    pt = np.stack([rng.permutation(W // 64) for _ in lens]).astype(np.int32)
    wl = synth.BlockTableWorkload("blocks_junk", 68, blocks, lens, pt, 64)
    run_table(topk, wl, W)


def test_block_table_lengths_past_n_cols(topk):
    # lengths past n_cols count as n_cols: ids at or past ceil(n_cols / 8) are
    # dropped, and a row whose clamped block count is at most k takes the
    # identity table whatever its length says
    rng = np.random.default_rng(71)
    k, ps = 64, 64
    for n_cols in (8 * 500 + 3, 8 * 64, 8 * 64 + 1):
        nb = -(-n_cols // 8)
        lens = np.array([n_cols, n_cols + 1, n_cols + 8, n_cols + 5000, 2**31 - 1, n_cols - 9, -2], np.int32)
        blocks = np.stack([rng.choice(nb + 200, k, replace=False) for _ in lens]).astype(np.int32)
        pt = np.stack([rng.permutation(-(-(nb + 200) // (ps // 8))) for _ in lens]).astype(np.int32)
        wl = synth.BlockTableWorkload(f"blocks_past_n_cols_{n_cols}", 71, blocks, lens, pt, ps)
        run_table(topk, wl, n_cols)


# ----------------------------------------------------------------------------
# the two-level indexer, chained
# ----------------------------------------------------------------------------

def test_amax8_on_the_bench_batch(topk, c3):
    # the block max exactly as the bench times it: the 1024 x 131072 decode
    # batch, topk = 512
    wl = synth.Amax8Workload("amax8_c3", 3, c3.scores, c3.lengths, c3.n_cols // 8, 512)
    run_amax(topk, wl)


def test_two_level_indexer_chain(topk, c3):
    # the whole decode batch, as the bench chains it, with edge lengths in the
    # first rows
    B, k, ps = c3.batch, 512, 64
    scores = c3.scores[:B]
    lengths = c3.lengths[:B].copy()
    lengths[:8] = [0, 1, 7, 8 * k, 8 * k + 1, 100, 4000, 8 * k - 3]
    nblk = c3.n_cols // 8
    s = torch.from_numpy(np.ascontiguousarray(scores)).cuda()
    ln = torch.from_numpy(lengths).cuda()
    keys = torch.full((B, nblk), 7.0, dtype=torch.float32, device="cuda")
    topk.amax8_varlen(s, ln, k, out=keys)
    nb = torch.from_numpy(((np.maximum(lengths, 0).astype(np.int64) + 7) // 8).astype(np.int32)).cuda()
    blocks = topk.topk_select(keys, nb, k)
    rng = np.random.default_rng(69)
    pt_h = np.stack([rng.permutation(nblk // (ps // 8)) for _ in range(B)]).astype(np.int32)
    pages = topk.sort_candidate_blocks(blocks, ln, torch.from_numpy(pt_h).cuda(), ps, n_cols=c3.n_cols)
    torch.cuda.synchronize()

    want_keys = np.full((B, nblk), 7.0, np.float32)
    oracle.amax8(scores, lengths, k, want_keys)
    assert np.array_equal(keys.cpu().numpy().view(np.uint32), want_keys.view(np.uint32))
    nb_h = nb.cpu().numpy()
    want_sel = oracle.topk(want_keys, nb_h, k)
    table, slots = oracle.sort_candidate_blocks(want_sel, lengths, pt_h, ps, n_cols=c3.n_cols)
    assert np.array_equal(blocks.cpu().numpy(), table)
    assert np.array_equal(pages.cpu().numpy(), slots)
