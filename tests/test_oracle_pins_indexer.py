"""Pins for the oracle's bf16 selection and the two-level indexer's neighbours.

Definitions under test ("dsv4.1: Top-k kernels and candidate selection",
implementation section 2 and code excerpts): the bf16 small-row top-k (the
fp32 selection over exactly widened bf16 rows), the block max of every 8
scores (NaN ignored, the newest block +inf, rows with at most topk blocks
untouched) and the candidate block table (ids ascending, INT32_MAX padding,
pool slots page_table[b, id // bpp] * bpp + id % bpp with bpp = page_size / 8,
the identity table for rows with at most k blocks).

No page prints a worked example, so every expectation comes from something
other than the oracle's own code: bf16 values decoded independently through
``struct``, subset brute force, torch's bf16 topk and amax, closed forms, and
the inverse of the page mapping. Each pin takes the function under test as an
argument, so the planted-mistake tests at the end can show that a plausible
slip in any of the three definitions fails some pin.
"""
from __future__ import annotations

import itertools
import math
import struct

import numpy as np
import pytest
import torch

import oracle

INT32_MAX = 2**31 - 1

# bf16 patterns: -inf, -1, -0, +0, smallest subnormal, 1, 65536, largest finite, +inf
BF16_ALPHABET = np.array([0xFF80, 0xBF80, 0x8000, 0x0000, 0x0001, 0x3F80, 0x4780, 0x7F7F, 0x7F80],
                         dtype=np.uint16)


def bf16_value(bits: int) -> float:
    """Decode a bf16 pattern without the oracle's helper: it is the big-endian
    fp32 whose first two bytes are the pattern."""
    return struct.unpack(">f", struct.pack(">HH", int(bits), 0))[0]


def rank_tuple(v: float):
    return (v, not math.copysign(1.0, v) < 0)


# ----------------------------------------------------------------------------
# bf16 top-k
# ----------------------------------------------------------------------------

def pin_bf16_brute_force(fn, seed=61, cases=250):
    rng = np.random.default_rng(seed)
    for _ in range(cases):
        L = int(rng.integers(0, 9))
        k = int(rng.integers(1, L + 3))
        row = np.full((1, max(L, 1) + 1), 0x7FC0, np.uint16)
        row[0, :L] = rng.choice(BF16_ALPHABET, L)
        got = fn(row, np.array([L], np.int32), k, n_cols=row.shape[1])[0]
        m = min(k, L)
        keys = [rank_tuple(bf16_value(v)) for v in row[0, :L]]
        valid = [s for s in itertools.combinations(range(L), m)
                 if not s or len(s) == L
                 or min(keys[i] for i in s) >= max(keys[i] for i in range(L) if i not in s)]
        assert list(got[m:]) == [-1] * (k - m)
        chosen = tuple(sorted(got[:m].tolist()))
        assert chosen in valid and chosen == min(valid), (row, k, got)


def pin_bf16_torch_topk(fn, seed=62):
    rng = np.random.default_rng(seed)
    for L, k in [(1000, 37), (16384, 2048), (2000, 2000), (777, 1)]:
        vals = torch.randn(L, generator=torch.Generator().manual_seed(int(rng.integers(1 << 30))))
        vals = vals * 3 + 0.25
        t = vals.to(torch.bfloat16)
        bits = t.view(torch.int16).numpy().view(np.uint16)[None, :].copy()
        got = fn(bits, np.array([L], np.int32), k)[0]
        m = min(k, L)
        ref = torch.topk(t.float(), m).values
        sel = torch.from_numpy(np.array([bf16_value(b) for b in bits[0, got[:m]]], np.float32))
        assert torch.equal(torch.sort(sel, descending=True).values, ref)


def pin_bf16_closed_forms(fn):
    W, k = 600, 64
    # ascending positive patterns are ascending values: the last m positions
    asc = np.arange(1, W + 1, dtype=np.uint16)[None, :]
    got = fn(asc, np.array([500], np.int32), k, n_cols=W)[0]
    assert set(got.tolist()) == set(range(500 - k, 500))
    # negative patterns: larger pattern, smaller value -> the first m positions
    neg = (0x8000 + np.arange(1, W + 1)).astype(np.uint16)[None, :]
    got = fn(neg, np.array([W], np.int32), k, n_cols=W)[0]
    assert set(got.tolist()) == set(range(k))
    # constant, short and empty rows
    const = np.full((3, W), 0x3F80, np.uint16)
    got = fn(const, np.array([W, 10, 0], np.int32), k, n_cols=W)
    assert set(got[0].tolist()) == set(range(k))
    assert sorted(got[1, :10].tolist()) == list(range(10)) and np.all(got[1, 10:] == -1)
    assert np.all(got[2] == -1)
    # signed zeros: the positives, then +0s before any -0
    z = np.array([[0x8000, 0x0000, 0x8000, 0x3F80, 0x0000, 0x8000, 0xBF80]], np.uint16)
    got = fn(z, np.array([7], np.int32), 4, n_cols=7)[0]
    assert set(got.tolist()) == {3, 1, 4, 0}


def pin_bf16_paged(fn):
    rng = np.random.default_rng(63)
    W, k, ps = 640, 40, 64
    bits = np.arange(1, W + 1, dtype=np.uint16)[None, :].repeat(2, 0)
    pt = np.stack([rng.permutation(W // ps) + 100 * b for b in range(2)]).astype(np.int32)
    got = fn(bits, np.array([W, 300], np.int32), k, n_cols=W, page_table=pt, page_size=ps)
    for b, L in enumerate((W, 300)):
        inv = {int(p): j for j, p in enumerate(pt[b])}
        raw = sorted(inv[int(s) // ps] * ps + int(s) % ps for s in got[b])
        assert raw == list(range(L - k, L))


BF16_PINS = [pin_bf16_brute_force, pin_bf16_torch_topk, pin_bf16_closed_forms, pin_bf16_paged]


# ----------------------------------------------------------------------------
# block max
# ----------------------------------------------------------------------------

AMAX_ALPHABET = np.array([np.nan, -np.inf, -2.5, -0.0, 0.0, 1e-45, 3.0, np.inf], np.float32)


def ref_block(vals) -> float:
    """Independent statement: the largest under (value, +0 above -0) of the
    non-NaN entries; NaN if there are none."""
    live = [float(v) for v in vals if not math.isnan(float(v))]
    return max(live, key=rank_tuple) if live else math.nan


def same_bits(a: float, b: float) -> bool:
    if math.isnan(a) or math.isnan(b):
        return math.isnan(a) and math.isnan(b)
    return a == b and math.copysign(1.0, a) == math.copysign(1.0, b)


def pin_amax_brute_force(fn, seed=71, cases=300):
    rng = np.random.default_rng(seed)
    for _ in range(cases):
        W = 8 * int(rng.integers(1, 7))
        n_cols = int(rng.integers(0, W + 1))  # the scores past n_cols are never read
        L = int(rng.integers(-2, W + 12))
        topk = int(rng.integers(0, 4))
        x = rng.choice(AMAX_ALPHABET, (1, W)).astype(np.float32)
        out = np.full((1, W // 8 + 3), 77.0, np.float32)
        fn(x, np.array([L], np.int32), topk, out, n_cols=n_cols)
        nb = -(-min(max(L, 0), n_cols) // 8)
        skipped = nb == 0 or (topk > 0 and nb <= topk)
        for i in range(out.shape[1]):
            if skipped or i >= nb:
                assert out[0, i] == 77.0
            elif i == nb - 1:
                assert out[0, i] == np.inf
            else:
                assert same_bits(float(out[0, i]), ref_block(x[0, 8 * i:8 * i + 8])), (x, L, i, out)


def pin_amax_torch(fn, seed=72):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((3, 4096)) + 0.01).astype(np.float32)  # no zeros, no NaN
    lengths = np.array([4096, 4001, 17], np.int32)
    out = np.zeros((3, 512), np.float32)
    fn(x, lengths, 0, out)
    for b, L in enumerate(lengths):
        nb = -(-int(L) // 8)
        ref = torch.from_numpy(x[b, :8 * (nb - 1)].copy()).view(-1, 8).amax(dim=1).numpy()
        assert np.array_equal(out[b, :nb - 1], ref) and out[b, nb - 1] == np.inf


def pin_amax_closed_forms(fn):
    W = 128
    asc = np.arange(W, dtype=np.float32)[None, :].repeat(4, 0)
    out = np.full((4, W // 8), -5.0, np.float32)
    fn(asc, np.array([W, 41, 1, 0], np.int32), 0, out)
    assert np.array_equal(out[0, :-1], np.arange(7, W - 8, 8, dtype=np.float32)) and out[0, -1] == np.inf
    assert np.array_equal(out[1, :5], [7, 15, 23, 31, 39]) and out[1, 5] == np.inf and np.all(out[1, 6:] == -5)
    assert out[2, 0] == np.inf and np.all(out[2, 1:] == -5)
    assert np.all(out[3] == -5)
    # the skip rule: nb <= topk leaves the row alone, nb > topk writes it
    out = np.full((2, W // 8), -5.0, np.float32)
    fn(asc[:2], np.array([8 * 3, 8 * 3 + 1], np.int32), 3, out)
    assert np.all(out[0] == -5) and out[1, 3] == np.inf and out[1, 0] == 7


def pin_amax_length_clamp(fn):
    """Lengths past n_cols act as n_cols: on ascending rows block i holds
    8 i + 7, the block at ceil(n_cols / 8) - 1 is +inf and nothing later is
    written, even though the row's storage goes on with larger values."""
    W = 128
    for n_cols in (80, 83, 121):
        nb = -(-n_cols // 8)
        lens = np.array([n_cols, n_cols + 1, n_cols + 7, n_cols + 8, n_cols + 40, 2**31 - 1], np.int32)
        x = np.arange(W, dtype=np.float32)[None, :].repeat(lens.size, 0)
        x[:, n_cols:] = 1e30
        out = np.full((lens.size, W // 8 + 2), -5.0, np.float32)
        fn(x, lens, 0, out, n_cols=n_cols)
        want = np.full(W // 8 + 2, -5.0, np.float32)
        want[:nb - 1] = 8 * np.arange(nb - 1) + 7
        want[nb - 1] = np.inf
        for b in range(lens.size):
            assert np.array_equal(out[b], want), (n_cols, int(lens[b]), out[b])
        # the skip rule counts the clamped blocks
        out = np.full((1, W // 8 + 2), -5.0, np.float32)
        fn(x[:1], np.array([n_cols + 60], np.int32), nb, out, n_cols=n_cols)
        assert np.all(out == -5.0)


AMAX_PINS = [pin_amax_brute_force, pin_amax_torch, pin_amax_closed_forms, pin_amax_length_clamp]


# ----------------------------------------------------------------------------
# candidate block table
# ----------------------------------------------------------------------------

def pin_blocks_invariants(fn, seed=81, cases=200):
    """Table = the row's in-range ids, strictly ascending, INT32_MAX after;
    every slot inverts through the row's page table to its id."""
    rng = np.random.default_rng(seed)
    for _ in range(cases):
        k = int(rng.integers(1, 12))
        ps = int(2 ** rng.integers(3, 7))
        bpp = ps // 8
        L = int(rng.integers(-3, 8 * 3 * k))
        nb = -(-max(L, 0) // 8)
        if nb > k:
            row = rng.choice(nb, k, replace=False).astype(np.int32)
            if rng.random() < 0.4:  # entries outside [0, nb): -1 padding and stray ids
                junk = rng.random(k) < 0.3
                row[junk] = rng.choice([-1, nb, nb + 7, -5], int(junk.sum()))
        else:
            row = rng.integers(-1, nb + 3, k).astype(np.int32)
        pages = -(-max(nb, 1) // bpp) + 1
        pt = (rng.permutation(pages) + 1000).astype(np.int32)[None, :]
        table, slots = fn(row[None, :].copy(), np.array([L], np.int32), pt, ps, n_cols=8 * 3 * k)
        want = list(range(nb)) if nb <= k else sorted(set(v for v in row.tolist() if 0 <= v < nb))
        n = len(want)
        assert table[0, :n].tolist() == want and np.all(table[0, n:] == INT32_MAX)
        assert np.all(slots[0, n:] == INT32_MAX)
        inv = {int(p): j for j, p in enumerate(pt[0])}
        for j in range(n):
            s = int(slots[0, j])
            assert inv[s // bpp] * bpp + s % bpp == want[j]


def pin_blocks_identity_pages(fn):
    rng = np.random.default_rng(82)
    k, L = 64, 8 * 1000
    row = rng.choice(1000, k, replace=False).astype(np.int32)[None, :]
    pt = np.arange(200, dtype=np.int32)[None, :]
    table, slots = fn(row, np.array([L], np.int32), pt, 64, n_cols=L)
    assert np.array_equal(table[0], np.sort(row[0])) and np.array_equal(slots[0], table[0])


def pin_blocks_short_rows(fn):
    # at most k blocks: the identity table whatever the input holds
    k = 16
    rows = np.full((3, k), 999, np.int32)
    rows[1] = -1
    pt = np.tile(np.arange(20, dtype=np.int32)[::-1], (3, 1))
    table, slots = fn(rows, np.array([8 * k, 8 * 5 - 7, 0], np.int32), pt, 8, n_cols=8 * 20)
    assert table[0].tolist() == list(range(k))
    assert table[1, :5].tolist() == list(range(5)) and np.all(table[1, 5:] == INT32_MAX)
    assert np.all(table[2] == INT32_MAX) and np.all(slots[2] == INT32_MAX)
    assert slots[0].tolist() == [19 - i for i in range(k)]


def pin_blocks_length_clamp(fn):
    """Lengths past n_cols act as n_cols. With n_cols = 323 a row spans 41
    blocks: ids 41 and up are dropped from a selection however long the row
    claims to be. With n_cols = 128 and k = 16 a row spans 16 <= k blocks, so
    its table is the identity whatever it holds and whatever its length."""
    k = 16
    given = np.array([40, 3, 41, 0, 17, 42, 99, 5, 39, 200, 1, 6, 2, 60, 7, 8], np.int32)
    want = sorted(v for v in given.tolist() if v < 41)
    lens = np.array([323, 324, 330, 1000, 2**31 - 1], np.int32)
    pt = np.tile(np.arange(100, dtype=np.int32) + 500, (lens.size, 1))
    table, slots = fn(np.tile(given, (lens.size, 1)), lens, pt, 8, n_cols=323)
    for b in range(lens.size):
        assert table[b, :len(want)].tolist() == want and np.all(table[b, len(want):] == INT32_MAX)
        assert slots[b, :len(want)].tolist() == [500 + v for v in want]
    table, slots = fn(np.tile(given, (3, 1)), np.array([128, 129, 5000], np.int32), pt[:3], 8, n_cols=128)
    assert np.array_equal(table, np.tile(np.arange(k, dtype=np.int32), (3, 1)))
    assert np.array_equal(slots, table + 500)


BLOCK_PINS = [pin_blocks_invariants, pin_blocks_identity_pages, pin_blocks_short_rows, pin_blocks_length_clamp]


# ----------------------------------------------------------------------------
# the oracle against its pins
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("pin", BF16_PINS, ids=lambda p: p.__name__)
def test_bf16_oracle_meets_pin(pin):
    pin(oracle.topk_bf16)


@pytest.mark.parametrize("pin", AMAX_PINS, ids=lambda p: p.__name__)
def test_amax8_oracle_meets_pin(pin):
    pin(oracle.amax8)


@pytest.mark.parametrize("pin", BLOCK_PINS, ids=lambda p: p.__name__)
def test_block_table_oracle_meets_pin(pin):
    pin(oracle.sort_candidate_blocks)


def test_bf16_oracle_limits():
    with pytest.raises(ValueError):
        oracle.topk_bf16(np.zeros((1, 16385), np.uint16), None, 8)
    with pytest.raises(ValueError):
        oracle.topk_bf16(np.zeros((1, 64), np.uint16), None, 2049)
    with pytest.raises(ValueError):
        oracle.topk_bf16(np.zeros((1, 64), np.float32), None, 8)


# ----------------------------------------------------------------------------
# planted mistakes: each must fail some pin
# ----------------------------------------------------------------------------

def bf16_mutant(mutation):
    def fn(bits, lengths, k, n_cols=None, page_table=None, page_size=0):
        u = bits.astype(np.uint32)
        if mutation == "fp16_decode":
            x = bits.view(np.float16).astype(np.float32)
        elif mutation == "shift_15":
            x = (u << np.uint32(15)).view(np.float32)
        elif mutation == "sign_magnitude_unsigned":  # raw patterns compared as unsigned ints
            x = u.astype(np.float32)
        else:
            x = (u << np.uint32(16)).view(np.float32)
        return oracle.topk(np.ascontiguousarray(x), lengths, k, n_cols=n_cols, page_table=page_table,
                           page_size=page_size)
    return fn


def amax_mutant(mutation):
    def fn(scores, lengths, topk, out, n_cols=None):
        n_cols = scores.shape[1] if n_cols is None else n_cols
        for b in range(scores.shape[0]):
            L = max(int(lengths[b]), 0)
            if mutation == "clamp_to_width":
                L = min(L, scores.shape[1])
            elif mutation != "no_upper_clamp":
                L = min(L, n_cols)
            nb = L // 8 if mutation == "floor_blocks" else -(-L // 8)
            if nb == 0 or (topk > 0 and (nb < topk if mutation == "skip_strict" else nb <= topk)):
                continue
            for i in range(nb - 1):
                blk = scores[b, 8 * i:8 * i + 8]
                if mutation == "nan_propagates":
                    v = np.float32(np.nan) if np.isnan(blk).any() else blk.max()
                elif mutation == "minus_zero_wins":
                    live = blk[~np.isnan(blk)]
                    v = live.max() if live.size else np.nan
                    v = np.float32(-0.0) if v == 0 else v
                else:
                    v = np.float32(ref_block(blk))
                out[b, i] = v
            out[b, nb - 1] = np.float32(np.inf) if mutation != "no_inf_newest" else \
                (np.float32(ref_block(scores[b, 8 * (nb - 1):L])) if L > 8 * (nb - 1) else out[b, nb - 1])
        return out
    return fn


def blocks_mutant(mutation):
    def fn(blocks, lengths, page_table, page_size, n_cols):
        bpp = page_size if mutation == "bpp_is_page_size" else page_size // 8
        B, k = blocks.shape
        table = np.full((B, k), INT32_MAX, np.int32)
        pages = np.full((B, k), INT32_MAX, np.int32)
        for b in range(B):
            L = max(int(lengths[b]), 0)
            L = L if mutation == "no_upper_clamp" else min(L, n_cols + 8 if mutation == "clamp_one_block_late" else n_cols)
            nb = -(-L // 8)
            ident = nb < k if mutation == "identity_strict" else nb <= k
            if ident:
                ids = list(range(nb))
            else:
                ids = sorted(set(int(v) for v in blocks[b] if (mutation == "keep_minus_one" or v >= 0) and v < nb))
            if mutation == "descending":
                ids = ids[::-1]
            for j, i in enumerate(ids):
                table[b, j] = i
                pages[b, j] = page_table[b, i // bpp] * bpp + i % bpp
        return table, pages
    return fn


def caught_by(pins, fn):
    caught = []
    for pin in pins:
        try:
            pin(fn)
        except (AssertionError, IndexError, ValueError, KeyError):
            caught.append(pin.__name__)
    return caught


def test_unmutated_statements_meet_the_pins():
    assert not caught_by(BF16_PINS, bf16_mutant(None))
    assert not caught_by(AMAX_PINS, amax_mutant(None))
    assert not caught_by(BLOCK_PINS, blocks_mutant(None))


@pytest.mark.parametrize("mutation", ["fp16_decode", "shift_15", "sign_magnitude_unsigned"])
def test_bf16_pins_reject_planted_mistakes(mutation):
    assert caught_by(BF16_PINS, bf16_mutant(mutation))


@pytest.mark.parametrize("mutation", ["floor_blocks", "skip_strict", "nan_propagates", "minus_zero_wins",
                                      "no_inf_newest", "no_upper_clamp", "clamp_to_width"])
def test_amax8_pins_reject_planted_mistakes(mutation):
    assert caught_by(AMAX_PINS, amax_mutant(mutation))


@pytest.mark.parametrize("mutation", ["bpp_is_page_size", "identity_strict", "keep_minus_one", "descending",
                                      "no_upper_clamp", "clamp_one_block_late"])
def test_block_table_pins_reject_planted_mistakes(mutation):
    assert caught_by(BLOCK_PINS, blocks_mutant(mutation))
