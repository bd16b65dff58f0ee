"""Pins for the CPU oracle, against things other than the oracle itself.

The pages print no worked example of a selection, so every expected value here
is fixed by mathematics: brute force over every subset of tiny rows, closed
forms (empty, short, ascending, descending, constant, -inf-padded, signed-zero,
single-bin and planted rows, paged identity), and library sorts (numpy, torch)
on rows without signed zeros. Each pin is a function of an oracle callable, so
``test_pins_reject_planted_mistakes`` can run the same pins against copies of
the oracle with one plausible mistake planted and show that some pin fails.

Definition under test: "dsv4.1: Top-k kernels and candidate selection", code
excerpts (bf16 top-k docstring) and "Fix incorrect sparse-attention top-k
selection when candidate bins overflow", comment thread (exact value
multisets, swaps only among equal scores); readings: +0 ranks above -0, ties
by lower index, lengths clamped to [0, n_cols].
"""
from __future__ import annotations

import itertools
import math

import numpy as np
import pytest
import torch

import oracle
import synth

ALPHABET = np.array([-np.inf, -1.0, -0.0, 0.0, 1e-45, 1.0, 65536.0, 70000.0, np.inf], dtype=np.float32)


def c_oracle(scores, lengths, k, n_cols=None, page_table=None, page_size=0):
    return oracle.topk(scores, lengths, k, n_cols=n_cols, page_table=page_table, page_size=page_size)


def rank_tuple(v: float):
    """Independent statement of the order: value, then +0 above -0."""
    return (float(v), not math.copysign(1.0, float(v)) < 0)


# ----------------------------------------------------------------------------
# pins
# ----------------------------------------------------------------------------

def pin_brute_force(fn, seed=11, cases=300):
    """Every m-subset of tiny rows; the oracle's must be valid and canonical."""
    rng = np.random.default_rng(seed)
    for _ in range(cases):
        L = int(rng.integers(0, 9))
        k = int(rng.integers(1, L + 3))
        W = L + int(rng.integers(0, 3))
        row = np.full((1, max(W, 1)), np.nan, dtype=np.float32)
        row[0, :L] = rng.choice(ALPHABET, L)
        got = fn(row, np.array([L], np.int32), k, n_cols=max(W, 1))[0]
        m = min(k, L)
        valid = []
        keys = [rank_tuple(v) for v in row[0, :L]]
        for sub in itertools.combinations(range(L), m):
            rest = [i for i in range(L) if i not in sub]
            if not sub or not rest or min(keys[i] for i in sub) >= max(keys[i] for i in rest):
                valid.append(sub)
        multisets = {tuple(sorted(row[0, list(s)].view(np.uint32).tolist())) for s in valid}
        assert len(multisets) == 1, "all valid answers must share one bit multiset"
        assert list(got[m:]) == [-1] * (k - m)
        chosen = tuple(sorted(got[:m].tolist()))
        assert chosen in valid, (row, k, got)
        assert chosen == min(tuple(sorted(s)) for s in valid), "ties must go to the lowest indices"


def pin_pairwise_invariant(fn, seed=17, cases=40):
    """Rows up to 512 from small alphabets: every selected value ranks at or
    above every unselected one, no index repeats, exactly m are selected and
    ties at the cutoff go to the lowest indices (O(L^2) pair checks)."""
    rng = np.random.default_rng(seed)
    for _ in range(cases):
        L = int(rng.integers(1, 513))
        k = int(rng.integers(1, 600))
        alpha = ALPHABET[rng.choice(len(ALPHABET), int(rng.integers(2, len(ALPHABET) + 1)), replace=False)]
        row = np.full((1, L + 3), np.nan, np.float32)
        row[0, :L] = rng.choice(alpha, L)
        got = fn(row, np.array([L], np.int32), k, n_cols=L)[0]
        m = min(k, L)
        sel = got[:m]
        assert np.all(got[m:] == -1) and len(set(sel.tolist())) == m
        assert np.all((sel >= 0) & (sel < L))
        keys = [rank_tuple(v) for v in row[0, :L]]
        chosen = np.zeros(L, bool)
        chosen[sel] = True
        worst = min(keys[i] for i in sel)
        for i in range(L):
            if not chosen[i]:
                assert keys[i] <= worst, "an unselected value ranks above a selected one"
                if keys[i] == worst:
                    assert all(j < i for j in sel if keys[j] == worst), "ties must go to the lowest indices"


def pin_library_sort(fn, seed=12):
    """Sorted selected values equal numpy's and torch's sorts (no signed zeros)."""
    rng = np.random.default_rng(seed)
    for L, k, W in [(1000, 37, 1000), (1000, 1000, 1000), (513, 600, 700), (2048, 2048, 2048), (4096, 512, 4100)]:
        x = np.full((3, W), np.nan, dtype=np.float32)
        x[0, :L] = rng.standard_normal(L).astype(np.float32)
        x[1, :L] = rng.integers(-20, 20, L).astype(np.float32) + 0.5       # heavy ties, no zero
        x[2, :L] = np.where(rng.random(L) < 0.3, -np.inf, rng.standard_normal(L) * 1e5).astype(np.float32)
        lengths = np.full(3, L, np.int32)
        got = fn(x, lengths, k, n_cols=W)
        m = min(k, L)
        for b in range(3):
            sel = np.sort(x[b, got[b, :m]])[::-1]
            ref = np.sort(x[b, :L])[::-1][:m]
            assert np.array_equal(sel, ref)
            tv = torch.topk(torch.from_numpy(x[b, :L].copy()), m).values.numpy()
            assert np.array_equal(sel, tv)


def pin_closed_forms(fn):
    W, k = 300, 64
    # empty, negative and over-long lengths
    x = np.random.default_rng(13).standard_normal((4, W)).astype(np.float32)
    got = fn(x, np.array([0, -1, -1000, W + 17], np.int32), k, n_cols=W)
    assert np.all(got[:3] == -1)
    assert np.array_equal(np.sort(got[3]), np.sort(np.argsort(-x[3], kind="stable")[:k]))
    # a length past n_cols stops at n_cols even when the row stride holds more
    wide = np.full((2, W + 50), 1e30, np.float32)
    wide[:, :W] = x[0]
    got = fn(wide, np.array([W + 17, W], np.int32), k, n_cols=W)
    assert np.array_equal(np.sort(got[0]), np.sort(got[1])) and got.max() < W
    # short rows: every position, then -1
    for L in (1, k - 1, k):
        got = fn(x, np.full(4, L, np.int32), k, n_cols=W)
        assert np.array_equal(np.sort(got[0, :L]), np.arange(L)) and np.all(got[0, L:] == -1)
    # ascending / descending / constant
    L = 250
    rows = np.stack([np.arange(W), W - np.arange(W), np.full(W, 3.25)]).astype(np.float32)
    got = fn(rows, np.full(3, L, np.int32), k, n_cols=W)
    assert set(got[0].tolist()) == set(range(L - k, L))
    assert set(got[1].tolist()) == set(range(k))
    assert set(got[2].tolist()) == set(range(k))
    # F finite values, the rest -inf: all finite ones plus the lowest -inf ones
    F = 10
    row = np.full((1, W), -np.inf, np.float32)
    fin = np.array([5, 77, 120, 121, 122, 200, 250, 251, 280, 299])
    row[0, fin] = np.arange(F, dtype=np.float32)
    got = fn(row, np.array([W], np.int32), k, n_cols=W)[0]
    others = [i for i in range(W) if i not in set(fin.tolist())][: k - F]
    assert set(got.tolist()) == set(fin.tolist()) | set(others)
    # signed zeros: positives, then +0 (lowest first), then -0 (lowest first)
    rng = np.random.default_rng(14)
    row = np.where(rng.random(W) < 0.5, 0.0, -0.0).astype(np.float32)[None, :]
    pos = rng.choice(W, 20, replace=False)
    row[0, pos] = 1.5
    neg = np.setdiff1d(np.arange(W), pos)[:30]
    row[0, neg] = -2.0
    got = fn(row, np.array([W], np.int32), k, n_cols=W)[0]
    bits = row[0].view(np.uint32)
    plus0 = [i for i in range(W) if bits[i] == 0]
    minus0 = [i for i in range(W) if bits[i] == 0x80000000]
    need = k - 20
    expect = set(pos.tolist()) | set(plus0[:need]) | set(minus0[: max(0, need - len(plus0))])
    assert set(got.tolist()) == expect
    # one coarse bin: 0x3F800000 + r -- counting sort over r gives the answer
    r = rng.integers(0, 64, 2000)
    row = (0x3F800000 + r).astype(np.uint32).view(np.float32)[None, :]
    got = fn(row, np.array([2000], np.int32), 500, n_cols=2000)[0]
    counts = np.bincount(r, minlength=64)
    expect_r = []
    for v in range(63, -1, -1):
        expect_r += [v] * counts[v]
    expect_r = expect_r[:500]
    assert sorted(r[got].tolist()) == sorted(expect_r)
    cut = expect_r[-1]
    ties = [i for i in range(2000) if r[i] == cut][: expect_r.count(cut)]
    assert set(got.tolist()) == set(np.flatnonzero(r > cut).tolist()) | set(ties)
    # planted winners above a clipped background
    bg = np.clip(rng.standard_normal(5000), -5, 4.9).astype(np.float32)[None, :]
    win = rng.choice(5000, 333, replace=False)
    bg[0, win] = rng.uniform(6, 7, 333).astype(np.float32)
    got = fn(bg, np.array([5000], np.int32), 333, n_cols=5000)[0]
    assert set(got.tolist()) == set(win.tolist())
    # above the fp16 maximum: 70000 + j at permuted positions
    perm = rng.permutation(3000)
    row = np.empty((1, 3000), np.float32)
    row[0, perm] = 70000.0 + np.arange(3000)
    got = fn(row, np.array([3000], np.int32), 100, n_cols=3000)[0]
    assert set(got.tolist()) == set(perm[2900:].tolist())


def pin_paged(fn):
    """Paged output is the raw answer pushed through the row's page table."""
    rng = np.random.default_rng(15)
    W, k, ps = 1000, 70, 8
    pages = -(-W // ps)
    rows = np.tile(np.arange(W, dtype=np.float32), (3, 1))
    pt = np.stack([rng.permutation(pages) + 1000 * b for b in range(3)]).astype(np.int32)
    lengths = np.array([W, 500, 10], np.int32)
    got = fn(rows, lengths, k, n_cols=W, page_table=pt, page_size=ps)
    for b, L in enumerate(lengths):
        m = min(k, int(L))
        raw = np.arange(L - m, L)
        expect = pt[b, raw // ps] * ps + raw % ps
        assert set(got[b, :m].tolist()) == set(expect.tolist())
        assert np.all(got[b, m:] == -1)


ALL_PINS = [pin_brute_force, pin_pairwise_invariant, pin_library_sort, pin_closed_forms, pin_paged]


# ----------------------------------------------------------------------------
# the oracle against its pins
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_meets_pin(pin):
    pin(c_oracle)


def test_oracle_reads_only_valid_prefix():
    W = 64
    x = np.full((2, W), np.nan, np.float32)
    x[:, :10] = np.arange(10, dtype=np.float32)
    got = oracle.topk(x, np.array([10, 3], np.int32), 4)
    assert set(got[0].tolist()) == {6, 7, 8, 9}
    assert sorted(got[1, :3].tolist()) == [0, 1, 2] and got[1, 3] == -1
    with pytest.raises(ValueError):
        oracle.topk(x, np.array([11, 3], np.int32), 4)


def test_oracle_row_stride_and_offset_views():
    rng = np.random.default_rng(16)
    big = rng.standard_normal((5, 512)).astype(np.float32)
    view = big[1:4, 8:300]            # base offset and row stride 512 > n_cols
    got = oracle.topk(view, None, 20)
    dense = np.ascontiguousarray(view)
    assert np.array_equal(got, oracle.topk(dense, None, 20))


def test_oracle_threads_do_not_change_result():
    wl = synth.c2(1024, width=4096, rows_per_kind=1)
    one = oracle.topk(wl.scores, wl.lengths, wl.k, threads=1)
    many = oracle.topk(wl.scores, wl.lengths, wl.k, threads=4)
    assert np.array_equal(one, many)


# ----------------------------------------------------------------------------
# the pins against planted mistakes (each must be caught)
# ----------------------------------------------------------------------------

def py_oracle(scores, lengths, k, n_cols=None, page_table=None, page_size=0, mutation=None):
    """A Python statement of the oracle's definition with an optional planted bug."""
    B = scores.shape[0]
    n_cols = scores.shape[1] if n_cols is None else n_cols
    out = np.full((B, k), -1, np.int32)
    for b in range(B):
        L = n_cols if lengths is None else int(lengths[b])
        if mutation != "no_upper_clamp":
            L = min(L, n_cols)
        L = max(L, 0)
        m = min(k, L) if mutation != "m_minus_one" else max(min(k, L) - 1, 0)
        x = scores[b, :L]

        def key(i):
            v = float(x[i])
            if mutation == "fp16_key":
                with np.errstate(over="ignore"):
                    v = float(np.float16(v))
            zero_rank = 0 if mutation == "no_signed_zero" else (1 if math.copysign(1.0, v) < 0 else 0)
            tie = -i if mutation == "ties_high_index" else i
            return (-v, zero_rank, tie)

        idx = sorted(range(L), key=key)
        if mutation == "drop_neginf":
            idx = [i for i in idx if x[i] != -np.inf]
        sel = idx[:m]
        for j, i in enumerate(sel):
            if page_table is None:
                out[b, j] = i
            else:
                row = 0 if mutation == "page_row_zero" else b
                out[b, j] = page_table[row, i // page_size] * page_size + i % page_size
    return out


MUTATIONS = ["ties_high_index", "no_signed_zero", "fp16_key", "drop_neginf",
             "m_minus_one", "no_upper_clamp", "page_row_zero"]


def test_python_statement_agrees_with_oracle():
    for pin in (pin_brute_force, pin_pairwise_invariant, pin_closed_forms, pin_paged):
        pin(py_oracle)
    wl = synth.c2(512, width=2048, rows_per_kind=1)
    assert np.array_equal(py_oracle(wl.scores, wl.lengths, wl.k), oracle.topk(wl.scores, wl.lengths, wl.k))


@pytest.mark.parametrize("mutation", MUTATIONS)
def test_pins_reject_planted_mistakes(mutation):
    def broken(*a, **kw):
        return py_oracle(*a, mutation=mutation, **kw)

    caught = []
    for pin in ALL_PINS:
        try:
            pin(broken)
        except (AssertionError, IndexError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {mutation!r}"
