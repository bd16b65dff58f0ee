"""The checker must reject what a broken selection looks like.

Failure signatures from "[Bug]: persistent_topk silently drops top-k
candidates when many values share a coarse histogram bin" (caveats and cause
analysis: values silently replaced by smaller ones, no -1 and no duplicate to
show it) and the checks of "dsv4.1: Top-k kernels and candidate selection"
(tests section: count, range, uniqueness, value set): each mutation of a
correct output below must be reported.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from topk_check import check, check_fast_raw


@pytest.fixture(scope="module")
def case():
    wl = synth.mixed_rows(["normal", "heavy_ties", "signed_zero", "ascending"], 3000, 200, seed=91)
    wl.lengths = np.array([3000, 2500, 150, 3000], np.int32)
    synth.poison_tails(wl.scores, wl.lengths)
    return wl, oracle.topk(wl.scores, wl.lengths, wl.k)


def mutate(want, wl, kind):
    got = want.copy()
    L0 = int(wl.lengths[0])
    chosen = set(got[0, :200].tolist())
    order = np.argsort(-wl.scores[0, :L0], kind="stable")
    worse = next(int(i) for i in order[::-1] if int(i) not in chosen)  # a strictly smaller value
    if kind == "dropped_value":
        got[0, 5] = worse
    elif kind == "duplicate":
        got[0, 7] = got[0, 8]
    elif kind == "minus_one_inside":
        got[0, 3] = -1
    elif kind == "filled_past_m":
        got[2, 160] = 0  # row 2 has m = 150
    elif kind == "out_of_range":
        got[1, 0] = 2600  # past row 1's length
    elif kind == "tie_from_the_wrong_end":
        # among equal values, a higher index than the oracle's
        row = wl.scores[1, :2500]
        cut = row[got[1, 199]]
        ties = [i for i in range(2500) if row[i] == cut and i not in set(got[1, :200].tolist())]
        got[1, 199] = ties[-1]
    return got


@pytest.mark.parametrize("kind", ["dropped_value", "duplicate", "minus_one_inside", "filled_past_m",
                                  "out_of_range", "tie_from_the_wrong_end"])
def test_checker_rejects(case, kind):
    wl, want = case
    got = mutate(want, wl, kind)
    assert check(wl.scores, wl.lengths, wl.n_cols, wl.k, got, want)
    assert check_fast_raw(got, want, wl.lengths, wl.n_cols, wl.k)


def test_checker_accepts_a_reordering(case):
    wl, want = case
    rng = np.random.default_rng(92)
    got = want.copy()
    for b in range(wl.batch):
        m = min(wl.k, int(wl.lengths[b]))
        got[b, :m] = rng.permutation(got[b, :m])
    assert not check(wl.scores, wl.lengths, wl.n_cols, wl.k, got, want)
    assert not check_fast_raw(got, want, wl.lengths, wl.n_cols, wl.k)


def test_checker_rejects_a_wrong_page_slot():
    wl = synth.c5(batch=8, width=4096, k=128, page_size=64)
    want = oracle.topk(wl.scores, wl.lengths, wl.k, page_table=wl.page_table, page_size=wl.page_size)
    b = next(i for i in range(wl.batch) if min(wl.k, int(wl.lengths[i])) > 1)
    got = want.copy()
    got[b, 0] = got[b, 0] + 64 * 1000  # a page slot no page of the row maps to
    assert check(wl.scores, wl.lengths, wl.n_cols, wl.k, got, want, page_table=wl.page_table,
                 page_size=wl.page_size)
