"""Acceptance predicates for a top-k result against the oracle's, row by row.

Checks, after "[Bug]: persistent_topk silently drops top-k candidates when many
values share a coarse histogram bin" (verification: gather the selected
scores, sort, compare value by value with no tolerance), vLLM PR #56346 report
(implementation items 4-5: -1 on invalid slots, no duplicate indices, exact
equality) and "dsv4.1: Top-k kernels and candidate selection" (tests section:
count, range, uniqueness and value set):

A1  slot j holds -1 exactly when j >= m = min(k, clamp(length, 0, n_cols));
A2  the first m slots are distinct positions in [0, L) (paged: distinct slots
    that invert through the row's page table to such positions);
A3  the selected scores equal the oracle's as a multiset of bit patterns;
A6  the selected positions equal the oracle's (the oracle takes the lowest
    indices among ties at the cutoff; so does the GPU path by design).
"""
from __future__ import annotations

import numpy as np


def clamp_len(lengths, n_cols):
    return np.clip(np.asarray(lengths, dtype=np.int64), 0, n_cols)


def invert_pages(got_row: np.ndarray, page_row: np.ndarray, page_size: int):
    """Map page-table slots back to raw positions; None where a slot is foreign."""
    inv = {int(p): j for j, p in enumerate(page_row)}
    out = np.empty(got_row.shape, dtype=np.int64)
    for t, s in enumerate(got_row):
        s = int(s)
        j = inv.get(s // page_size)
        if j is None or s < 0:
            return None
        out[t] = j * page_size + s % page_size
    return out


def check(scores, lengths, n_cols, k, got, want, *, page_table=None, page_size=0,
          require_same_set=True, rows=None, max_report=5):
    """Return a list of failure strings (empty when every checked row passes)."""
    got = np.asarray(got)
    want = np.asarray(want)
    bits = scores.view(np.uint32)
    L_all = clamp_len(lengths if lengths is not None else np.full(scores.shape[0], n_cols), n_cols)
    rows = range(scores.shape[0]) if rows is None else rows
    fails = []
    for b in rows:
        if len(fails) >= max_report:
            break
        L = int(L_all[b])
        m = min(k, L)
        g = got[b]
        w = want[b]
        if not (np.all(g[m:] == -1) and np.all(g[:m] != -1)):
            fails.append(f"row {b}: A1 -1 slots wrong (m={m}, got {np.count_nonzero(g != -1)} filled)")
            continue
        gm, wm = g[:m].astype(np.int64), w[:m].astype(np.int64)
        if page_table is not None:
            gr = invert_pages(gm, page_table[b], page_size)
            wr = invert_pages(wm, page_table[b], page_size)
            if gr is None:
                fails.append(f"row {b}: A2 slot not in the row's page table")
                continue
            gm, wm = gr, wr
        if gm.size and (gm.min() < 0 or gm.max() >= L):
            fails.append(f"row {b}: A2 index out of [0, {L})")
            continue
        if np.unique(gm).size != gm.size:
            fails.append(f"row {b}: A2 duplicate indices")
            continue
        gv = np.sort(bits[b, gm])
        wv = np.sort(bits[b, wm])
        if not np.array_equal(gv, wv):
            nd = int(np.count_nonzero(gv != wv))
            fails.append(f"row {b}: A3 value multiset differs ({nd} of {m} sorted entries)")
            continue
        if require_same_set and not np.array_equal(np.sort(gm), np.sort(wm)):
            fails.append(f"row {b}: A6 index set differs from the oracle's lowest-index ties")
    return fails


def check_fast_raw(got, want, lengths, n_cols, k):
    """Vectorised A1 + A6 for raw outputs: equal index sets per row.

    Equal index sets imply equal value multisets, so this subsumes A2/A3 when
    the oracle's output is itself valid (the oracle tests pin that).
    """
    L = clamp_len(lengths, n_cols)
    m = np.minimum(L, k)
    slot = np.arange(k)[None, :]
    a1 = np.all((got == -1) == (slot >= m[:, None]), axis=1)
    same = np.all(np.sort(got, axis=1) == np.sort(want, axis=1), axis=1)
    bad = np.flatnonzero(~(a1 & same))
    return [int(b) for b in bad]


def check_codes(stats, lengths, n_cols, k, force, cap):
    """Each row's path code (row_stats[b, 0]) is one its forced path allows:
    direct rows (L <= k) 0, or 1 when L > 0; full-row forced 6; LDS forced 2
    up to the capacity, else 6; sampled 3, or 4/5 after an overflow or
    underflow fallback; automatic 2 up to the capacity, else 3/4/5. The
    second word is L wherever no stream ran. Returns the failures."""
    fails = []
    L = np.clip(np.asarray(lengths, np.int64), 0, n_cols)
    for b in range(L.size):
        code, seen = int(stats[b, 0]), int(stats[b, 1])
        if L[b] <= k:
            ok = {0 if L[b] == 0 else 1}
        elif force == 3 or (force == 1 and L[b] > cap):
            ok = {6}
        elif force == 1 or (force == 0 and L[b] <= cap):
            ok = {2}
        else:
            ok = {3, 4, 5}
        if code not in ok:
            fails.append(f"row {b}: L={L[b]} force={force} cap={cap}: code {code}, allowed {sorted(ok)}")
        elif code in (0, 1, 2, 6) and seen != L[b]:
            fails.append(f"row {b}: code {code} reports {seen}, L={L[b]}")
    return fails
