"""Seeded synthetic score rows for exact per-row top-k.

The one module that both the CPU oracle's tests and the GPU path's tests and
bench draw their inputs from. It holds no part of the selection itself: it only
fills float32 rows, lengths and page tables from seeded numpy generators
(``numpy.random.default_rng``, PCG64). Positions at or past a row's length are
poisoned with quiet NaN, which would rank first if any reader touched them.

Workload shapes follow the pages' measurements:

* decode batches of B=1024 rows at widths 128K and 256K with lengths uniform
  in 80-100 % of the width, k=2048 and k=512 -- vLLM PR #56346 report,
  summary and implementation item 5 (bench with ragged lengths);
* adversarial rows where many values share one coarse bin, values above the
  fp16 maximum 65504, -inf entries, signed zeros, ties, constant and
  ascending rows -- "[Bug]: persistent_topk silently drops top-k candidates
  when many values share a coarse histogram bin", cause analysis; vLLM PR
  #56346 report, implementation item 4 (random, 10LSBits, ascending, constant
  and sampled-peaks distributions); "Fix incorrect sparse-attention top-k
  selection when candidate bins overflow", comment thread (signed zero,
  permutations, offsets, idle rows, all-equal oversized bins);
* paged output with page_size 64 -- "dsv4.1: Top-k kernels and candidate
  selection", code excerpts (page-table transform) and tests section
  (page_size sweep).
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass, field

import numpy as np

POISON_BITS = 0x7FC00000  # +quiet NaN
FP16_MAX = 65504.0


@dataclass
class Workload:
    name: str
    seed: int
    scores: np.ndarray            # float32 [batch, row_stride]
    lengths: np.ndarray           # int32 [batch]
    n_cols: int
    k: int
    page_table: np.ndarray | None = None   # int32 [batch, pages]
    page_size: int = 0
    kinds: list = field(default_factory=list)  # per-row kind names, when mixed

    @property
    def batch(self) -> int:
        return self.scores.shape[0]

    def read_bytes(self) -> int:
        """Score bytes the selection must read: 4 per valid position."""
        L = np.clip(self.lengths.astype(np.int64), 0, self.n_cols)
        return int(4 * L.sum())


def _rng(seed, *more):
    return np.random.default_rng(np.random.SeedSequence([seed, *more]))


def poison_tails(scores: np.ndarray, lengths: np.ndarray) -> None:
    """Write quiet NaN into every position at or past a row's length."""
    bits = scores.view(np.uint32)
    for b, L in enumerate(np.asarray(lengths)):
        L = max(int(L), 0)
        if L < scores.shape[1]:
            bits[b, L:] = POISON_BITS


def _from_bits(u) -> np.ndarray:
    return np.asarray(u, dtype=np.uint32).view(np.float32)


# ----------------------------------------------------------------------------
# adversarial row kinds (width W, k), each a float32 row of W valid scores
# ----------------------------------------------------------------------------

def _kind_onebin(rng, W, k):
    # [1.0, 1.0 + 2^-10): 8192 distinct float32 patterns, one fp16 bin
    return _from_bits(0x3F800000 + rng.integers(0, 8192, W))


def _crowd(rng, W, n, base_bits, span):
    x = rng.standard_normal(W, dtype=np.float32)
    pos = rng.choice(W, size=min(n, W), replace=False)
    x[pos] = _from_bits(base_bits + rng.integers(0, span, pos.size))
    return x


def _kind_crowd4096(rng, W, k):
    return _crowd(rng, W, 4096, 0x40000000, 8192)       # [2, 2 + 2^-9)


def _kind_crowd16385(rng, W, k):
    return _crowd(rng, W, 16385, 0x40000000, 8192)      # [2, 2 + 2^-9)


def _kind_crowd16385_top(rng, W, k):
    return _crowd(rng, W, 16385, 0x40800000, 8192)      # [4, 4 + 2^-8)


def _kind_above_fp16(rng, W, k):
    x = (rng.standard_normal(W) * 10.0).astype(np.float32)
    perm = rng.permutation(W)
    a, b = W // 2, (3 * W) // 4
    x[perm[:a]] = (70000.0 + np.arange(a)).astype(np.float32)
    x[perm[a:b]] = np.exp(rng.uniform(np.log(65536.0), np.log(3.0e38), b - a)).astype(np.float32)
    x[perm[b:b + 8]] = np.inf
    x[perm[b + 8:b + 16]] = (FP16_MAX + rng.uniform(0.5, 15.5, 8)).astype(np.float32)
    return x


def _kind_neginf_half(rng, W, k):
    x = rng.standard_normal(W, dtype=np.float32)
    x[rng.random(W) < 0.5] = -np.inf
    return x


def _kind_neginf_few_finite(rng, W, k):
    x = np.full(W, -np.inf, dtype=np.float32)
    pos = rng.choice(W, size=max(k // 2, 1), replace=False)
    x[pos] = rng.standard_normal(pos.size, dtype=np.float32)
    return x


def _kind_signed_zero(rng, W, k):
    x = np.where(rng.random(W) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
    perm = rng.permutation(W)
    P = max(k // 4, 1)
    x[perm[:P]] = rng.uniform(0.5, 2.0, P).astype(np.float32)
    x[perm[P:2 * P]] = -rng.uniform(0.5, 2.0, P).astype(np.float32)
    return x


def _kind_heavy_ties(rng, W, k):
    return rng.integers(0, 16, W).astype(np.float32)


def _kind_constant(rng, W, k):
    return np.full(W, np.float32(rng.standard_normal()), dtype=np.float32)


def _kind_ascending(rng, W, k):
    return np.arange(W, dtype=np.float32)


def _kind_descending(rng, W, k):
    return (W - np.arange(W)).astype(np.float32)


def _kind_clustered_peaks(rng, W, k):
    # k peaks in one contiguous window: a sparse sample can miss all of them
    x = rng.standard_normal(W, dtype=np.float32)
    n = min(k, W)
    start = int(rng.integers(0, W - n + 1))
    x[start:start + n] = (6.0 + rng.standard_normal(n)).astype(np.float32)
    return x


def _kind_periodic_peaks(rng, W, k):
    x = rng.standard_normal(W, dtype=np.float32)
    off = int(rng.integers(0, 16))
    x[off::16] += np.float32(6.0)
    return x


def _kind_subnormal(rng, W, k):
    mag = rng.integers(1, 0x00800000, W).astype(np.uint32)
    sign = (rng.random(W) < 0.5).astype(np.uint32) << np.uint32(31)
    x = _from_bits(mag | sign).copy()
    r = rng.random(W)
    x[r < 0.1] = np.float32(0.0)
    x[(r >= 0.1) & (r < 0.2)] = np.float32(-0.0)
    tiny = (r >= 0.2) & (r < 0.25)
    x[tiny] = _from_bits(0x00800000 + rng.integers(0, 1 << 20, int(tiny.sum())))
    return x


def _kind_lowbits10(rng, W, k):
    # patterns that differ only in their 10 low bits
    return _from_bits(0x3F800000 | rng.integers(0, 1024, W))


def _kind_normal(rng, W, k):
    return rng.standard_normal(W, dtype=np.float32)


ROW_KINDS = {
    "onebin": _kind_onebin,
    "crowd4096": _kind_crowd4096,
    "crowd16385": _kind_crowd16385,
    "crowd16385_top": _kind_crowd16385_top,
    "above_fp16": _kind_above_fp16,
    "neginf_half": _kind_neginf_half,
    "neginf_few_finite": _kind_neginf_few_finite,
    "signed_zero": _kind_signed_zero,
    "heavy_ties": _kind_heavy_ties,
    "constant": _kind_constant,
    "ascending": _kind_ascending,
    "descending": _kind_descending,
    "clustered_peaks": _kind_clustered_peaks,
    "periodic_peaks": _kind_periodic_peaks,
    "subnormal": _kind_subnormal,
    "lowbits10": _kind_lowbits10,
    "normal": _kind_normal,
}


def row_of_kind(kind: str, W: int, k: int, seed: int, row: int = 0) -> np.ndarray:
    return ROW_KINDS[kind](_rng(seed, row, zlib.crc32(kind.encode())), W, k)


def mixed_rows(kinds, W: int, k: int, seed: int, *, row_stride: int | None = None,
               lengths=None, name: str = "mixed") -> Workload:
    """One row per entry of ``kinds``; every row full length unless given."""
    B = len(kinds)
    stride = row_stride or W
    scores = np.empty((B, stride), dtype=np.float32)
    for b, kind in enumerate(kinds):
        scores[b, :W] = row_of_kind(kind, W, k, seed, b)
    if lengths is None:
        lengths = np.full(B, W, dtype=np.int32)
    lengths = np.asarray(lengths, dtype=np.int32)
    poison_tails(scores, lengths)
    return Workload(name, seed, scores, lengths, W, k, kinds=list(kinds))


def cutoff_group_rows(group: int, kind: str, batch: int = 4, width: int = 16384, k: int = 512,
                      seed: int = 43) -> Workload:
    """Rows whose k-th largest score falls inside a group of ``group`` scores
    that nothing else comes near: k - 17 distinct scores well above it, the
    group, and a background well below, so 17 of the group are selected.
    ``kind`` "ties": the group is one value repeated; "cluster": the group is
    ``group`` consecutive fp32 patterns (distinct values closer together than
    any coarse bin). Even rows: N(0,1) background, the group at +32, the
    scores above from +64 up; odd rows: background below -2, the group at -1,
    the scores above from +1 up. Every fourth row pair is ragged. (The exact
    capacity boundaries the sparse-attention top-k fix thread found bugs at,
    applied to each finisher's direct-ranking limit.)"""
    rng = _rng(seed, group, zlib.crc32(kind.encode()))
    above = k - 17
    scores = np.empty((batch, width), np.float32)
    lengths = np.full(batch, width, np.int32)
    for b in range(batch):
        if b % 2 == 0:
            row = np.clip(rng.standard_normal(width, dtype=np.float32), -31.0, 31.0)
            g0, top0 = 0x42000000, 0x42800000
        else:
            row = (-2.0 - np.abs(rng.standard_normal(width))).astype(np.float32)
            g0, top0 = 0xBF800000, 0x3F800000
        if b % 4 >= 2:
            lengths[b] = width - 1 - int(rng.integers(0, 64))
        L = int(lengths[b])
        pos = rng.permutation(L)[:above + group]
        row[pos[:above]] = _from_bits(top0 + (np.arange(above, dtype=np.uint32) << np.uint32(16)))
        if kind == "ties":
            g = np.full(group, g0, np.uint32)
        elif kind == "cluster":  # consecutive patterns; for the negative group larger bits are smaller values
            g = g0 + np.arange(group, dtype=np.uint32)
        else:
            raise ValueError(kind)
        row[pos[above:]] = _from_bits(g)
        scores[b] = row
    poison_tails(scores, lengths)
    return Workload(f"group{group}_{kind}_{batch}x{width}", seed, scores, lengths, width, k)


# ----------------------------------------------------------------------------
# the five named workloads
# ----------------------------------------------------------------------------

def c1() -> Workload:
    """8 rows x 4096, N(0,1), all full length, k=512, raw indices."""
    rng = np.random.default_rng(1)
    scores = rng.standard_normal((8, 4096), dtype=np.float32)
    lengths = np.full(8, 4096, dtype=np.int32)
    return Workload("c1_8x4096_k512", 1, scores, lengths, 4096, 512)


C2_KINDS = ["onebin", "crowd4096", "crowd16385", "crowd16385_top", "above_fp16",
            "neginf_half", "neginf_few_finite", "signed_zero", "heavy_ties",
            "constant", "ascending", "descending", "clustered_peaks",
            "periodic_peaks", "subnormal", "lowbits10"]


def c2(k: int, width: int = 32768, rows_per_kind: int = 4, seed: int = 2) -> Workload:
    """Adversarial rows: 16 kinds x 4 rows = 64 rows of 32768, full length."""
    kinds = [kd for kd in C2_KINDS for _ in range(rows_per_kind)]
    wl = mixed_rows(kinds, width, k, seed, name=f"c2_{len(kinds)}x{width}_k{k}")
    return wl


def ragged_lengths(rng, batch: int, width: int) -> np.ndarray:
    """Lengths uniform over the integers in [ceil(0.8 * width), width]."""
    lo = -(-8 * width // 10)
    return rng.integers(lo, width, size=batch, endpoint=True).astype(np.int32)


def c3(batch: int = 1024, width: int = 131072) -> Workload:
    """Decode batch: 1024 x 131072 N(0,1), lengths 80-100 % ragged, k=2048."""
    rng = np.random.default_rng(3)
    lengths = ragged_lengths(rng, batch, width)
    scores = rng.standard_normal((batch, width), dtype=np.float32)
    poison_tails(scores, lengths)
    return Workload(f"c3_{batch}x{width}_k2048", 3, scores, lengths, width, 2048)


def c4(batch: int = 1024, width: int = 262144) -> Workload:
    """Decode batch: 1024 x 262144 N(0,1) with sparse peaks, 80-100 % ragged, k=512.

    Each valid entry is, with probability 0.001, a peak that gets +N(6,1) added.
    """
    rng = np.random.default_rng(4)
    lengths = ragged_lengths(rng, batch, width)
    scores = rng.standard_normal((batch, width), dtype=np.float32)
    for b in range(batch):
        L = int(lengths[b])
        hit = np.flatnonzero(rng.random(L) < 0.001)
        scores[b, hit] += (6.0 + rng.standard_normal(hit.size)).astype(np.float32)
    poison_tails(scores, lengths)
    return Workload(f"c4_{batch}x{width}_k512", 4, scores, lengths, width, 512)


C5_CATEGORIES = ("zero", "one", "k_minus_1", "k", "k_plus_1", "uniform")


def c5(batch: int = 256, width: int = 65536, k: int = 1024, page_size: int = 64,
       global_pool: bool = False) -> Workload:
    """Paged output: 256 x 65536 N(0,1), k=1024, page_size=64.

    Lengths come from {0, 1, k-1, k, k+1, uniform[1, width]}, the first six
    rows covering each category once. Row b of the page table is a random
    permutation of its page slots (or, with ``global_pool``, the rows share one
    permutation of batch * pages distinct slots).
    """
    rng = np.random.default_rng(5)
    cats = np.concatenate([np.arange(6), rng.integers(0, 6, batch - 6)])[:batch]
    lengths = np.empty(batch, dtype=np.int32)
    fixed = {0: 0, 1: 1, 2: k - 1, 3: k, 4: k + 1}
    for b, c in enumerate(cats):
        lengths[b] = fixed[c] if c in fixed else rng.integers(1, width, endpoint=True)
    scores = rng.standard_normal((batch, width), dtype=np.float32)
    pages = -(-width // page_size)
    if global_pool:
        page_table = rng.permutation(batch * pages).astype(np.int32).reshape(batch, pages)
    else:
        page_table = np.stack([rng.permutation(pages) for _ in range(batch)]).astype(np.int32)
    poison_tails(scores, lengths)
    name = f"c5_{batch}x{width}_k{k}_ps{page_size}" + ("_pool" if global_pool else "")
    wl = Workload(name, 5, scores, lengths, width, k, page_table=page_table, page_size=page_size)
    wl.kinds = [C5_CATEGORIES[c] for c in cats]
    return wl


# ----------------------------------------------------------------------------
# bf16 rows and the two-level indexer's inputs
# ----------------------------------------------------------------------------

BF16_POISON = 0x7FC0  # bf16 +quiet NaN


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), rounded to nearest, ties to even;
    NaN becomes the quiet NaN 0x7FC0."""
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r[np.isnan(x)] = BF16_POISON
    return r


def poison_tails_bf16(bits: np.ndarray, lengths: np.ndarray) -> None:
    for b in range(bits.shape[0]):
        L = max(int(lengths[b]), 0)
        bits[b, L:] = BF16_POISON


@dataclass
class Bf16Workload:
    name: str
    seed: int
    bits: np.ndarray              # uint16 [batch, row_stride]
    lengths: np.ndarray           # int32 [batch]
    n_cols: int
    k: int
    page_table: np.ndarray | None = None
    page_size: int = 0

    @property
    def batch(self) -> int:
        return self.bits.shape[0]


def _page_table(rng, batch: int, width: int, page_size: int) -> np.ndarray:
    pages = -(-width // page_size)
    return np.stack([rng.permutation(pages) for _ in range(batch)]).astype(np.int32)


def bf16_rows(batch: int = 1024, width: int = 16384, k: int = 2048, seed: int = 6, *,
              paged: bool = True, page_size: int = 64) -> Bf16Workload:
    """The bf16 consumer rows of "dsv4.1: Top-k kernels and candidate selection"
    (implementation section 2: rows of at most 16384 scores, k at most 2048,
    page-table output): N(0,1) rounded to bf16, lengths uniform in 80-100 % of
    the width, a per-row permutation page table of page_size 64."""
    rng = np.random.default_rng(seed)
    lengths = ragged_lengths(rng, batch, width)
    bits = to_bf16_bits(rng.standard_normal((batch, width), dtype=np.float32))
    poison_tails_bf16(bits, lengths)
    pt = _page_table(rng, batch, width, page_size) if paged else None
    return Bf16Workload(f"bf16_{batch}x{width}_k{k}", seed, bits, lengths, width, k, pt,
                        page_size if paged else 0)


def bf16_adversarial(k: int, width: int = 16384, seed: int = 7, rows_per_kind: int = 2) -> Bf16Workload:
    """The adversarial fp32 row kinds, rounded to bf16: rounding merges many
    distinct values into one, so ties are heavier still."""
    kinds = [kd for kd in C2_KINDS for _ in range(rows_per_kind)]
    rows = np.stack([row_of_kind(kd, width, k, seed, b) for b, kd in enumerate(kinds)])
    bits = to_bf16_bits(rows)
    lengths = np.full(len(kinds), width, np.int32)
    return Bf16Workload(f"bf16_adv_{len(kinds)}x{width}_k{k}", seed, bits, lengths, width, k)


@dataclass
class Amax8Workload:
    name: str
    seed: int
    scores: np.ndarray            # float32 [batch, row_stride], row_stride % 8 == 0
    lengths: np.ndarray           # int32 [batch]
    out_blocks: int               # columns of the level-one key matrix
    topk: int

    @property
    def batch(self) -> int:
        return self.scores.shape[0]


def amax8_rows(batch: int = 1024, width: int = 131072, topk: int = 512, seed: int = 8, *,
               nan_rate: float = 0.0, zero_rate: float = 0.0) -> Amax8Workload:
    """Scores of the two-level indexer's first level ("dsv4.1: Top-k kernels and
    candidate selection", implementation section 2): N(0,1), lengths uniform in
    80-100 % of the width; optionally NaN (ignored by the block max) and signed
    zeros sprinkled inside the rows. Past each length: NaN poison."""
    rng = np.random.default_rng(seed)
    lengths = ragged_lengths(rng, batch, width)
    scores = rng.standard_normal((batch, width), dtype=np.float32)
    if nan_rate > 0:
        scores[rng.random(scores.shape) < nan_rate] = np.nan
    if zero_rate > 0:
        z = rng.random(scores.shape) < zero_rate
        scores[z] = np.where(rng.random(int(z.sum())) < 0.5, np.float32(0.0), np.float32(-0.0))
    poison_tails(scores, lengths)
    return Amax8Workload(f"amax8_{batch}x{width}", seed, scores, lengths, -(-width // 8), topk)


@dataclass
class BlockTableWorkload:
    name: str
    seed: int
    blocks: np.ndarray            # int32 [batch, k]: selected block ids, any order, -1 padded
    lengths: np.ndarray           # int32 [batch] token counts (blocks = ceil(L / 8))
    page_table: np.ndarray        # int32 [batch, pages]
    page_size: int

    @property
    def batch(self) -> int:
        return self.blocks.shape[0]


def candidate_blocks(batch: int = 1024, width: int = 131072, k: int = 512, seed: int = 9, *,
                     page_size: int = 64, short_rows: bool = True) -> BlockTableWorkload:
    """Selected block ids as a top-k over level-one keys leaves them: k distinct
    ids of [0, ceil(L / 8)) in random order; rows with at most k blocks hold
    whatever (the identity table applies). Page table: a per-row permutation."""
    rng = np.random.default_rng(seed)
    lengths = ragged_lengths(rng, batch, width)
    if short_rows:  # some rows with at most k blocks, and idle rows
        pick = rng.random(batch) < 0.1
        lengths[pick] = rng.integers(-3, 8 * k + 9, int(pick.sum()))
    blocks = np.full((batch, k), -1, np.int32)
    for b in range(batch):
        nb = -(-max(int(lengths[b]), 0) // 8)
        if nb > k:
            blocks[b] = rng.choice(nb, k, replace=False)
        else:
            blocks[b] = rng.integers(-1, nb + 5, k)
    bpp = page_size // 8
    pages = -(-(-(-width // 8)) // bpp)
    pt = np.stack([rng.permutation(pages) for _ in range(batch)]).astype(np.int32)
    return BlockTableWorkload(f"blocks_{batch}x{k}", seed, blocks, lengths.astype(np.int32), pt, page_size)
