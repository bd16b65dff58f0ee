"""Seeded generators: determinism, shapes, length ranges, poison, page tables."""
from __future__ import annotations

import hashlib
import os

import numpy as np

import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def page_constants():
    vals = {}
    with open(os.path.join(HERE, "golden", "page_constants.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                name, value = line.split()[:2]
                vals[name] = float(value)
    return vals


def digest(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def test_same_seed_same_bytes():
    assert digest(synth.c1().scores) == digest(synth.c1().scores)
    a, b = synth.c2(1024), synth.c2(1024)
    assert digest(a.scores) == digest(b.scores) and a.kinds == b.kinds
    p, q = synth.c5(batch=16, width=4096), synth.c5(batch=16, width=4096)
    assert digest(p.scores) == digest(q.scores) and digest(p.page_table) == digest(q.page_table)


def test_c2_rows_and_kinds():
    wl = synth.c2(2048)
    assert wl.scores.shape == (64, 32768) and len(set(wl.kinds)) == 16
    assert np.all(wl.lengths == 32768) and not np.isnan(wl.scores).any()
    consts = page_constants()
    row = wl.scores[wl.kinds.index("crowd16385")]
    bits = row.view(np.uint32)
    crowd = (bits >= 0x40000000) & (bits < 0x40000000 + 8192)
    assert crowd.sum() >= consts["filtered_drop_population"]
    row = wl.scores[wl.kinds.index("above_fp16")]
    assert (row > consts["fp16_max"]).sum() > row.size // 2
    # values in (65504, 65520) round to 65504 in fp16; from 65520 up they become inf
    near = row[(row > 65504) & (row < 65520)]
    assert near.size == 8 and np.all(near.astype(np.float16) == np.float16(65504))
    with np.errstate(over="ignore"):
        assert np.all(np.isinf(row[row >= 65520].astype(np.float16)))
    sz = wl.scores[wl.kinds.index("signed_zero")].view(np.uint32)
    assert (sz == 0).any() and (sz == 0x80000000).any()


def test_decode_batches_small_replica():
    # the full-size batches are built the same way; check the recipe at 1/64 width
    wl = synth.c3(batch=64, width=2048)
    assert wl.lengths.min() >= 1639 and wl.lengths.max() <= 2048
    for b in range(64):
        L = wl.lengths[b]
        assert not np.isnan(wl.scores[b, :L]).any()
        assert np.all(wl.scores[b, L:].view(np.uint32) == synth.POISON_BITS)
    w4 = synth.c4(batch=32, width=8192)
    assert w4.k == 512 and (w4.scores[np.isfinite(w4.scores)] > 4.5).sum() > 0


def test_c5_categories_and_page_table():
    wl = synth.c5(batch=64, width=4096)
    k = wl.k
    assert list(wl.lengths[:5]) == [0, 1, k - 1, k, k + 1]
    assert wl.page_size == 64 and wl.page_table.shape == (64, 64)
    for b in range(64):
        assert np.array_equal(np.sort(wl.page_table[b]), np.arange(64))
    pool = synth.c5(batch=8, width=4096, global_pool=True)
    assert np.unique(pool.page_table).size == pool.page_table.size


def test_bf16_rounding_is_nearest_even():
    # values exactly between two bf16 numbers go to the even pattern; NaN
    # becomes the quiet NaN; overflow past the largest bf16 rounds to +inf
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -7, -2.5, 3.4e38, np.nan],
                 np.float32)
    got = synth.to_bf16_bits(x)
    assert got.tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020, 0x7F80, 0x7FC0]


def test_bf16_workloads():
    a, b = synth.bf16_rows(64, 16384, 2048), synth.bf16_rows(64, 16384, 2048)
    assert digest(a.bits) == digest(b.bits) and digest(a.page_table) == digest(b.page_table)
    assert a.bits.dtype == np.uint16 and a.bits.shape == (64, 16384)
    assert np.all((a.lengths >= int(np.ceil(0.8 * 16384))) & (a.lengths <= 16384))
    for r in range(a.batch):
        L = int(a.lengths[r])
        assert np.all(a.bits[r, L:] == synth.BF16_POISON)
        assert not np.any((a.bits[r, :L] & 0x7FFF) > 0x7F80)  # no NaN inside the row
        assert sorted(a.page_table[r].tolist()) == list(range(16384 // 64))
    adv = synth.bf16_adversarial(512)
    assert adv.bits.shape == (2 * len(synth.C2_KINDS), 16384)


def test_amax8_and_block_table_workloads():
    w = synth.amax8_rows(16, 4096, 64, nan_rate=0.01, zero_rate=0.01)
    assert w.out_blocks == 512 and w.scores.shape == (16, 4096)
    inside = np.concatenate([w.scores[r, :int(w.lengths[r])] for r in range(16)])
    assert np.isnan(inside).any() and (inside == 0).any()  # NaN and zeros inside the rows
    c = synth.candidate_blocks(128, 8192, 32, page_size=64)
    for r in range(c.batch):
        nb = -(-max(int(c.lengths[r]), 0) // 8)
        if nb > 32:  # a top-k selection: 32 distinct ids of [0, nb)
            row = c.blocks[r]
            assert len(set(row.tolist())) == 32 and row.min() >= 0 and row.max() < nb
    assert c.page_table.shape == (128, 8192 // 8 // 8)
