"""Seeded random cases through every entry point of the short-row and split
kernels, against the CPU oracle.

Each case draws a width (short-row widths, and in two blocks widths for the
persistent kernel up to 262144; odd widths with a padded row stride), k, a
batch of rows of mixed kinds (the adversarial kinds of the parity workloads
and N(0,1) rows), lengths from -2 to past the width, and optionally a page
table (page sizes 1, 3, 16, 64 and 100); it runs one of `topk_select`
(automatic kernel), `topk_select_ex` with the short-row or the persistent
kernel and the sampled path forced, or `topk_select_split`, and, for widths
of at most 16384, `topk_select_bf16` on the same rows rounded to bf16. Every
output is checked against the oracle (values as a multiset of bit patterns,
positions, -1 padding, page mapping). The pages base the fix's correctness on
forcing every backend over many cases ("vLLM PR #56346 report", discussion);
this adds seeded variety to the fixed workloads of the other tests.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from topk_check import check

pytestmark = pytest.mark.gpu

WIDTHS = [700, 4096, 9000, 16384, 16385, 20000, 32767, 32768]
LONG_WIDTHS = [32769, 40000, 65536, 100003, 131072, 262144]
KS = [1, 7, 64, 511, 512, 1000, 2048]
KINDS = synth.C2_KINDS + ["normal"] * 8
ENTRIES = ["auto", "short_sampled", "split"]
LONG_ENTRIES = ["auto", "persistent_sampled", "split"]


@pytest.fixture(scope="module")
def topk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_row_top_fp32_amd as topk_mod
    topk_mod._load()
    return topk_mod


def draw_case(rng, widths, entries):
    W = int(rng.choice(widths))
    k = min(int(rng.choice(KS)), max(1, W // 4))  # some row kinds plant k / 2 values
    B = int(rng.integers(1, 40))
    kinds = [str(rng.choice(KINDS)) for _ in range(B)]
    seed = int(rng.integers(1 << 30))
    stride = (W + 7) // 8 * 8  # 16-byte rows for fp32 and bf16 alike
    wl = synth.mixed_rows(kinds, W, k, seed, row_stride=stride)
    wl.lengths = rng.integers(-2, W + 20, B).astype(np.int32)
    synth.poison_tails(wl.scores, wl.lengths)
    ps = int(rng.choice([0, 0, 1, 3, 16, 64, 100]))
    pt = synth._page_table(rng, B, W, ps) if ps else None
    entry = str(rng.choice(entries))
    return wl, W, k, ps, pt, entry


# four blocks of short widths, two of long ones (the persistent kernel)
BLOCKS = [(b, WIDTHS, ENTRIES, 40) for b in range(4)] + [(4 + b, LONG_WIDTHS, LONG_ENTRIES, 20) for b in range(2)]


@pytest.mark.parametrize("block,widths,entries,cases", BLOCKS, ids=[f"block{b[0]}" for b in BLOCKS])
def test_random_cases(topk, block, widths, entries, cases):
    rng = np.random.default_rng(9100 + block)
    for case in range(cases):
        wl, W, k, ps, pt_h, entry = draw_case(rng, widths, entries)
        B = wl.batch
        print(f"  case {block}.{case}: {entry} B={B} W={W} k={k} ps={ps} seed={wl.seed}", flush=True)
        s = torch.from_numpy(wl.scores).cuda()
        ln = torch.from_numpy(wl.lengths).cuda()
        pt = torch.from_numpy(pt_h).cuda() if ps else None
        out = torch.full((B, k), -5, dtype=torch.int32, device="cuda")
        if entry == "auto":
            topk.topk_select(s, ln, k, out, pt, ps, n_cols=W)
        elif entry == "short_sampled":
            topk.topk_select_ex(s, ln, k, out, pt, ps, n_cols=W, kernel=topk.KERNEL_SHORT, force_path=topk.PATH_SAMPLED)
        elif entry == "persistent_sampled":
            topk.topk_select_ex(s, ln, k, out, pt, ps, n_cols=W, kernel=topk.KERNEL_PERSISTENT,
                                force_path=topk.PATH_SAMPLED)
        else:
            topk.topk_select_split(s, ln, k, out, pt, ps, n_cols=W)
        torch.cuda.synchronize()
        want = oracle.topk(wl.scores, wl.lengths, k, n_cols=W, page_table=pt_h, page_size=ps)
        fails = check(wl.scores, wl.lengths, W, k, out.cpu().numpy(), want, page_table=pt_h, page_size=ps)
        assert not fails, "\n".join(fails)
        if W <= 16384:
            bits = synth.to_bf16_bits(wl.scores)
            sb = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
            ob = torch.full((B, k), -5, dtype=torch.int32, device="cuda")
            topk.topk_select_bf16(sb, ln, k, ob, pt, ps, n_cols=W)
            torch.cuda.synchronize()
            wb = oracle.topk_bf16(bits, wl.lengths, k, n_cols=W, page_table=pt_h, page_size=ps)
            fb = check(oracle.bf16_to_f32(bits), wl.lengths, W, k, ob.cpu().numpy(), wb, page_table=pt_h,
                       page_size=ps)
            assert not fb, "bf16: " + "\n".join(fb)
        assert topk.topk_watchdog_trips() == 0, "a workgroup gave up waiting"
