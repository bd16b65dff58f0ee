#!/usr/bin/env python3
"""Bench: exact per-row top-k on the two decode batches, one MI355X.

A step is one pass of the whole selection over both decode batches, the shapes
of the pages' own latency figures (vLLM PR #56346 report, summary: B=1024,
lengths uniform in 80-100 % of the width):
  * 1024 rows of width 131072, N(0,1) scores, k=2048;
  * 1024 rows of width 262144, N(0,1) scores with 0.1 % peaks (+N(6,1)), k=512.
Inputs are generated on the host from fixed seeds and copied to HBM before
the timed region. `value` is the algorithmic bytes of one step (4 B per valid
score read, 4 B per length read, 4 B per output slot written) divided by the
wall time per step, in GB/s.

Besides the step, the same JSON line carries three sections timed after it,
none part of `value`: `plain_read_context` (a plain row-max read of the same
score buffers, for how close the selection comes to a bare streaming read),
`small_batch` (the first 40 rows of each batch, one
workgroup per row against the split-row entry, eager and replayed from a
HIP graph) and `indexer` (the bf16 top-k and the two-level indexer's block
max, block-key top-k and block table, each with its algorithmic bytes and
fraction of peak).

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, AMD's published peak
# B300 warm latency of the sampled path at these shapes (vLLM PR #56346
# report, summary), context for vs_baseline only
B300_US = {"c3": 207.06, "c4": 301.72}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "topk_rows_kernel_traffic_c3c4.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "exact_row_top_fp32_amd", "csrc", f)
                  for f in ("topk_rows.hip", "topk_device.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(wl) -> int:
    L = np.clip(wl.lengths.astype(np.int64), 0, wl.n_cols)
    return int(4 * L.sum() + 4 * wl.batch + 4 * wl.batch * wl.k)


def source_digest() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(bytes_per_launch: dict):
    """HBM bytes per launch from the committed rocprofv3 counter summary.

    None when there is no summary, or when the kernel source changed since the
    counters were taken.
    """
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            parts = line.split()
            if len(parts) >= 2 and not line.startswith("#"):
                vals[parts[0]] = parts[1]
    if vals.get("kernel_source_sha256_16") != source_digest():
        return None
    try:
        per = [float(vals[f"hbm_bytes_per_launch_{w}"]) for w in ("c3", "c4")]
    except KeyError:
        return None
    return sum(per) / len(per)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cold-iters", type=int, default=10)
    ap.add_argument("--only", choices=["c3", "c4"], default=None,
                    help="time one batch only (for profiling a single launch shape)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-indexer", action="store_true",
                    help="skip timing the bf16 top-k, block-max and block-table kernels")
    ap.add_argument("--small-batch", type=int, default=40,
                    help="also time the first N rows of each batch through topk_select and the "
                         "split-row topk_select_split (0 = skip)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB (a known "
                         "read and write size for calibrating memory counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU (--gpus {args.gpus} is not supported): rows are "
              f"independent, so several GPUs would each take a share of the rows", file=sys.stderr)
        return 2

    import torch

    import exact_row_top_fp32_amd as topk
    import synth

    topk._load()  # raises if the HIP library is not built
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    names = [args.only] if args.only else ["c3", "c4"]
    t0 = time.time()
    wls = {n: getattr(synth, n)() for n in names}
    log(f"generated {names} in {time.time() - t0:.1f}s")
    d_scores = {n: torch.from_numpy(w.scores).to(dev) for n, w in wls.items()}
    d_len = {n: torch.from_numpy(w.lengths).to(dev) for n, w in wls.items()}
    d_out = {n: torch.empty((w.batch, w.k), dtype=torch.int32, device=dev) for n, w in wls.items()}
    nbytes = {n: algorithmic_bytes(w) for n, w in wls.items()}
    stream = torch.cuda.current_stream(dev)

    def launch(n):
        topk.topk_select(d_scores[n], d_len[n], wls[n].k, d_out[n], stream=stream)

    # fallback rows of one call, for the record
    fallbacks = {}
    for n, w in wls.items():
        stats = torch.empty((w.batch, 2), dtype=torch.int32, device=dev)
        topk.topk_select_ex(d_scores[n], d_len[n], w.k, d_out[n], row_stats=stats)
        torch.cuda.synchronize()
        st = stats.cpu().numpy()
        fallbacks[n] = {"full_row_rows": int((st[:, 0] >= topk.ROW_FULL_OVERFLOW).sum()),
                        "survivors_mean": float(st[:, 1].mean()),
                        "survivors_max": int(st[:, 1].max())}
    log("row paths:", fallbacks)

    for _ in range(args.warmup):
        for n in names:
            launch(n)
    torch.cuda.synchronize()

    ev = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)] for n in names}
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        for n in names:
            ev[n][i][0].record(stream)
            launch(n)
            ev[n][i][1].record(stream)
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    ms_per_step = (t_end - t_start) * 1e3 / args.steps
    warm_us = {n: np.array([a.elapsed_time(b) * 1e3 for a, b in ev[n]]) for n in names}
    log(f"timed {args.steps} steps: {ms_per_step:.4f} ms/step")

    # cold: write then read 1 GiB between launches, so that neither L2 nor
    # MALL holds the rows, and no dirty lines of the write are still waiting
    # to be written back when the timed launch starts
    scratch = torch.empty(256 * 1024 * 1024, dtype=torch.float32, device=dev)
    cold_us = {n: [] for n in names}
    for i in range(args.cold_iters):
        for n in names:
            scratch.fill_(float(i))
            scratch.sum()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            launch(n)
            b.record(stream)
            torch.cuda.synchronize()
            cold_us[n].append(a.elapsed_time(b) * 1e3)
    del scratch

    if args.copy_mib > 0:
        src = torch.ones(args.copy_mib * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {args.copy_mib} MiB device to device")
        del src, dst

    step_bytes = sum(nbytes.values())
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    detail = {}
    for n in names:
        w = warm_us[n]
        detail[n] = {
            "rows": wls[n].batch, "width": wls[n].n_cols, "k": wls[n].k, "seed": wls[n].seed,
            "algorithmic_bytes": nbytes[n],
            "warm_us_median": float(np.median(w)), "warm_us_p10": float(np.percentile(w, 10)),
            "warm_us_p90": float(np.percentile(w, 90)),
            "cold_us_median": float(np.median(cold_us[n])),
            "warm_gbs": nbytes[n] / (np.median(w) * 1e-6) / 1e9,
            "cold_gbs": nbytes[n] / (np.median(cold_us[n]) * 1e-6) / 1e9,
            "rows_per_s": wls[n].batch / (np.median(w) * 1e-6),
            "b300_warm_us_context": B300_US[n],
            **fallbacks[n],
        }
    # dominant (only) kernel: per-launch bytes over per-launch duration, from
    # the events that bracket each launch on its stream
    mean_dur_s = float(np.mean(np.concatenate([warm_us[n] for n in names]))) * 1e-6
    mean_bytes = step_bytes / len(names)
    achieved = mean_bytes / mean_dur_s / 1e9
    traffic = read_traffic(nbytes) if not args.only else None
    roofline = {"kernel": "topk_rows_kernel", "bound": "hbm", "achieved": round(achieved, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": traffic}

    plain = plain_read(wls, d_scores, names, detail, stream) if not args.only else None

    small = small_batch(topk, wls, d_scores, d_len, names, args.small_batch, stream) \
        if args.small_batch > 0 and not args.only else None

    indexer = indexer_kernels(topk, wls, d_scores, d_len, stream) \
        if not args.no_indexer and not args.only else None

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wls, d_out, names)

    b300_step_us = sum(B300_US[n] for n in names)
    line = {
        "metric": "exact top-k µs/batch + HBM GB/s, B=1024 ragged 128K/256K fp32",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(b300_step_us / (ms_per_step * 1e3), 3),
        "dtype": "u32",
        "data": "synthetic",
        "config": {
            "workload": "+".join(f"{wls[n].batch}x{wls[n].n_cols} fp32 ragged 80-100% k={wls[n].k}"
                                 for n in names),
            "rows": 1024, "widths": [wls[n].n_cols for n in names], "k": [wls[n].k for n in names],
            "scores": {"c3": "N(0,1)", "c4": "N(0,1) + 0.1% peaks of +N(6,1)"},
            "index_output": "raw", "parallelism": "single GPU",
        },
        "detail": detail,
        "roofline": roofline,
        "plain_read_context": plain,
        "small_batch": small,
        "indexer": indexer,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def plain_read(wls, d_scores, names, detail, stream):
    """Context for the roofline fraction: a plain streaming read of the same
    score buffers (torch's row max over every column, no selection), its rate,
    and the selection's warm rate as a fraction of it."""
    import torch

    res = {}
    for n in names:
        w = wls[n]
        s = d_scores[n][:, :w.n_cols]
        nbytes = 4 * w.batch * w.n_cols
        us = time_us(lambda: torch.amax(s, dim=1), stream)
        gbs = nbytes / (us * 1e-6) / 1e9
        res[n] = {"kernel": "torch.amax(scores, dim=1)", "bytes": nbytes, "warm_us_median": round(us, 2),
                  "gbs": round(gbs, 1), "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4),
                  "topk_gbs_over_plain_read": round(detail[n]["warm_gbs"] / gbs, 3)}
    log(f"plain read: {res}")
    return res


def small_batch(topk, wls, d_scores, d_len, names, rows, stream, iters=200):
    """The first `rows` rows of each batch: one workgroup per row (topk_select)
    against rows split over several workgroups (topk_select_split), eager and
    replayed from a HIP graph; warm medians of HIP events on the launch
    stream, and equal outputs (the graph's last replay against the eager
    topk_select)."""
    import torch

    res = {}
    for n in names:
        w = wls[n]
        s, ln = d_scores[n][:rows], d_len[n][:rows]
        out_a = torch.empty((rows, w.k), dtype=torch.int32, device=s.device)
        out_b = torch.empty_like(out_a)
        ws = torch.empty(topk.topk_split_workspace_bytes(rows), dtype=torch.uint8, device=s.device)
        L = np.clip(w.lengths[:rows].astype(np.int64), 0, w.n_cols)
        nbytes = int(4 * L.sum() + 4 * rows + 4 * rows * w.k)
        calls = {"topk_select": lambda: topk.topk_select(s, ln, w.k, out_a, stream=stream),
                 "topk_select_split": lambda: topk.topk_select_split(s, ln, w.k, out_b, workspace=ws,
                                                                     stream=stream)}
        entry = {"rows": rows, "width": w.n_cols, "k": w.k, "algorithmic_bytes": nbytes}
        for name, fn in calls.items():
            for _ in range(10):
                fn()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(iters)]
            for a, b in ev:
                a.record(stream)
                fn()
                b.record(stream)
            torch.cuda.synchronize()
            us = float(np.median([a.elapsed_time(b) * 1e3 for a, b in ev]))
            entry[name] = {"warm_us_median": round(us, 2), "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
                           "frac_of_peak": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
        # the split call's three launches captured once and replayed
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            topk.topk_select_split(s, ln, w.k, out_b, workspace=ws)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            topk.topk_select_split(s, ln, w.k, out_b, workspace=ws)
        torch.cuda.synchronize()
        out_b.fill_(-1)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(iters)]
        for a, b in ev:
            a.record(stream)
            g.replay()
            b.record(stream)
        torch.cuda.synchronize()
        us = float(np.median([a.elapsed_time(b) * 1e3 for a, b in ev]))
        entry["topk_select_split_graph_replay"] = {
            "warm_us_median": round(us, 2), "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
            "frac_of_peak": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
        del g
        entry["same_selection"] = bool(torch.equal(torch.sort(out_a, 1).values, torch.sort(out_b, 1).values))
        log(f"small batch {n}: {entry}")
        res[n] = entry
    return res


def time_us(fn, stream, iters=100, warmup=10):
    """Median of HIP events around `fn` on the launch stream, in µs."""
    import torch

    for _ in range(warmup):
        fn()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) * 1e3 for a, b in ev]))


def rate(nbytes, us):
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"warm_us_median": round(us, 2), "algorithmic_bytes": int(nbytes), "gbs": round(gbs, 1),
            "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4)}


def indexer_kernels(topk, wls, d_scores, d_len, stream):
    """The kernels beside the fp32 selection, each on its own stream-ordered
    launches: bf16 top-k over 1024 x 16384 consumer rows (k=2048, paged,
    page_size 64), and the two-level indexer over the 128K decode batch
    (block max with topk=512 -> fp32 top-k of 512 blocks over the block keys
    -> block table, page_size 64), each step and the chain. The block keys
    (short rows) are selected both by topk_select and by the split-row entry;
    the chain uses topk_select."""
    import torch

    import synth

    dev = d_scores[next(iter(d_scores))].device
    res = {}
    # bf16 consumer rows
    wb = synth.bf16_rows()
    s = torch.from_numpy(wb.bits.view(np.int16)).to(dev).view(torch.bfloat16)
    ln = torch.from_numpy(wb.lengths).to(dev)
    pt = torch.from_numpy(wb.page_table).to(dev)
    out = torch.empty((wb.batch, wb.k), dtype=torch.int32, device=dev)
    L = np.clip(wb.lengths.astype(np.int64), 0, wb.n_cols)
    m = np.minimum(L, wb.k)
    nbytes = 2 * L.sum() + 4 * wb.batch + 4 * wb.batch * wb.k + 4 * np.minimum(m, -(-L // wb.page_size)).sum()
    us = time_us(lambda: topk.topk_select_bf16(s, ln, wb.k, out, pt, wb.page_size, stream=stream), stream)
    res["bf16_topk_1024x16384_k2048_paged"] = rate(nbytes, us)
    log(f"indexer bf16: {res['bf16_topk_1024x16384_k2048_paged']}")
    del s, ln, pt, out

    if "c3" not in wls:
        return res
    w = wls["c3"]
    k, ps = 512, 64
    sc, ln = d_scores["c3"], d_len["c3"]
    nblk = w.n_cols // 8
    L = np.clip(w.lengths.astype(np.int64), 0, w.n_cols)
    nb_h = (L + 7) // 8
    nb = torch.from_numpy(nb_h.astype(np.int32)).to(dev)
    keys = torch.empty((w.batch, nblk), dtype=torch.float32, device=dev)
    sel = torch.empty((w.batch, k), dtype=torch.int32, device=dev)
    blocks = torch.empty_like(sel)
    pages = torch.empty_like(sel)
    rng = np.random.default_rng(10)
    bpp = ps // 8
    ptab = torch.from_numpy(np.stack([rng.permutation(nblk // bpp) for _ in range(w.batch)]).astype(np.int32)).to(dev)
    amax_bytes = (32 * np.maximum(nb_h - 1, 0) + 4 * nb_h).sum() + 4 * w.batch
    mk = np.minimum(nb_h, k)
    sel_bytes = 4 * nb_h.sum() + 4 * w.batch + 4 * w.batch * k
    tab_bytes = 4 * w.batch * k + 4 * w.batch + 8 * w.batch * k + 4 * np.minimum(mk, -(-nb_h // bpp)).sum()

    def step_amax():
        topk.amax8_varlen(sc, ln, k, out=keys, stream=stream)

    ws = torch.empty(topk.topk_split_workspace_bytes(w.batch), dtype=torch.uint8, device=dev)

    def step_select():
        topk.topk_select(keys, nb, k, sel, stream=stream)

    def step_select_split():
        topk.topk_select_split(keys, nb, k, sel, workspace=ws, stream=stream)

    def step_table():
        blocks.copy_(sel)
        topk.sort_candidate_blocks(blocks, ln, ptab, ps, out_pages=pages, n_cols=w.n_cols, stream=stream)

    def chain():
        step_amax()
        topk.topk_select(keys, nb, k, blocks, stream=stream)
        topk.sort_candidate_blocks(blocks, ln, ptab, ps, out_pages=pages, n_cols=w.n_cols, stream=stream)

    chain()
    res["amax8_1024x131072"] = rate(amax_bytes, time_us(step_amax, stream))
    res["topk_select_block_keys_1024x16384_k512"] = rate(sel_bytes, time_us(step_select, stream))
    res["topk_select_split_block_keys_1024x16384_k512"] = rate(sel_bytes, time_us(step_select_split, stream))
    copy_us = time_us(lambda: blocks.copy_(sel), stream)
    table_us = time_us(step_table, stream) - copy_us
    res["block_table_1024_k512"] = rate(tab_bytes, table_us)
    res["two_level_chain_1024x131072"] = rate(amax_bytes + sel_bytes + tab_bytes, time_us(chain, stream))
    log(f"indexer two-level: {res}")
    return res


CPU_TARGET_S = 10.0  # oracle wall time to aim for
CPU_LIMIT_S = 30.0   # and never run past


def cpu_baseline(wls, d_out, names):
    """The oracle on a bounded sample of the same workload, timed on the host cores.

    The sample is both whole batches, passed again until about CPU_TARGET_S
    of oracle time has run. The first pass also checks the GPU's selection of
    every row against the oracle's.
    """
    import oracle

    total_bytes, total_s, passes, ok = 0, 0.0, 0, True
    while total_s < CPU_TARGET_S and passes < 64:
        for n in names:
            w = wls[n]
            want, secs = oracle.timed_topk(w.scores, w.lengths, w.k, n_cols=w.n_cols)
            total_bytes += algorithmic_bytes(w)
            total_s += secs
            if passes == 0:
                got = d_out[n].cpu().numpy()
                same = np.array_equal(np.sort(got, 1), np.sort(want, 1))
                ok &= bool(same)
                log(f"oracle {n}: {w.batch} rows in {secs:.2f}s; GPU selection equal on every row: {same}")
        passes += 1
        if total_s > CPU_LIMIT_S:
            break
    if not ok:
        raise SystemExit("GPU selection differs from the oracle")
    # one thread, a few rows of each batch: the per-row cost without the
    # parallel loop
    one_thread = {}
    for n in names:
        w = wls[n]
        rows = min(8, w.batch)
        _, secs = oracle.timed_topk(w.scores[:rows], w.lengths[:rows], w.k, n_cols=w.n_cols, threads=1)
        one_thread[n] = round(secs / rows * 1e6, 1)
    sample = "; ".join(f"all {wls[n].batch} rows of the {wls[n].batch}x{wls[n].n_cols} k={wls[n].k} batch"
                       for n in names)
    return {"value": round(total_bytes / total_s / 1e9, 3), "unit": "GB/s",
            "cores": oracle.max_threads(), "kind": "oracle",
            "sample": f"{sample}, {passes} passes (full sort per row, OpenMP over rows)",
            "seconds": round(total_s, 3), "gpu_matches_oracle_on_every_row": ok,
            "one_thread_us_per_row": one_thread, "cpu_model": cpu_model()}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    sys.exit(main())
