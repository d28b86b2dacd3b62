#!/usr/bin/env python3
"""Benchmark of the DSA lightning-indexer selection path on one MI355X.

The headline step is one pass of the unpooled indexer over the long-context
workload (B=1, S=Skv=65536, H=64, D=128, 5% of keys x4, causal, topk=2048,
query rows in 1024-row chunks, no score matrix formed): dsai_score_topk in
its default score order (one launch of the fused score + causal mask + top-k
kernel, then the row sort into score-descending order), inputs resident in
device memory.  `value` = query tokens (B*S) per second of that step.
`roofline` is the fused kernel's: 2*H*D flops per visible (query, key) pair
over its launch time, against the dense bf16 peak; the launch time comes
from the same step in index order (the fused kernel alone, one launch per
step), timed with events on the stream the kernel runs on, right after the
headline steps.

Measured in the same run and reported in `breakdown` (not part of `value`):
  * the other indexer workloads in the same call and order - prefill
    (S=Skv=4096, topk=2048) and C4 (B=2, S=16384, Skv=4096, ratio 4,
    topk=512) - each with its own fraction of the bf16 peak, and every
    workload in index order (no score ordering);
  * the pooled decode pipeline over a 65536-token cache (KP=4, Q=64, H=32,
    index_topk=512): kpool_compress and expand_selection with the device's
    caches flushed before every timed launch (a 512 MiB read evicts the
    256 MB last-level cache), as GB/s against HBM peak, also at a scaled
    size (kpool over 2^20 tokens, expand over 65536 rows); select with
    expand, its static-scratch form, and the whole decode chain replayed
    from a HIP graph;
  * the cache write's k_norm (cold), scores at supplied indices, packed
    sequences and the backward (prefill workload);
  * a library bf16 GEMM (torch.matmul, 8192^3) on the same box: the dense
    bf16 rate the box's clock allows under matrix-core load, beside the
    fused kernel's.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
  --step-only             run and time only the headline step (profiling runs)
  --copy-calibration      also run a plain device copy of known size (the
                          yardstick for the FETCH_SIZE / WRITE_SIZE counters)
  --pmc-summary F W OUT   turn two rocprofv3 --pmc CSV directories (F with
                          FETCH_SIZE, W with WRITE_SIZE) into the traffic
                          summary OUT that later runs report as `traffic`
  --counter-summary DIR OUT CMD  per-kernel averages of any rocprofv3 --pmc run
  --stats-summary CSV OUT CMD   text table of a rocprofv3 kernel_trace.csv
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synthetic as SY  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 4 SIMD x 1024 flop/clk x 2.4 GHz, dense bf16
PEAK_HBM_GBS = 8000.0
COPY_BYTES = 1 << 30        # copy calibration: 1 GiB read + 1 GiB written
FLUSH_BYTES = 512 << 20     # read before each cold launch (> 256 MB last-level cache)
SCORE_KERNEL = "score_select_kernel"
METRIC = "indexer query tokens/s (score+top-k) and % bf16 MFMA peak; pool/expand GB/s"


def traffic_file(workload):
    return os.path.join(ROOT, "profiles", f"score_select_{workload}_traffic.txt")


def visible_pairs(case) -> int:
    t = np.arange(case.S, dtype=np.int64)
    return int(np.minimum(case.Skv, (t + 1) // case.compress_ratio).sum()) * case.B


def indexer_flops(case) -> float:
    return 2.0 * case.H * case.D * visible_pairs(case)


def selected_entries(case) -> int:
    """Usable (row, key) entries of the top-k output: sum over rows of
    min(topk, n_t) - the pairs the gather form scores when fed that output."""
    t = np.arange(case.S, dtype=np.int64)
    n = np.minimum(case.Skv, (t + 1) // case.compress_ratio)
    return int(np.minimum(case.topk, n).sum()) * case.B


def kpool_bytes(N, D, KP, first_key=0) -> int:
    # read k_normed (bf16) + gate (fp32) + valid (u8) of the pooled tokens + ape;
    # write pool_k (bf16) + pool_tok (i32) + pool_valid (u8)
    P = max(0, N - first_key) // KP
    n = P * KP
    return n * D * 2 + n * D * 4 + n + KP * D * 4 + P * D * 2 + P * 4 + P


def expand_bytes(Q, select_k, KP) -> int:
    return Q * select_k * 4 + Q * select_k * KP * 4


def select_flops(pc, P) -> float:
    return 2.0 * pc.Q * pc.H * pc.D * P


# The files the fused score + top-k kernel is compiled from (its source and
# every header it includes) and the build script with its flags.
FUSED_KERNEL_SOURCES = ("score_topk.hip", "score_tile.h", "topk_wave.h", "device_common.h",
                        "internal.h")


def kernel_sources_sha1() -> str:
    """Fingerprint of what the fused kernel is built from: a counter summary
    taken on other sources no longer describes it."""
    h = hashlib.sha1()
    csrc = os.path.join(ROOT, "sparse_attention_token_index_amd", "csrc")
    files = [os.path.join(csrc, f) for f in FUSED_KERNEL_SOURCES]
    files.append(os.path.join(ROOT, "sparse_attention_token_index_amd", "build.py"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def read_traffic(workload):
    """HBM bytes per launch of the fused kernel from the committed counter
    summary, or None when it is missing or was taken on other kernel sources."""
    try:
        kv = dict(line.split(":", 1) for line in open(traffic_file(workload)) if ":" in line
                  and not line.startswith("#"))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("source_sha1") != kernel_sources_sha1():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------
# rocprofv3 output summaries
# ---------------------------------------------------------------------------

def _pmc_rows(d):
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        rows += list(csv.DictReader(open(f)))
    if not rows:
        sys.exit(f"no counter_collection.csv under {d}")
    return rows


def _per_dispatch(rows, counter, match):
    vals = {}
    for r in rows:
        if r["Counter_Name"] == counter and match(r["Kernel_Name"]):
            key = r.get("Dispatch_Id") or r.get("Correlation_Id") or str(len(vals))
            vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    return list(vals.values())


def pmc_summary(fetch_dir, write_dir, out, workload="long"):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the fused kernel, each
    scaled by what the counter reads for the copy of COPY_BYTES.  A
    --step-only run launches the fused kernel on one workload only (once per
    step, in both orders), so every dispatch of that kernel is counted."""
    fr, wr = _pmc_rows(fetch_dir), _pmc_rows(write_dir)
    is_copy = lambda n: "copy" in n.lower() or "elementwise" in n.lower()
    is_score = lambda n: SCORE_KERNEL in n
    names = sorted({r["Kernel_Name"] for r in fr if is_score(r["Kernel_Name"])})
    f_k, w_k = _per_dispatch(fr, "FETCH_SIZE", is_score), _per_dispatch(wr, "WRITE_SIZE", is_score)
    f_c, w_c = _per_dispatch(fr, "FETCH_SIZE", is_copy), _per_dispatch(wr, "WRITE_SIZE", is_copy)
    if not (f_k and w_k and f_c and w_c):
        sys.exit("missing dispatches of the fused kernel or of the calibration copy")
    big = lambda v: [x for x in v if x * 1024 > COPY_BYTES / 4]   # the 1 GiB copies only
    f_c, w_c = big(f_c), big(w_c)
    fscale = COPY_BYTES / (np.mean(f_c) * 1024)
    wscale = COPY_BYTES / (np.mean(w_c) * 1024)
    fk, wk = np.mean(f_k) * 1024 * fscale, np.mean(w_k) * 1024 * wscale
    cmd = (f"python3 bench.py --workload {workload} --steps 2 --warmup 1 --step-only "
           f"--no-cpu-baseline --copy-calibration")
    lines = [
        f"# HBM traffic per launch of the fused score + top-k kernel, workload {workload},",
        "# rocprofv3 --pmc counters (one counter per pass), scaled by a 1 GiB device copy.",
        "# commands (from the repository root):",
        f"#   rocprofv3 --pmc FETCH_SIZE -f csv -d <F> -o run -- {cmd}",
        f"#   rocprofv3 --pmc WRITE_SIZE -f csv -d <W> -o run -- {cmd}",
        f"#   python3 bench.py --pmc-summary <F> <W> profiles/score_select_{workload}_traffic.txt "
        f"--workload {workload}",
        f"kernel: {names[0] if names else SCORE_KERNEL}",
        f"source_sha1: {kernel_sources_sha1()}",
        f"dispatches: fetch {len(f_k)}, write {len(w_k)}",
        f"fetch_kib_per_dispatch: {np.mean(f_k):.1f}",
        f"write_kib_per_dispatch: {np.mean(w_k):.1f}",
        f"copy_bytes: {COPY_BYTES}",
        f"copy_fetch_kib: {np.mean(f_c):.1f}",
        f"copy_write_kib: {np.mean(w_c):.1f}",
        f"fetch_scale: {fscale:.4f}",
        f"write_scale: {wscale:.4f}",
        f"fetch_bytes_per_launch: {fk:.0f}",
        f"write_bytes_per_launch: {wk:.0f}",
        f"traffic_bytes_per_launch: {fk + wk:.0f}",
    ]
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def counter_summary(pmc_dir, out, command):
    """Per-kernel averages (per dispatch) of every counter of a rocprofv3
    --pmc run, with the derived matrix-core and LDS figures when their
    counters are present (GRBM_GUI_ACTIVE counts per XCD and is summed over
    the 8 XCDs; SQ_VALU_MFMA_BUSY_CYCLES over the 1024 SIMDs)."""
    rows = _pmc_rows(pmc_dir)
    per = {}
    for r in rows:
        name = r["Kernel_Name"]
        d = per.setdefault(name, {})
        key = r.get("Dispatch_Id") or r.get("Correlation_Id")
        d.setdefault(r["Counter_Name"], {})
        d[r["Counter_Name"]][key] = d[r["Counter_Name"]].get(key, 0.0) + float(r["Counter_Value"])
    lines = ["# rocprofv3 --pmc counters, average per dispatch, per kernel",
             f"# command: {command}"]
    for name, cs in sorted(per.items(), key=lambda kv: kv[0]):
        if "at::" in name:
            continue
        nd = max(len(v) for v in cs.values())
        lines.append(f"kernel: {name[:150]}")
        lines.append(f"  dispatches: {nd}")
        avg = {c: float(np.mean(list(v.values()))) for c, v in cs.items()}
        for c in sorted(avg):
            lines.append(f"  {c}: {avg[c]:.0f}")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in avg and "GRBM_GUI_ACTIVE" in avg:
            cyc = avg["GRBM_GUI_ACTIVE"] / 8.0
            lines.append(f"  derived_mfma_busy_frac: {avg['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc * 1024):.3f}")
        if "SQ_LDS_BANK_CONFLICT" in avg and avg.get("SQ_LDS_IDX_ACTIVE"):
            lines.append("  derived_lds_bank_conflict_frac: "
                         f"{avg['SQ_LDS_BANK_CONFLICT'] / avg['SQ_LDS_IDX_ACTIVE']:.3f}")
        if "SQ_INSTS_VALU" in avg and avg.get("SQ_INSTS_MFMA"):
            lines.append(f"  derived_valu_per_mfma: {avg['SQ_INSTS_VALU'] / avg['SQ_INSTS_MFMA']:.2f}")
        if "GRBM_GUI_ACTIVE" in avg:
            simd_cyc = avg["GRBM_GUI_ACTIVE"] / 8.0 * 1024
            # SQ_ACTIVE_INST_VALU counts quad-cycles summed over the SIMDs
            if "SQ_ACTIVE_INST_VALU" in avg:
                lines.append("  derived_valu_busy_frac: "
                             f"{4.0 * avg['SQ_ACTIVE_INST_VALU'] / simd_cyc:.3f}")
            if "SQ_VALU_MFMA_COEXEC_CYCLES" in avg:
                lines.append("  derived_valu_mfma_coexec_frac: "
                             f"{avg['SQ_VALU_MFMA_COEXEC_CYCLES'] / simd_cyc:.3f}")
        if "SQ_WAIT_INST_ANY" in avg and avg.get("SQ_WAVE_CYCLES"):
            lines.append("  derived_wave_wait_frac: "
                         f"{avg['SQ_WAIT_INST_ANY'] / avg['SQ_WAVE_CYCLES']:.3f}")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def stats_summary(csv_path, out, command):
    """Short text table of a rocprofv3 --kernel-trace run (its
    kernel_trace.csv), one line per kernel and grid size.  `avg_us` is the
    mean dispatch duration; `union_us` is the time during which at least one
    dispatch of that line ran, per dispatch (launches that overlap on two
    streams count once), which is what a host timer around the calls sees."""
    groups = {}
    for r in csv.DictReader(open(csv_path)):
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        groups.setdefault((r["Kernel_Name"].strip('"'), grid), []).append(
            (int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    total = sum(sum(e - s for s, e in v) for v in groups.values())
    lines = ["# rocprofv3 kernel-trace statistics per kernel and grid size (threads)",
             f"# command: {command}",
             f"# {'kernel':<64s} {'grid':>8s} {'calls':>6s} {'avg_us':>9s} {'union_us':>9s} "
             f"{'min_us':>9s} {'max_us':>9s} {'pct':>6s}"]

    def union(iv):
        iv = sorted(iv)
        tot, cs, ce = 0, iv[0][0], iv[0][1]
        for s, e in iv[1:]:
            if s > ce:
                tot += ce - cs
                cs, ce = s, e
            else:
                ce = max(ce, e)
        return tot + ce - cs

    for (name, grid), v in sorted(groups.items(), key=lambda kv: -sum(e - s for s, e in kv[1])):
        d = [(e - s) / 1e3 for s, e in v]
        name = name if len(name) <= 64 else name[:61] + "..."
        lines.append(f"  {name:<64s} {grid:8d} {len(v):6d} {np.mean(d):9.2f} "
                     f"{union(v) / 1e3 / len(v):9.2f} {min(d):9.2f} {max(d):9.2f} "
                     f"{100 * sum(d) * 1e3 / total:6.2f}")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands
# ---------------------------------------------------------------------------

def _sample_rows(case, n):
    """Deterministic spread of query positions over the whole range."""
    return np.unique(np.linspace(0, case.S - 1, n).round().astype(np.int64))


def cpu_baseline(case, budget_s=20.0):
    """The oracle (fp64 NumPy, as it stands) on a bounded sample of the
    headline workload: query rows spread over the positions (256 rows from
    each of 8 evenly spaced 1024-row blocks, so their inputs are drawn
    without drawing the rest), each scored against all its visible keys and
    ranked, in a shuffled order until `budget_s` of oracle time has passed.
    The time per visible (query, key) pair on the rows done, times the
    workload's visible pairs, gives the step time on the host."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    k = SY.bf16_bits_to_f32(SY.indexer_k_bits(case)).astype(np.float64)
    nblk = max(1, case.S // SY.BLOCK)
    blocks = np.unique(np.linspace(0, nblk - 1, min(8, nblk)).round().astype(np.int64))
    rows = np.concatenate([b * SY.BLOCK + np.linspace(0, min(SY.BLOCK, case.S - b * SY.BLOCK) - 1,
                                                      256).round().astype(np.int64)
                           for b in blocks])
    rows = np.unique(rows)
    inp = SY.indexer_inputs(case, rows=rows)
    q = SY.bf16_bits_to_f32(inp["q_bits"]).astype(np.float64)
    w = inp["w"].astype(np.float64)
    order = np.random.default_rng(0).permutation(rows.size)
    pairs, done, spent = 0, 0, 0.0
    for i in order:
        t = int(rows[i])
        t0 = time.perf_counter()
        oracle.score_topk(q[i:i + 1], k, w[i:i + 1], case.compress_ratio, case.topk, rows=[t])
        spent += time.perf_counter() - t0
        done += 1
        pairs += case.B * oracle.visible_keys(t, case.Skv, case.compress_ratio)
        if spent > budget_s:
            break
    step_s = spent / pairs * visible_pairs(case)
    sample = (f"{done} of {case.B * case.S} {case.name} query rows (up to 256 from each of "
              f"{blocks.size} evenly spaced 1024-row blocks, shuffled), each against all its "
              f"visible keys in score order, fp64 NumPy, {spent:.1f} s; extrapolated to the "
              f"whole workload by visible (query, key) pairs")
    cpu = ""
    try:
        with open("/proc/cpuinfo") as fh:
            cpu = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": case.B * case.S / step_s, "unit": "query tokens/s", "cores": int(cores),
            "kind": "oracle", "sample": sample, "cpu": cpu}


# ---------------------------------------------------------------------------
# GPU measurement
# ---------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="long", choices=sorted(SY.CASES))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--step-only", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--pmc-summary", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "OUT"))
    ap.add_argument("--counter-summary", nargs=3, metavar=("PMC_DIR", "OUT", "COMMAND"))
    ap.add_argument("--stats-summary", nargs=3, metavar=("KERNEL_TRACE_CSV", "OUT", "COMMAND"))
    args = ap.parse_args()

    if args.pmc_summary:
        pmc_summary(*args.pmc_summary, workload=args.workload)
        return
    if args.counter_summary:
        counter_summary(*args.counter_summary)
        return
    if args.stats_summary:
        stats_summary(*args.stats_summary)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the selection path runs on a single MI355X "
              "(no sharding); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_attention_token_index_amd as dsai

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def timed(fn, reps, warm=2):
        """Average ms of fn() over `reps` calls queued back to back (HIP events
        on torch's current stream, the stream every library call runs on)."""
        for _ in range(warm):
            fn()
        a, b = ev(), ev()
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    flush_buf = None

    def timed_cold(fn, reps):
        """Average ms of fn() with the caches flushed before each launch: a
        FLUSH_BYTES read (outside the timed interval, clean lines, so no
        write-back competes with fn) evicts the last-level cache and the
        L2s, so fn's inputs come from HBM."""
        nonlocal flush_buf
        sink = torch.empty((), dtype=torch.float32, device=dev)
        if flush_buf is None:
            flush_buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
            for _ in range(3):
                torch.sum(flush_buf, dim=0, out=sink)
        for _ in range(2):  # untimed flush + launch rounds (a first round runs slow)
            torch.sum(flush_buf, dim=0, out=sink)
            fn()
        pairs = [(ev(), ev()) for _ in range(reps)]
        for a, b in pairs:
            torch.sum(flush_buf, dim=0, out=sink)
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in pairs]))

    def indexer_case(case, order):
        inp = SY.indexer_inputs(case)
        q, k = bf16(inp["q_bits"]), bf16(inp["k_bits"])
        w = torch.from_numpy(inp["w"]).to(dev)
        ix = dsai.Indexer(heads=case.H, dim=case.D, chunk_rows=case.chunk_rows, order=order)
        oi = torch.empty((case.B, case.S, case.topk), dtype=torch.int32, device=dev)
        osc = torch.empty((case.B, case.S, case.topk), dtype=torch.float32, device=dev)
        run = lambda: ix.score_topk(q, k, w, case.compress_ratio, case.topk, out_idx=oi,
                                    out_score=osc)
        return run, (q, k, w, oi, osc)

    # ---- headline step ------------------------------------------------------
    case = SY.CASES[args.workload]
    step, held = indexer_case(case, dsai.DSAI_ORDER_SCORE)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    marks = [ev() for _ in range(args.steps + 1)]   # one event between steps
    marks[0].record()
    for i in range(args.steps):
        step()
        marks[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = marks[0].elapsed_time(marks[-1]) / args.steps
    step_ms = [marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)]
    # The fused kernel alone: the same step in index order skips only the
    # row sort, so its launches (one per step) time the kernel by itself.
    q, k, w, oi, osc = held
    ixk = dsai.Indexer(heads=case.H, dim=case.D, chunk_rows=case.chunk_rows,
                       order=dsai.DSAI_ORDER_INDEX)
    kstep = lambda: ixk.score_topk(q, k, w, case.compress_ratio, case.topk, out_idx=oi,
                                   out_score=osc)
    kstep()
    torch.cuda.synchronize()
    ks, ke = ev(), ev()
    ks.record()
    for _ in range(args.steps):
        kstep()
    ke.record()
    torch.cuda.synchronize()
    kernel_ms = ks.elapsed_time(ke) / args.steps
    if args.copy_calibration:
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    flops = indexer_flops(case)
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    result = {
        "metric": METRIC,
        "value": case.B * case.S / (ms_per_step * 1e-3),
        "unit": "query tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "step_ms_median": float(np.median(step_ms)),
        "step_ms_min": float(np.min(step_ms)),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": case.name, "B": case.B, "S": case.S, "Skv": case.Skv,
                   "H": case.H, "D": case.D, "topk": case.topk,
                   "compress_ratio": case.compress_ratio, "chunk_rows": case.chunk_rows,
                   "heavy_keys": f"{case.heavy_frac:g} of keys x{case.heavy_scale:g}",
                   "order": "score descending", "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "kernel": f"{SCORE_KERNEL}<64,128,...> (fused score+mask+top-k)",
                     "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": read_traffic(case.name),
                     "flops_per_launch": flops, "launches_per_step": 1,
                     "avg_launch_ms": kernel_ms},
    }
    if args.step_only:
        print(json.dumps(result), flush=True)
        return

    bd = {"wall_s": wall}
    # ---- indexer workloads --------------------------------------------------
    # Every workload in both orders (the headline one from the runs above).
    ix_case = {}
    for name in ("prefill", "c4", "long"):
        c = SY.CASES[name]
        reps = max(3, args.steps) if name == "long" else max(10, 2 * args.steps)
        ent = {}
        for order, tag in ((dsai.DSAI_ORDER_SCORE, "score"), (dsai.DSAI_ORDER_INDEX, "index")):
            if name == case.name:   # measured above, on the resident inputs
                ms = ms_per_step if tag == "score" else kernel_ms
            else:
                run, keep = indexer_case(c, order)
                ms = timed(run, reps)
                del run, keep
            fl = indexer_flops(c)
            ent[f"{tag}_order_ms"] = ms
            ent[f"{tag}_order_tokens_per_s"] = c.B * c.S / (ms * 1e-3)
            ent[f"{tag}_order_frac"] = fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS
        ent["gflop"] = indexer_flops(c) / 1e9
        ix_case[name] = ent
        torch.cuda.empty_cache()
    bd["indexer"] = ix_case

    # ---- pooled decode pipeline ----------------------------------------------
    pc = SY.POOLED_CASES["pooled_decode"]
    pin = SY.pooled_inputs(pc)
    pix = dsai.Indexer(heads=pc.H, dim=pc.D, kpool=pc.KP, index_topk=pc.index_topk,
                       first_key=pc.first_key)
    P = pix.pool_count(pc.N)
    kn, gate = bf16(pin["k_normed_bits"]), torch.from_numpy(pin["gate"]).to(dev)
    valid, ape = torch.from_numpy(pin["valid"]).to(dev), torch.from_numpy(pin["ape"]).to(dev)
    pq, pw = bf16(pin["q_bits"]), torch.from_numpy(pin["w"]).to(dev)
    pool_k = torch.empty((P, pc.D), dtype=torch.bfloat16, device=dev)
    pool_tok = torch.empty((P,), dtype=torch.int32, device=dev)
    pool_valid = torch.empty((P,), dtype=torch.uint8, device=dev)
    sel = pc.index_topk // pc.KP
    ws = torch.empty((pix.select_workspace_size(pc.Q, P),), dtype=torch.uint8, device=dev)
    pids = torch.empty((pc.Q, sel), dtype=torch.int32, device=dev)
    pscores = torch.empty((pc.Q, sel), dtype=torch.float32, device=dev)
    toks = torch.empty((pc.Q, pc.index_topk), dtype=torch.int32, device=dev)
    reps = max(10, args.steps)

    kp_run = lambda: pix.kpool_compress(kn, gate, valid, ape, pool_k=pool_k, pool_tok=pool_tok,
                                        pool_valid=pool_valid)
    kp_ms = timed_cold(kp_run, reps)
    kb = kpool_bytes(pc.N, pc.D, pc.KP, pc.first_key)
    sel_run = lambda: pix.select(pq, pw, pool_k, pool_valid, workspace=ws, pool_ids=pids,
                                 pool_scores=pscores, tokens=toks, expand=True)
    sel_ms = timed(sel_run, reps)
    st_run = lambda: pix.select_expand_static(pq, pw, pool_k, pool_valid, pids, pscores, toks)
    st_ms = timed(st_run, reps)
    ex_run = lambda: pix.expand(pids, tokens=toks)
    ex_ms = timed_cold(ex_run, reps)
    eb = expand_bytes(pc.Q, sel, pc.KP)

    # scaled diagnostics: kpool over 2^20 tokens, expand over 65536 rows
    NB = 1 << 20
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    kn_b = torch.randn((NB, pc.D), generator=g, device=dev).to(torch.bfloat16)
    gate_b = torch.randn((NB, pc.D), generator=g, device=dev)
    valid_b = (torch.rand((NB,), generator=g, device=dev) < pc.valid_p).to(torch.uint8)
    PB = pix.pool_count(NB)
    pk_b = torch.empty((PB, pc.D), dtype=torch.bfloat16, device=dev)
    pt_b = torch.empty((PB,), dtype=torch.int32, device=dev)
    pv_b = torch.empty((PB,), dtype=torch.uint8, device=dev)
    kpb_ms = timed_cold(lambda: pix.kpool_compress(kn_b, gate_b, valid_b, ape, pool_k=pk_b,
                                                   pool_tok=pt_b, pool_valid=pv_b), reps)
    kbb = kpool_bytes(NB, pc.D, pc.KP, pc.first_key)
    # cold kpool against the token count (the first n of the 2^20 rows): a
    # least-squares line ms = fixed + bytes / marginal rate separates the
    # per-launch start-up from the streaming rate
    sweep_n, sweep_ms, sweep_b = [], [], []
    for lg in range(16, 21):
        n = 1 << lg
        pn = pix.pool_count(n)
        sweep_ms.append(timed_cold(lambda: pix.kpool_compress(
            kn_b[:n], gate_b[:n], valid_b[:n], ape, pool_k=pk_b[:pn], pool_tok=pt_b[:pn],
            pool_valid=pv_b[:pn]), reps))
        sweep_n.append(n)
        sweep_b.append(kpool_bytes(n, pc.D, pc.KP, pc.first_key))
    slope, icpt = np.polyfit(np.array(sweep_b, dtype=np.float64), np.array(sweep_ms), 1)
    kpool_sweep = {"tokens": sweep_n, "bytes": sweep_b, "cold_ms": sweep_ms,
                   "fixed_us": float(icpt) * 1e3,
                   "marginal_GBps": float(1.0 / slope / 1e6) if slope > 0 else None}
    del kn_b, gate_b, valid_b, pk_b, pt_b, pv_b
    QB = 65536
    ids_b = torch.randint(-1, P, (QB, sel), generator=g, device=dev, dtype=torch.int32)
    tok_b = torch.empty((QB, pc.index_topk), dtype=torch.int32, device=dev)
    exb_ms = timed_cold(lambda: pix.expand(ids_b, tokens=tok_b), reps)
    ebb = expand_bytes(QB, sel, pc.KP)
    del ids_b, tok_b

    # the decode chain (kpool -> select with expand) captured once and replayed
    def pooled():
        kp_run()
        sel_run()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        pooled()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        pooled()
    graph_ms = timed(graph.replay, reps)
    del graph

    gbs = lambda b, ms: b / (ms * 1e-3) / 1e9
    bd["pooled_decode"] = {
        "N": pc.N, "KP": pc.KP, "Q": pc.Q, "H": pc.H, "index_topk": pc.index_topk, "P": P,
        "kpool_cold_ms": kp_ms, "kpool_bytes": kb, "kpool_cold_GBps": gbs(kb, kp_ms),
        "kpool_cold_frac_hbm": gbs(kb, kp_ms) / PEAK_HBM_GBS,
        "kpool_2p20_cold_ms": kpb_ms, "kpool_2p20_bytes": kbb,
        "kpool_2p20_cold_GBps": gbs(kbb, kpb_ms), "kpool_2p20_cold_frac_hbm": gbs(kbb, kpb_ms) / PEAK_HBM_GBS,
        "kpool_cold_sweep": kpool_sweep,
        "select_expand_ms": sel_ms,
        "select_expand_TFLOPs": select_flops(pc, P) / (sel_ms * 1e-3) / 1e12,
        "select_expand_static_ms": st_ms,
        "expand_cold_ms": ex_ms, "expand_bytes": eb, "expand_cold_GBps": gbs(eb, ex_ms),
        "expand_q65536_cold_ms": exb_ms, "expand_q65536_bytes": ebb,
        "expand_q65536_cold_GBps": gbs(ebb, exb_ms),
        "expand_q65536_cold_frac_hbm": gbs(ebb, exb_ms) / PEAK_HBM_GBS,
        "decode_graph_ms": graph_ms,
        "decode_tokens_per_s": pc.Q / (graph_ms * 1e-3),
        "select_tokens_per_s": pc.Q / (sel_ms * 1e-3),   # index_scores + topk_pools (+ ids)
    }

    # the cache write's k_norm (LayerNorm with a bias) over the 65536 cache rows
    ln_g = torch.ones((pc.D,), dtype=torch.bfloat16, device=dev)
    ln_b = torch.zeros((pc.D,), dtype=torch.bfloat16, device=dev)
    ln_out = torch.empty_like(kn)
    ln_ms = timed_cold(lambda: pix.k_norm(kn, ln_g, ln_b, 1e-5, out=ln_out), reps)
    ln_bytes = 2 * kn.numel() * 2 + 2 * pc.D * 2
    bd["k_norm"] = {"rows": pc.N, "cold_ms": ln_ms, "bytes": ln_bytes,
                    "cold_GBps": gbs(ln_bytes, ln_ms), "cold_frac_hbm": gbs(ln_bytes, ln_ms) / PEAK_HBM_GBS}
    del held
    torch.cuda.empty_cache()

    # ---- prefill-workload extras: supplied indices, packed, backward ----------
    pcase = SY.CASES["prefill"]
    prun, (q, k, w, oi, osc) = indexer_case(pcase, dsai.DSAI_ORDER_INDEX)
    prun()
    at_ix = dsai.Indexer(heads=pcase.H, dim=pcase.D)
    at_idx, at_sc = torch.empty_like(oi), torch.empty_like(osc)
    at_ms = timed(lambda: at_ix.score_topk(q, k, w, pcase.compress_ratio, pcase.topk,
                                           topk_indices=oi, out_idx=at_idx, out_score=at_sc), reps)
    at_flops = 2.0 * pcase.H * pcase.D * selected_entries(pcase)
    nseq = 4
    cu = np.arange(nseq + 1, dtype=np.int64) * (pcase.S // nseq)
    pk_ix = dsai.Indexer(heads=pcase.H, dim=pcase.D)
    pk_i = torch.empty((pcase.S, pcase.topk), dtype=torch.int32, device=dev)
    pk_s = torch.empty((pcase.S, pcase.topk), dtype=torch.float32, device=dev)
    pk_ms = timed(lambda: pk_ix.score_topk_packed(q[:, 0], k[:, 0], w[:, 0], cu, cu,
                                                  pcase.compress_ratio, pcase.topk,
                                                  out_idx=pk_i, out_score=pk_s), reps)
    # the same rows as one batched call (B = 4 samples of 1024 rows: the
    # single-launch form of the packed problem)
    L = pcase.S // nseq
    q4 = q[:, 0].reshape(nseq, L, pcase.H, pcase.D).transpose(0, 1).contiguous()
    k4 = k[:, 0].reshape(nseq, L, pcase.D).transpose(0, 1).contiguous()
    w4 = w[:, 0].reshape(nseq, L, pcase.H).transpose(0, 1).contiguous()
    b4_i = pk_i.view(nseq, L, pcase.topk)
    b4_s = pk_s.view(nseq, L, pcase.topk)
    b4_ms = timed(lambda: pk_ix.score_topk(q4, k4, w4, pcase.compress_ratio, pcase.topk,
                                           out_idx=b4_i, out_score=b4_s), reps)
    del q4, k4, w4
    t = np.arange(pcase.S // nseq, dtype=np.int64)
    pk_flops = 2.0 * pcase.H * pcase.D * nseq * float(
        np.minimum(pcase.S // nseq, (t + 1) // pcase.compress_ratio).sum())
    bw_g = torch.from_numpy(SY.score_grads(pcase.seed, pcase.B, pcase.S, pcase.topk)).to(dev)
    bw_ws = torch.empty(at_ix.backward_workspace_size(pcase.S, pcase.Skv, pcase.B, pcase.topk,
                                                      pcase.compress_ratio),
                        dtype=torch.uint8, device=dev)
    bw_out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(w))
    bw_ms = timed(lambda: at_ix.indexer_backward(q, k, w, oi, bw_g, pcase.compress_ratio,
                                                 workspace=bw_ws, grad_q=bw_out[0],
                                                 grad_k=bw_out[1], grad_weights=bw_out[2]), reps)
    bw_entries = selected_entries(pcase)
    bd["prefill_extras"] = {
        "score_at_indices_ms": at_ms,
        "score_at_indices_TFLOPs": at_flops / (at_ms * 1e-3) / 1e12,
        "packed_4x1024_ms": pk_ms,
        "packed_4x1024_TFLOPs": pk_flops / (pk_ms * 1e-3) / 1e12,
        "batched_4x1024_ms": b4_ms,
        "packed_vs_batched_rate": b4_ms / pk_ms,
        "backward_ms": bw_ms,
        "backward_TFLOPs": 6.0 * pcase.H * pcase.D * bw_entries / (bw_ms * 1e-3) / 1e12,
        "backward_key_adds_G_per_s": pcase.D * bw_entries / (bw_ms * 1e-3) / 1e9,
    }
    # The same box's practical dense bf16 rate: a library GEMM (torch.matmul,
    # hipBLASLt) of 8192^3 on contiguous operands, beside the fused kernel's
    # rate.  Context for the fraction of the published peak, which the box's
    # clock under matrix-core load caps for every kernel.
    del bw_ws, bw_out, bw_g
    torch.cuda.empty_cache()
    gn = 8192
    ga = torch.randn(gn, gn, device=dev, dtype=torch.bfloat16)
    gb = torch.randn(gn, gn, device=dev, dtype=torch.bfloat16)
    gc = torch.empty(gn, gn, device=dev, dtype=torch.bfloat16)
    g_ms = timed(lambda: torch.matmul(ga, gb, out=gc), 10)
    g_tf = 2.0 * gn ** 3 / (g_ms * 1e-3) / 1e12
    bd["reference_gemm"] = {
        "what": "torch.matmul bf16 8192x8192x8192 (hipBLASLt), same box",
        "ms": g_ms, "TFLOPs": g_tf, "frac": g_tf / PEAK_BF16_TFLOPS,
        "fused_kernel_vs_gemm_rate": achieved / g_tf,
    }
    del ga, gb, gc
    result["breakdown"] = bd
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(case)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
