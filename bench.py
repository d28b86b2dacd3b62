#!/usr/bin/env python3
"""Benchmark of the DSA lightning-indexer selection path on one MI355X.

One step = one pass of the whole hot path on synthetic inputs already
resident in device memory:
  * the unpooled indexer on the prefill workload (B=1, S=Skv=4096, H=64,
    D=128, topk=2048, causal): the fused score + mask + top-k kernel
    (rows in index order), then the score-order pass (dsai_sort_rows) -- the
    same work and result as dsai_score_topk under DSAI_ORDER_SCORE, timed
    as two launches so the fused kernel has a duration of its own;
  * the pooled decode selection over one 65536-token indexer cache
    (kpool_compress -> select with expand: index_scores + topk_pools, whose
    kernel also writes the expanded token ids (dsai_select_expand);
    KP=4, 64 query rows, 32 heads, index_topk=512).
Outside the step, the same top-k rows are rescored through the
topk_indices form of dsai_score_topk (scores at supplied indices), and the
cache write's k_norm runs over the 65536 cache rows, and the backward
(gradients of the selected scores, with seeded incoming gradients) runs at
the step's top-k rows of whichever indexer workload is chosen, and the
prefill rows and keys run as 4 packed sequences of 1024 (dsai_score_topk_packed,
score order); all four are reported in `breakdown`
(score_at_indices_*, k_norm_*, backward_*: 6*H*D flops per selected entry,
and the D fp32 key-gradient adds per entry per second; packed_4x1024_*:
2*H*D flops per visible pair of the four sequences).  The pooled decode
stages are also captured once in a HIP graph and replayed
(pooled_decode_graph_ms).
`value` = prefill query tokens per second of the whole step (the pooled
stages' time is counted against it as well).  HIP events on the stream the
library launches on give per-stage times; the fused kernel's roofline is its
algorithmic matrix-core work (2*H*D flops per visible (query, key) pair)
over its average launch time against the dense bf16 peak.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
Profiling helpers (see the summaries under profiles/):
  --copy-calibration      also run a plain device copy of known size (the
                          yardstick for the FETCH_SIZE / WRITE_SIZE counters)
  --pmc-summary F W OUT   turn two rocprofv3 --pmc CSV directories (F with
                          FETCH_SIZE, W with WRITE_SIZE) into the traffic
                          summary OUT that later runs report as `traffic`
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
SCORE_KERNEL = "score_select_kernel"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "score_select_prefill_traffic.txt")


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


def kpool_bytes(pc, P) -> int:
    # read k_normed (bf16) + gate (fp32) + valid (u8) of the pooled tokens + ape;
    # write pool_k (bf16) + pool_tok (i32) + pool_valid (u8)
    n = P * pc.KP
    return n * pc.D * 2 + n * pc.D * 4 + n + pc.KP * pc.D * 4 + P * pc.D * 2 + P * 4 + P


def expand_bytes(pc) -> int:
    sel = pc.index_topk // pc.KP
    return pc.Q * sel * 4 + pc.Q * pc.index_topk * 4


def select_flops(pc, P) -> float:
    return 2.0 * pc.Q * pc.H * pc.D * P


def sort_bytes(case) -> int:
    return 2 * case.B * case.S * case.topk * 8   # read + write (int32 index, fp32 score)


def kernel_sources_sha1() -> str:
    """Fingerprint of everything the kernels are built from."""
    h = hashlib.sha1()
    files = sorted(glob.glob(os.path.join(ROOT, "sparse_attention_token_index_amd", "csrc", "*")))
    files.append(os.path.join(ROOT, "sparse_attention_token_index_amd", "build.py"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def read_traffic():
    """Bytes per launch of the fused kernel from the committed counter summary,
    or None when it is missing or was taken on other kernel sources."""
    try:
        kv = dict(line.split(":", 1) for line in open(TRAFFIC_FILE) if ":" in line
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


def pmc_summary(fetch_dir, write_dir, out):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the fused kernel, each
    scaled by what the counter reads for the copy of COPY_BYTES."""
    fr, wr = _pmc_rows(fetch_dir), _pmc_rows(write_dir)
    is_copy = lambda n: "copy" in n.lower() or "elementwise" in n.lower()
    is_score = lambda n: SCORE_KERNEL in n
    names = sorted({r["Kernel_Name"] for r in fr if is_score(r["Kernel_Name"])})
    # the prefill launch: the fused kernel's dispatches with the largest grid
    # (the packed sequences' launches of the same kernel are smaller)
    grid = max(int(r["Grid_Size"]) for r in fr + wr if is_score(r["Kernel_Name"]))
    fr = [r for r in fr if not is_score(r["Kernel_Name"]) or int(r["Grid_Size"]) == grid]
    wr = [r for r in wr if not is_score(r["Kernel_Name"]) or int(r["Grid_Size"]) == grid]
    f_k, w_k = _per_dispatch(fr, "FETCH_SIZE", is_score), _per_dispatch(wr, "WRITE_SIZE", is_score)
    f_c, w_c = _per_dispatch(fr, "FETCH_SIZE", is_copy), _per_dispatch(wr, "WRITE_SIZE", is_copy)
    if not (f_k and w_k and f_c and w_c):
        sys.exit("missing dispatches of the fused kernel or of the calibration copy")
    big = lambda v: [x for x in v if x * 1024 > COPY_BYTES / 4]   # the 1 GiB copies only
    f_c, w_c = big(f_c), big(w_c)
    fscale = COPY_BYTES / (np.mean(f_c) * 1024)
    wscale = COPY_BYTES / (np.mean(w_c) * 1024)
    fk, wk = np.mean(f_k) * 1024 * fscale, np.mean(w_k) * 1024 * wscale
    lines = [
        "# HBM traffic of the fused score + top-k kernel, prefill workload",
        "# (B=1, S=Skv=4096, H=64, D=128, topk=2048), rocprofv3 --pmc counters.",
        "# commands (from the repository root):",
        "#   rocprofv3 --pmc FETCH_SIZE -f csv -d <F> -o run -- python3 bench.py --steps 3 "
        "--warmup 1 --no-cpu-baseline --copy-calibration",
        "#   rocprofv3 --pmc WRITE_SIZE -f csv -d <W> -o run -- python3 bench.py --steps 3 "
        "--warmup 1 --no-cpu-baseline --copy-calibration",
        "#   python3 bench.py --pmc-summary <F> <W> profiles/score_select_prefill_traffic.txt",
        f"kernel: {names[0] if names else SCORE_KERNEL}",
        f"source_sha1: {kernel_sources_sha1()}",
        f"grid_threads: {grid}",
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


def stats_summary(csv_path, out, command):
    """Short text table of a rocprofv3 --kernel-trace run (its
    kernel_trace.csv), one line per kernel and grid size, so launches of one
    kernel at different sizes (the prefill launch and the packed sequences'
    launches of the fused kernel) are listed apart."""
    groups = {}
    for r in csv.DictReader(open(csv_path)):
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        groups.setdefault((r["Kernel_Name"].strip('"'), grid), []).append(dur)
    total = sum(sum(v) for v in groups.values())
    lines = ["# rocprofv3 kernel-trace statistics per kernel and grid size (threads)",
             f"# command: {command}",
             f"# {'kernel':<64s} {'grid':>8s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} "
             f"{'max_us':>9s} {'pct':>6s}"]
    for (name, grid), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        name = name if len(name) <= 64 else name[:61] + "..."
        lines.append(f"  {name:<64s} {grid:8d} {len(v):6d} {np.mean(v):9.2f} {min(v):9.2f} "
                     f"{max(v):9.2f} {100 * sum(v) / total:6.2f}")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cpu_baseline(case, pc, budget_s=15.0, cap_s=30.0):
    """The oracle (fp64 NumPy, as it stands) running the same step on the host:
    every prefill query row against all its visible keys in score order, then
    the pooled pipeline.  Whole steps are repeated until `budget_s` has
    passed; if one step would run past `cap_s` the prefill rows stop there and
    the step time is extrapolated from the rows done."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    inp = SY.indexer_inputs(case)
    q = SY.bf16_bits_to_f32(inp["q_bits"]).astype(np.float64)
    k = SY.bf16_bits_to_f32(inp["k_bits"]).astype(np.float64)
    w = inp["w"].astype(np.float64)
    pin = SY.pooled_inputs(pc)
    kn = SY.bf16_bits_to_f32(pin["k_normed_bits"]).astype(np.float64)
    pq = SY.bf16_bits_to_f32(pin["q_bits"]).astype(np.float64)

    def pooled():
        ref = oracle.kpool_compress(kn, pin["gate"], pin["valid"], pin["ape"], pc.first_key, pc.KP)
        s = oracle.pooled_index_scores(pq, pin["w"], ref["pool_k"], ref["pool_valid"])
        ids, _ = oracle.topk_pools(s, pc.index_topk // pc.KP)
        oracle.expand_selection(ids, pc.first_key, pc.KP)

    steps, t_rows, rows_done, t_pool, partial = 0, 0.0, 0, 0.0, False
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        for b in range(case.B):
            for t in range(case.S):
                oracle.score_topk(q[t:t + 1, b:b + 1], k[:, b:b + 1], w[t:t + 1, b:b + 1],
                                  case.compress_ratio, case.topk, rows=[t])
                rows_done += 1
                if time.perf_counter() - t_start > cap_s:
                    partial = True
                    break
            if partial:
                break
        t_rows += time.perf_counter() - t0
        if partial:
            break
        t0 = time.perf_counter()
        pooled()
        t_pool += time.perf_counter() - t0
        steps += 1
        if time.perf_counter() - t_start >= budget_s:
            break
    per_row = t_rows / rows_done
    if steps:
        step_s = (t_rows + t_pool) / steps
        sample = (f"{steps} whole step(s): all {case.B * case.S} {case.name} query rows in score "
                  f"order plus the pooled_decode pipeline, fp64 NumPy, "
                  f"{t_rows + t_pool:.1f} s")
    else:
        t0 = time.perf_counter()
        pooled()
        t_pool = time.perf_counter() - t0
        step_s = per_row * case.B * case.S + t_pool
        sample = (f"{rows_done} of {case.B * case.S} {case.name} query rows (t=0..) timed and "
                  f"extrapolated to the step, plus one pooled_decode pipeline, fp64 NumPy")
    return {"value": case.B * case.S / step_s, "unit": "query tokens/s", "cores": int(cores),
            "kind": "oracle", "sample": sample}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill", choices=sorted(SY.CASES))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--pmc-summary", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "OUT"))
    ap.add_argument("--stats-summary", nargs=3, metavar=("KERNEL_TRACE_CSV", "OUT", "COMMAND"))
    args = ap.parse_args()

    if args.pmc_summary:
        pmc_summary(*args.pmc_summary)
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

    # ---- inputs (resident before timing) ----------------------------------
    case = SY.CASES[args.workload]
    inp = SY.indexer_inputs(case)
    q, k = bf16(inp["q_bits"]), bf16(inp["k_bits"])
    w = torch.from_numpy(inp["w"]).to(dev)
    ix = dsai.Indexer(heads=case.H, dim=case.D, chunk_rows=case.chunk_rows,
                      order=dsai.DSAI_ORDER_INDEX)
    out_idx = torch.empty((case.B, case.S, case.topk), dtype=torch.int32, device=dev)
    out_sc = torch.empty((case.B, case.S, case.topk), dtype=torch.float32, device=dev)

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

    stages = ["score_topk", "sort_rows", "kpool_compress", "select_expand"]

    def step(ev=None):
        e = ev or {}

        def mark(name, i):
            if e:
                e[name][i].record()
        mark("score_topk", 0)
        ix.score_topk(q, k, w, case.compress_ratio, case.topk, out_idx=out_idx, out_score=out_sc)
        mark("score_topk", 1)
        mark("sort_rows", 0)
        ix.sort_rows(out_idx, out_sc)
        mark("sort_rows", 1)
        mark("kpool_compress", 0)
        pix.kpool_compress(kn, gate, valid, ape, pool_k=pool_k, pool_tok=pool_tok, pool_valid=pool_valid)
        mark("kpool_compress", 1)
        mark("select_expand", 0)   # index_scores + topk_pools + expand_selection
        pix.select(pq, pw, pool_k, pool_valid, workspace=ws, pool_ids=pids, pool_scores=pscores,
                   tokens=toks, expand=True)
        mark("select_expand", 1)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # whole-step timing
    t0 = time.perf_counter()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = start.elapsed_time(end) / args.steps

    # per-stage timing: HIP events on the stream the library launches on
    # (torch's current stream, which the binding passes to every call); the
    # steps are queued back to back so no event waits on the host
    per = {s: [] for s in stages}
    evs = [{s: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for s in stages} for _ in range(args.steps + 1)]
    for ev in evs:
        step(ev)
    torch.cuda.synchronize()
    for ev in evs[1:]:   # the first step of the batch starts from an idle queue
        for s in stages:
            per[s].append(ev[s][0].elapsed_time(ev[s][1]))
    avg = {s: float(np.mean(v)) for s, v in per.items()}
    med = {s: float(np.median(v)) for s, v in per.items()}

    # scores at supplied indices (the topk_indices form; not part of the
    # step): the step's own top-k rows rescored (prefill workload only)
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    at_ms = at_flops = None
    if case.name == "prefill":
        at_ix = dsai.Indexer(heads=case.H, dim=case.D, chunk_rows=case.chunk_rows)
        at_idx, at_sc = torch.empty_like(out_idx), torch.empty_like(out_sc)
        for _ in range(2):
            at_ix.score_topk(q, k, w, case.compress_ratio, case.topk, topk_indices=out_idx,
                             out_idx=at_idx, out_score=at_sc)
        a0.record()
        for _ in range(args.steps):
            at_ix.score_topk(q, k, w, case.compress_ratio, case.topk, topk_indices=out_idx,
                             out_idx=at_idx, out_score=at_sc)
        a1.record()
        torch.cuda.synchronize()
        at_ms = a0.elapsed_time(a1) / args.steps
        at_flops = 2.0 * case.H * case.D * selected_entries(case)

    # packed sequences (not part of the step): the prefill rows and keys cut
    # into 4 sequences of S/4, each causal on its own keys (prefill only)
    pk_ms = pk_flops = None
    if case.name == "prefill":
        nseq = 4
        cu = np.arange(nseq + 1, dtype=np.int64) * (case.S // nseq)
        pk_ix = dsai.Indexer(heads=case.H, dim=case.D)
        pq_, pk_, pw_ = q[:, 0], k[:, 0], w[:, 0]
        pk_i = torch.empty((case.S, case.topk), dtype=torch.int32, device=dev)
        pk_s = torch.empty((case.S, case.topk), dtype=torch.float32, device=dev)
        for _ in range(2):
            pk_ix.score_topk_packed(pq_, pk_, pw_, cu, cu, case.compress_ratio, case.topk,
                                    out_idx=pk_i, out_score=pk_s)
        a0.record()
        for _ in range(args.steps):
            pk_ix.score_topk_packed(pq_, pk_, pw_, cu, cu, case.compress_ratio, case.topk,
                                    out_idx=pk_i, out_score=pk_s)
        a1.record()
        torch.cuda.synchronize()
        pk_ms = a0.elapsed_time(a1) / args.steps
        t = np.arange(case.S // nseq, dtype=np.int64)
        pk_flops = 2.0 * case.H * case.D * nseq * float(
            np.minimum(case.S // nseq, (t + 1) // case.compress_ratio).sum())

    # the backward (gradients of the selected scores) at the step's own top-k
    # rows, with seeded incoming gradients (not part of the step)
    bw_ix = dsai.Indexer(heads=case.H, dim=case.D)
    bw_g = torch.from_numpy(SY.score_grads(case.seed, case.B, case.S, case.topk)).to(dev)
    bw_ws = torch.empty(bw_ix.backward_workspace_size(case.S, case.Skv, case.B, case.topk,
                                                      case.compress_ratio), dtype=torch.uint8,
                        device=dev)
    bw_out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(w))
    for _ in range(2):
        bw_ix.indexer_backward(q, k, w, out_idx, bw_g, case.compress_ratio, workspace=bw_ws,
                               grad_q=bw_out[0], grad_k=bw_out[1], grad_weights=bw_out[2])
    a0.record()
    for _ in range(args.steps):
        bw_ix.indexer_backward(q, k, w, out_idx, bw_g, case.compress_ratio, workspace=bw_ws,
                               grad_q=bw_out[0], grad_k=bw_out[1], grad_weights=bw_out[2])
    a1.record()
    torch.cuda.synchronize()
    bw_ms = a0.elapsed_time(a1) / args.steps
    bw_entries = selected_entries(case)
    del bw_ws, bw_out

    # the pooled decode stages (kpool_compress -> select with expand) captured
    # once in a HIP graph and replayed: the decode step's latency without
    # per-call launch work (not part of the step)
    def pooled():
        pix.kpool_compress(kn, gate, valid, ape, pool_k=pool_k, pool_tok=pool_tok, pool_valid=pool_valid)
        pix.select(pq, pw, pool_k, pool_valid, workspace=ws, pool_ids=pids, pool_scores=pscores,
                   tokens=toks, expand=True)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        pooled()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        pooled()
    graph.replay()
    torch.cuda.synchronize()
    a0.record()
    for _ in range(args.steps):
        graph.replay()
    a1.record()
    torch.cuda.synchronize()
    pooled_graph_ms = a0.elapsed_time(a1) / args.steps
    del graph

    # the cache write's k_norm (LayerNorm with a bias) over the pooled
    # workload's 65536 cache rows (not part of the step)
    ln_g = torch.ones((pc.D,), dtype=torch.bfloat16, device=dev)
    ln_b = torch.zeros((pc.D,), dtype=torch.bfloat16, device=dev)
    ln_out = torch.empty_like(kn)
    for _ in range(2):
        pix.k_norm(kn, ln_g, ln_b, 1e-5, out=ln_out)
    a0.record()
    for _ in range(args.steps):
        pix.k_norm(kn, ln_g, ln_b, 1e-5, out=ln_out)
    a1.record()
    torch.cuda.synchronize()
    ln_ms = a0.elapsed_time(a1) / args.steps
    ln_bytes = 2 * kn.numel() * 2 + 2 * pc.D * 2

    if args.copy_calibration:
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    flops = indexer_flops(case)
    launches = max(1, -(-case.S // case.chunk_rows)) if case.chunk_rows else 1
    launch_ms = avg["score_topk"] / launches
    achieved = flops / launches / (launch_ms * 1e-3) / 1e12
    kb, eb, sb = kpool_bytes(pc, P), expand_bytes(pc), sort_bytes(case)
    tokens = case.B * case.S
    result = {
        "metric": "indexer query tokens/s (score+top-k) and % bf16 MFMA peak; pool/expand GB/s",
        "value": tokens / (ms_per_step * 1e-3),
        "unit": "query tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{case.name}+pooled_decode", "B": case.B, "S": case.S,
                   "Skv": case.Skv, "H": case.H, "D": case.D, "topk": case.topk,
                   "compress_ratio": case.compress_ratio, "chunk_rows": case.chunk_rows,
                   "order": "score descending",
                   "pooled": {"N": pc.N, "KP": pc.KP, "Q": pc.Q, "H": pc.H, "D": pc.D,
                              "index_topk": pc.index_topk, "P": P},
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "kernel": f"{SCORE_KERNEL}<64,128> (fused score+mask+top-k)",
                     "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": read_traffic(),
                     "flops_per_launch": flops / launches, "avg_launch_ms": launch_ms},
        "breakdown": {
            "score_topk_ms": avg["score_topk"], "score_topk_median_ms": med["score_topk"],
            "sort_rows_ms": avg["sort_rows"], "sort_rows_GBps": sb / (avg["sort_rows"] * 1e-3) / 1e9,
            "kpool_ms": avg["kpool_compress"], "kpool_GBps": kb / (avg["kpool_compress"] * 1e-3) / 1e9,
            "kpool_bytes": kb,
            "select_expand_ms": avg["select_expand"],
            "select_expand_TFLOPs": select_flops(pc, P) / (avg["select_expand"] * 1e-3) / 1e12,
            "expand_bytes": eb, "wall_s": wall,
            "score_at_indices_ms": at_ms,
            "score_at_indices_TFLOPs": (at_flops / (at_ms * 1e-3) / 1e12) if at_ms else None,
            "k_norm_ms": ln_ms, "k_norm_GBps": ln_bytes / (ln_ms * 1e-3) / 1e9,
            "k_norm_bytes": ln_bytes,
            "pooled_decode_graph_ms": pooled_graph_ms,
            "packed_4x1024_ms": pk_ms,
            "packed_4x1024_TFLOPs": (pk_flops / (pk_ms * 1e-3) / 1e12) if pk_ms else None,
            "backward_ms": bw_ms,
            "backward_TFLOPs": 6.0 * case.H * case.D * bw_entries / (bw_ms * 1e-3) / 1e12,
            "backward_key_adds_G_per_s": case.D * bw_entries / (bw_ms * 1e-3) / 1e9,
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(case, pc)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
