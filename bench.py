#!/usr/bin/env python3
"""Benchmark of the DSA lightning-indexer selection path on one MI355X.

One step = one pass of the whole hot path on synthetic inputs already
resident in device memory:
  * the unpooled indexer (fused score + causal mask + top-k) on the prefill
    workload (B=1, S=Skv=4096, H=64, D=128, topk=2048), and
  * the pooled decode selection over one 65536-token indexer cache
    (kpool_compress -> select (index_scores + topk_pools) -> expand;
    KP=4, 64 query rows, 32 heads, index_topk=512).
`value` = prefill query tokens per second of the whole step (the pooled
stages' time is counted against it as well).  Per-kernel HIP-event times
give the roofline of the dominant kernel (the fused indexer: bf16 matrix
cores) and the bandwidth of the pooled streaming kernels.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synthetic as SY  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 4096 flop/clk x 2.4 GHz, dense
PEAK_HBM_GBS = 8000.0


def visible_pairs(case) -> int:
    t = np.arange(case.S, dtype=np.int64)
    return int(np.minimum(case.Skv, (t + 1) // case.compress_ratio).sum()) * case.B


def indexer_flops(case) -> float:
    return 2.0 * case.H * case.D * visible_pairs(case)


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


def cpu_baseline(case, budget_s=20.0):
    """The oracle (fp64 NumPy) on a bounded sample of the workload's rows."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    stride = 32
    rows = list(range(stride - 1, case.S, stride))
    inp = SY.indexer_inputs(case, rows=rows)
    q = SY.bf16_bits_to_f32(inp["q_bits"]).astype(np.float64)
    k = SY.bf16_bits_to_f32(inp["k_bits"]).astype(np.float64)
    w = inp["w"].astype(np.float64)
    done = 0
    t0 = time.perf_counter()
    for i, t in enumerate(rows):
        oracle.score_topk(q[i:i + 1], k, w[i:i + 1], case.compress_ratio, case.topk, rows=[t])
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": done * case.B / dt, "unit": "query tokens/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{done} of {case.S} query rows (every {stride}th, t={stride - 1}..), "
                      f"all visible keys, fp64 NumPy, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill", choices=sorted(SY.CASES))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the selection path runs on a single MI355X in this "
              "build (no sharding); run with --gpus 1.", file=sys.stderr)
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
    ix = dsai.Indexer(heads=case.H, dim=case.D, chunk_rows=case.chunk_rows)
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

    stages = ["score_topk", "kpool_compress", "select", "expand"]

    def step(ev=None):
        e = ev or {}
        def mark(name, i):
            if e:
                e[name][i].record()
        mark("score_topk", 0)
        ix.score_topk(q, k, w, case.compress_ratio, case.topk, out_idx=out_idx, out_score=out_sc)
        mark("score_topk", 1)
        mark("kpool_compress", 0)
        pix.kpool_compress(kn, gate, valid, ape, pool_k=pool_k, pool_tok=pool_tok, pool_valid=pool_valid)
        mark("kpool_compress", 1)
        mark("select", 0)
        pix.select(pq, pw, pool_k, pool_valid, workspace=ws, pool_ids=pids, pool_scores=pscores)
        mark("select", 1)
        mark("expand", 0)
        pix.expand(pids, tokens=toks)
        mark("expand", 1)

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

    # per-kernel timing: HIP events on the stream the library launches on
    per = {s: [] for s in stages}
    for _ in range(args.steps):
        ev = {s: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for s in stages}
        step(ev)
        torch.cuda.synchronize()
        for s in stages:
            per[s].append(ev[s][0].elapsed_time(ev[s][1]))
    avg = {s: float(np.mean(v)) for s, v in per.items()}
    med = {s: float(np.median(v)) for s, v in per.items()}

    flops = indexer_flops(case)
    launches = max(1, -(-case.S // case.chunk_rows)) if case.chunk_rows else 1
    achieved = flops / launches / (avg["score_topk"] / launches * 1e-3) / 1e12
    kb = kpool_bytes(pc, P)
    eb = expand_bytes(pc)
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
                   "pooled": {"N": pc.N, "KP": pc.KP, "Q": pc.Q, "H": pc.H, "D": pc.D,
                              "index_topk": pc.index_topk, "P": P},
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "kernel": "score_topk_kernel<64,128>",
                     "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None,
                     "flops_per_launch": flops / launches, "avg_launch_ms": avg["score_topk"] / launches},
        "breakdown": {
            "score_topk_ms": avg["score_topk"], "score_topk_median_ms": med["score_topk"],
            "score_topk_tokens_per_s": tokens / (avg["score_topk"] * 1e-3),
            "kpool_ms": avg["kpool_compress"], "kpool_GBps": kb / (avg["kpool_compress"] * 1e-3) / 1e9,
            "kpool_bytes": kb,
            "select_ms": avg["select"], "select_TFLOPs": select_flops(pc, P) / (avg["select"] * 1e-3) / 1e12,
            "expand_ms": avg["expand"], "expand_GBps": eb / (avg["expand"] * 1e-3) / 1e9,
            "expand_bytes": eb, "wall_s": wall,
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(case)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
