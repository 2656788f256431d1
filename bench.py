#!/usr/bin/env python3
"""Benchmark of the paged block-scoring indexer on one MI355X.

One step = one ``qsa_select_paged_tokens`` call over the whole batch of the
pages' kernel shape: the last 1,616-row prefill chunk of a single
184,000-token request (4 index heads, head dim 128, compress ratio 4, top-k
2,048 tokens = 512 blocks, contiguous 64-token pages), i.e. scoring of
74,009,164 visible (row, key) pairs plus the exact top-k of every row.
Inputs are seeded synthetic fp16 N(0,1) draws already resident in HBM.

Printed: one JSON line with rows/s (``value``), Gkeys scored/s, the
roofline of the dominant kernel (timed with HIP events on the stream the
kernels run on) and the CPU oracle timed on a bounded row sample.
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

PAGES_MS_PER_CALL = 10.86      # pages' exact-top-k arm on a Quadro RTX 8000, same workload (context only)
PEAK_MFMA_F16_TFLOPS = 2500.0  # MI355X dense fp16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
FLOPS_PER_ROW_KEY = 2 * 4 * 128  # 4 heads x 128 multiply-adds


WORKLOAD_TEXT = {
    "kernel_shape": "kernel_shape: last 1,616-row prefill chunk of one 184,000-token request, 4 index heads, "
                    "head_dim 128, compress_ratio 4, 64-token contiguous pages, exact top-k 2,048 tokens "
                    "(512 blocks), fp16 N(0,1)",
    "tie_stress": "tie_stress: 512 rows over a 32,768-token request, integer q,k in -2..2, top-k 2,048",
    "mixed": "mixed: 8 requests, contexts U{4k..131k}, ~1,500 rows, permuted 64-token pages, top-k 2,048",
    "decode": "decode: 256 requests x 1 row, contexts U{64k..184k}, permuted pages, 1% x8 outlier keys, top-k 2,048",
    "tiny": "tiny: 64 rows at positions 960..1023 of a 1,024-token request, top-k 64",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-rows", type=int, default=512)
    ap.add_argument("--workload", default="kernel_shape",
                    choices=["tiny", "kernel_shape", "tie_stress", "mixed", "decode"])
    ap.add_argument("--path", choices=["two_pass", "fused"], default=None,
                    help="force one execution arm (default: the library's choice)")
    return ap.parse_args()


def source_digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel_name, src_files, launches_per_step):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, only if
    it was taken on the kernel's current source."""
    path = os.path.join(ROOT, "profiles", f"{kernel_name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_digest") != source_digest(src_files):
        return None
    return rec.get("bytes_per_launch")


def time_calls(fn, steps, warmup, torch):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / steps, wall


KERNELS = {
    "fused": ["sample_scorer", "sample_threshold", "filter_scorer", "final_select"],
    "two_pass": ["scorer", "topk_rows"],
}


def kernel_times(fn, steps, names, torch, Q):
    """Average duration of each kernel of one step, from HIP events the
    library records between its launches on the stream it runs on."""
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(steps)]
    for i in range(steps):
        rec = Q.record_events(evs[i])
        fn()
        got = rec.recorded()
        if got != len(names) + 1:
            raise RuntimeError(f"expected {len(names) + 1} events, library recorded {got}")
    torch.cuda.synchronize()
    out = {}
    for k, n in enumerate(names):
        out[n] = sum(evs[i][k].elapsed_time(evs[i][k + 1]) for i in range(steps)) / steps
    total = sum(evs[i][0].elapsed_time(evs[i][-1]) for i in range(steps)) / steps
    return out, total


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(the indexer shards across GPUs only as a design, see the design notes)", file=sys.stderr)
        return 2
    if args.path:
        os.environ["QSA_FORCE_PATH"] = args.path
    import torch
    import workloads as W
    from paged_block_scoring_amd import qsa as Q

    w = W.make(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q = torch.from_numpy(w.q).to(dev)
    kc = torch.from_numpy(w.kcache).to(dev)
    pt = torch.from_numpy(w.page_table).to(dev)
    pos = torch.from_numpy(w.pos).to(dev)
    row_req = torch.from_numpy(w.row_req).to(dev)
    cr, k = w.compress_ratio, w.k
    vis = (w.pos.astype(np.int64) + 1) // cr
    sum_v = int(vis.sum())
    max_v = int(vis.max())
    rows = w.rows
    out = torch.empty((rows, k), dtype=torch.int32, device=dev)
    ws_bytes = Q.qsa_select_paged_tokens_workspace_size(rows, w.num_reqs, max_v, cr, k, 0)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    def step():
        Q.qsa_select_paged_tokens(q, kc, pt, pos, cr, k, row_req=row_req, max_visible=max_v, out=out,
                                  workspace=ws)

    # the timed region: exactly `steps` whole steps
    ms_step, wall = time_calls(step, args.steps, args.warmup, torch)
    path = Q.qsa_last_path()
    # per-kernel durations of the same launches (instrumented repeat)
    kms, ms_instrumented = kernel_times(step, args.steps, KERNELS[path], torch, Q)

    flops_full = FLOPS_PER_ROW_KEY * sum_v
    units = {}
    if path == "fused":
        stride = 16
        while (max_v + stride - 1) // stride > 4096:
            stride *= 2
        sampled = int(((vis + stride - 1) // stride).sum())
        units["filter_scorer"] = ("mfma", flops_full, PEAK_MFMA_F16_TFLOPS, "TFLOP/s")
        units["sample_scorer"] = ("mfma", FLOPS_PER_ROW_KEY * sampled, PEAK_MFMA_F16_TFLOPS, "TFLOP/s")
    else:
        units["scorer"] = ("mfma", flops_full, PEAK_MFMA_F16_TFLOPS, "TFLOP/s")
        units["topk_rows"] = ("hbm", 4 * sum_v + 4 * rows * k, PEAK_HBM_GBS, "GB/s")
    dom_name = max((n for n in kms if n in units), key=lambda n: kms[n])
    bound, work, peak, unit = units[dom_name]
    scale = 1e12 if unit == "TFLOP/s" else 1e9
    achieved = work / (kms[dom_name] * 1e-3) / scale
    src = ["paged_block_scoring_amd/csrc/score_core.hpp", "paged_block_scoring_amd/csrc/qsa_device.hpp"]
    roofline = {"kernel": dom_name, "bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": traffic_for(dom_name, src, 1),
                "ms_per_launch": round(kms[dom_name], 4)}

    rows_per_s = rows / (ms_step * 1e-3)
    is_headline = args.workload == "kernel_shape"
    result = {
        "metric": "indexer rows/s and Gkeys scored/s at 1616x184k; % MFMA/HBM roofline",
        "value": round(rows_per_s, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(rows_per_s / (rows / (PAGES_MS_PER_CALL * 1e-3)), 3) if is_headline else None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT.get(args.workload, args.workload),
                   "rows": rows, "requests": w.num_reqs, "k": k, "sum_visible_keys": sum_v,
                   "max_visible_keys": max_v, "parallelism": "single-gpu"},
        "gkeys_per_s": round(sum_v / (ms_step * 1e-3) / 1e9, 3),
        "path": path,
        "kernels_ms": {n: round(v, 4) for n, v in kms.items()},
        "ms_per_step_instrumented": round(ms_instrumented, 4),
        "roofline": roofline,
        "wall_s_timed": round(wall, 4),
    }

    if not args.no_cpu_baseline:
        import oracle
        n = min(args.cpu_sample_rows, rows)
        sample = np.unique(np.linspace(0, rows - 1, n).round().astype(np.int64))
        cores = os.cpu_count() or 1
        t0 = time.perf_counter()
        oracle.select_paged_tokens(w.q[sample], w.kcache, w.page_table, w.pos[sample], cr, k,
                                   row_req=w.row_req[sample], nthreads=cores)
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {
            "value": round(len(sample) / dt, 3), "unit": "rows/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(sample)} of the {rows} rows (evenly spaced), each over its full visible context; "
                      f"oracle score + exact select + expand took {dt:.1f} s",
        }
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
