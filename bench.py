#!/usr/bin/env python3
"""Throughput of causal factorized block-sparse attention (forward + backward) on one MI355X.

Metric: useful TFLOP/s of sparse-attention forward + backward at n = 12,288,
and its fraction of the bf16 MFMA peak.  Useful FLOPs per (batch, head) are
4 d P (forward) + 8 d P (backward: dV, dP, dQ, dK), P = visible (query, key)
pairs; the recomputation of the scores in the backward pass is not counted.

One step = forward + backward of both n = 12,288 workloads, on inputs already
resident in HBM:
  fixed_n12288    B=2, H=8, l=128, c=32, alternating same-block / summary heads
  strided_n12288  B=1, H=16, l=128, alternating local / stride heads,
                  shared period-128 sinusoid in Q and K
Timing: W untimed warm-up steps; then K steps between two HIP events with
nothing else recorded (ms_per_step, value); then K more steps with an event
pair around every launch for the per-kernel table and the roofline entry of
the longest kernel (those intervals include the cost of an event, reported
as event_overhead_us).

Prints one JSON line.  ``--gpus`` above 1 exits: the path runs on one GPU.
"""

from __future__ import annotations

import argparse
import json
import math
import multiprocessing as mp
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E (published)
D = 64
DEFAULT_WORKLOADS = ("fixed_n12288", "strided_n12288")


# ----------------------------------------------------------------------------
# algorithmic accounting
# ----------------------------------------------------------------------------

def kernel_work(label: str, B: int, H: int, n: int, pairs: int):
    """(flops, bytes) a launch must do at minimum, per kernel."""
    rows = B * H * n
    if label == "fwd":
        return 4 * D * pairs, rows * (4 * D * 2 + 4)            # Q, K, V read, O write, LSE
    # The backward's 8 d useful FLOPs per pair are split between its kernels as
    # the products each one forms for its own outputs: dQ = dS K (2 d) in the
    # query-tile pass; dV = P^T dO, dP = dO V^T and dK = dS^T Q (6 d) in the
    # key-tile pass.  Score recomputation is not counted.
    if label == "bwd_dq":
        return 2 * D * pairs, rows * (5 * D * 2 + 4 + 4)         # Q,K,V,O,dO read, dQ write; LSE, D
    if label == "bwd_dkdv":
        return 6 * D * pairs, rows * (6 * D * 2 + 8)             # Q,K,V,dO read, dK,dV write; LSE, D
    if label in ("fwd_merge", "bwd_merge"):
        return 0, 0  # merges of split tiles: no useful FLOPs of their own
    raise ValueError(label)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "n12288_fixed_strided_hbm_traffic.txt")
KERNEL_NAMES = {"fwd": "fwd_bf16_kernel", "fwd_merge": "fwd_merge_kernel", "bwd_dq": "bwd_dq_kernel",
                "bwd_dkdv": "bwd_dkdv_kernel", "bwd_merge": "bwd_merge_kernel"}


def measured_traffic(label: str, w):
    """HBM bytes (fetched + written) per launch of this kernel, from the committed
    counter summary; None when there is none or the kernel sources changed since."""
    from factorized_block_sparse_amd import profiling
    recorded, table = profiling.read_traffic(TRAFFIC_FILE)
    if recorded is None or recorded != profiling.source_hash():
        return None
    if label == "fwd_merge":
        key = f"{KERNEL_NAMES[label]}IDF16bLi{w.block_q}E"
    else:
        key = f"{KERNEL_NAMES[label]}<{w.block_q}, {w.block_k}>"
    hits = [v for name, v in table.items() if key in name]
    return round(sum(hits[0])) if len(hits) == 1 else None


def roofline_entry(flops: float, nbytes: float, seconds: float):
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if flops / max(nbytes, 1) >= ridge:
        ach = flops / seconds / 1e12
        return {"bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": ach / PEAK_BF16_TFLOPS}
    ach = nbytes / seconds / 1e9
    return {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": ach / PEAK_HBM_GBS}


# ----------------------------------------------------------------------------
# CPU baseline: the oracle (row-gather mode) on a bounded sample, all host cores
# ----------------------------------------------------------------------------

_CPU = {}


def _cpu_task(args):
    key, rows, deadline = args
    if time.time() > deadline:
        return 0, 0.0
    from oracle import attention as OA
    q, k, v, do, head, n = _CPU[key]
    kf = OA.keys_fn_for(head.kind, n, head.l, head.c or None, head.sub)
    OA.bwd_rows_full(q, k, v, do, kf, rows=rows)
    fl = 0
    for i in rows:
        fl += 12 * D * kf(i).size
    return len(rows), float(fl)


def cpu_baseline(workloads, inputs, seconds: float):
    """Oracle forward + backward rows for ~`seconds` of wall time on a process pool."""
    import numpy as np
    cores = min(os.cpu_count() or 1, 16)
    tasks = []
    for w in workloads:
        inp = inputs[w.name]
        for b in range(w.B):
            for h, head in enumerate(w.heads):
                key = (w.name, b, h)
                _CPU[key] = tuple(inp[x][b, h].double().numpy() for x in ("q", "k", "v", "do")) + (head, w.n)
                rng = np.random.default_rng(1000 * b + h + 17)
                perm = rng.permutation(w.n)
                for c in range(0, w.n, 8):
                    tasks.append((key, sorted(perm[c:c + 8].tolist())))
    total_rows = sum(len(t[1]) for t in tasks)
    rng = np.random.default_rng(0)
    order = rng.permutation(len(tasks))
    os.environ.setdefault("OMP_NUM_THREADS", "1")
    ctx = mp.get_context("fork")
    t0 = time.time()
    deadline = t0 + seconds
    rows_done = 0
    flops = 0.0
    with ctx.Pool(cores) as pool:
        for r, f in pool.imap_unordered(_cpu_task, [(tasks[i][0], tasks[i][1], deadline) for i in order],
                                        chunksize=1):
            rows_done += r
            flops += f
    wall = time.time() - t0
    return {"value": flops / wall / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": (f"{rows_done} of the {total_rows} query rows of {'+'.join(w.name for w in workloads)} "
                       f"(random order over every batch element and head) through the float64 row-gather "
                       f"oracle forward+backward in {wall:.1f} s of wall time (deadline {seconds:.0f} s); "
                       f"useful FLOPs 12*d*keys per row"),
            "seconds": wall}


# ----------------------------------------------------------------------------
# GPU run
# ----------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workloads", default=",".join(DEFAULT_WORKLOADS))
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before the workloads, run one device-to-device copy of this many MiB "
                         "(a plain copy kernel of known size, for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported "
              "(the attention path is single-GPU; see the design notes for how it would shard)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from factorized_block_sparse_amd import binding as bd
    from factorized_block_sparse_amd import workloads as W

    dev = torch.device("cuda:0")
    if args.copy_calibration_mib > 0:
        nbytes = args.copy_calibration_mib << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    names = [s for s in args.workloads.split(",") if s]
    wls = [W.WORKLOADS[nm] for nm in names]
    inputs, runs = {}, []
    for w in wls:
        lay = bd.Layout(w.n, w.heads, w.block_q, w.block_k)
        inp = W.workload_inputs(w)
        inputs[w.name] = inp
        q, k, v, do = (inp[x].to(dev) for x in ("q", "k", "v", "do"))
        dt = bd.SA_BF16 if w.dtype == "bf16" else bd.SA_FP32
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.n), dtype=torch.float32, device=dev)
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
        ws = torch.empty(bd.bwd_workspace_bytes(lay, w.B, w.H), dtype=torch.uint8, device=dev)
        fws = torch.empty(max(1, bd.fwd_workspace_bytes(lay, w.B, w.H, dtype=dt)), dtype=torch.uint8,
                          device=dev)
        pairs = lay.pairs_per_batch() * w.B
        split_q, split_k = lay.header.comb_sched_len > 0, lay.header.red_sched_len > 0
        calls = []
        for label, ph in (("fwd", bd.SA_FWD_MAIN), ("fwd_merge", bd.SA_FWD_MERGE)):
            if label == "fwd_merge" and not split_q:
                continue
            calls.append((label, lambda lay=lay, q=q, k=k, v=v, o=o, lse=lse, fws=fws, ph=ph:
                          bd.sparse_attn_fwd(lay, q, k, v, out=o, lse=lse, workspace=fws, phases=ph)))
        if w.backward:
            for label, ph in (("bwd_dq", bd.SA_BWD_DQ), ("bwd_dkdv", bd.SA_BWD_DKDV),
                              ("bwd_merge", bd.SA_BWD_MERGE)):
                if label == "bwd_merge" and not (split_q or split_k):
                    continue
                calls.append((label, lambda lay=lay, q=q, k=k, v=v, o=o, lse=lse, do=do, ws=ws, grads=grads, ph=ph:
                              bd.sparse_attn_bwd(lay, q, k, v, o, lse, do, workspace=ws, grads=grads, phases=ph)))
        useful = (12 if w.backward else 4) * D * pairs
        tiles = lay.tiles_per_batch() * w.B
        runs.append(dict(w=w, lay=lay, calls=calls, pairs=pairs, useful=useful,
                         padding=tiles * w.block_q * w.block_k / pairs))

    flat = [(r["w"], label, fn) for r in runs for (label, fn) in r["calls"]]

    def step(evs=None):
        for i, (_, _, fn) in enumerate(flat):
            if evs is not None:
                evs[i].record()
            fn()
        if evs is not None:
            evs[len(flat)].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K whole steps between two events, nothing recorded inside
    # (each event costs the GPU about 5 us, which would inflate the step).
    K = args.steps
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for s in range(K):
        step()
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / K

    # Per-kernel breakdown: K more steps with an event before and after every
    # launch, on the stream the library launches on (torch's current stream).
    # These intervals include the event cost; it is measured right after, with
    # back-to-back events queued behind the last launches.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(flat) + 1)] for _ in range(K)]
    for s in range(K):
        step(evs[s])
    b2b = [torch.cuda.Event(enable_timing=True) for _ in range(9)]
    for e in b2b:
        e.record()
    torch.cuda.synchronize()
    per_call_ms = [sum(evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(K)) / K for i in range(len(flat))]
    event_us = 1000 * b2b[0].elapsed_time(b2b[-1]) / (len(b2b) - 1)

    useful = sum(r["useful"] for r in runs)
    value = useful / (ms_per_step * 1e-3) / 1e12

    # per-workload and per-kernel breakdown
    per_wl, kernels, idx = {}, [], 0
    for r in runs:
        w = r["w"]
        ms = 0.0
        for label, _ in r["calls"]:
            t = per_call_ms[idx]
            ms += t
            fl, by = kernel_work(label, w.B, w.H, w.n, r["pairs"])
            kernels.append(dict(workload=w.name, kernel=label, ms=t, flops=fl, bytes=by))
            idx += 1
        tf = r["useful"] / (ms * 1e-3) / 1e12
        per_wl[w.name] = {"ms": round(ms, 4), "useful_tflops": round(tf, 2),
                          "pct_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
                          "pairs": r["pairs"], "tile_padding_overhead": round(r["padding"], 3)}
    dom = max(kernels, key=lambda k: k["ms"])
    roof = roofline_entry(dom["flops"], dom["bytes"], dom["ms"] * 1e-3)
    roof.update({"traffic": measured_traffic(dom["kernel"], W.WORKLOADS[dom["workload"]]),
                 "kernel": f"{dom['kernel']} ({dom['workload']})",
                 "launch_us": round(dom["ms"] * 1e3, 2), "event_overhead_us": round(event_us, 2)})
    for k in kernels:
        k["ms"] = round(k["ms"], 4)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wls, inputs, args.cpu_seconds)

    line = {
        "metric": "sparse-attn fwd+bwd useful TFLOP/s at n=12288; % of bf16 MFMA peak",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "pct_of_bf16_mfma_peak": round(100 * value / PEAK_BF16_TFLOPS, 3),
        "config": {"workload": "+".join(names),
                   "shapes": {w.name: {"B": w.B, "H": w.H, "n": w.n, "d": w.d,
                                       "heads": sorted({h.kind for h in w.heads}),
                                       "tiles": [w.block_q, w.block_k]} for w in wls},
                   "per_workload": per_wl, "kernels": kernels},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
