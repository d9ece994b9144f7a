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
pair around every launch for the per-kernel table, the forward-only times and
the roofline entry of the longest kernel (those intervals include the cost of
an event, reported as event_overhead_us); then K steps with one event between
consecutive steps (p10 / p50 / p90 of single steps); then K cache-cold steps
that rotate three input sets; then K steps with each workload on a stream of
its own (value_two_streams; the headline stays the one-stream value); then a
vendor bf16 GEMM as a measured peak reference and device-to-device copies as
measured HBM and Infinity-Cache bandwidths.  The layout build is timed once
on the host.

Prints one JSON line.  ``--gpus`` above 1 exits: the path runs on one GPU.
``--sweep-n`` (the O(n sqrt n) scaling check) and ``--crossover`` (dense
causal against the strided pattern) replace the benchmark with a sweep that
prints one JSON line per configuration.
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
        return 2 * D * pairs, rows * (6 * D * 2 + 4 + 4)         # Q,K,V,O,dO read, dQ write; LSE, D
    if label == "bwd_dkdv":
        return 6 * D * pairs, rows * (6 * D * 2 + 8)             # Q,K,V,dO read, dK,dV write; LSE, D
    # Segment pass (stride heads' classes): all 8 d per pair in one kernel.
    if label == "bwd_seg":
        return 8 * D * pairs, rows * (8 * D * 2 + 4)             # Q,K,V,O,dO read, dQ,dK,dV write; LSE
    if label in ("fwd_merge", "bwd_merge"):
        return 0, 0  # merges of split tiles: no useful FLOPs of their own
    raise ValueError(label)


def algorithmic_bytes(w) -> int:
    """HBM bytes one forward (+ backward) of a workload must move: the forward
    reads Q, K, V and writes O and LSE; the backward reads Q, K, V, O, dO, LSE
    and D (the per-row dO . O, one float) and writes dQ, dK, dV."""
    elt = 2 if w.dtype == "bf16" else 4
    rows = w.B * w.H * w.n
    fwd = rows * (4 * D * elt + 4)
    return fwd + (rows * (8 * D * elt + 8) if w.backward else 0)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "n12288_fixed_strided_hbm_traffic.txt")
KERNEL_NAMES = {"fwd": "fwd_bf16_kernel", "fwd_merge": "fwd_merge_kernel", "bwd_dq": "bwd_dq_kernel",
                "bwd_dkdv": "bwd_dkdv_kernel", "bwd_merge": "bwd_merge_kernel", "bwd_seg": "bwd_seg_kernel"}


def segment_heads(lay) -> tuple:
    """(heads run by the segment pass, their visible pairs) for one batch element."""
    items = lay.xcd_items("seg").reshape(-1, 9)
    heads = sorted({int(r[0]) for r in items if r[0] >= 0})
    hp = lay.head_pattern_index()
    return len(heads), sum(int(lay.pattern_rec(int(hp[h])).pairs) for h in heads)


def launch_work(label: str, w, lay) -> tuple:
    """kernel_work over the heads a launch processes: the segment pass takes the
    segmented heads, the dQ and dK/dV passes the others."""
    hs, ps = segment_heads(lay)
    pairs = lay.pairs_per_batch()
    if label == "bwd_seg":
        return kernel_work(label, w.B, hs, w.n, ps * w.B)
    if label in ("bwd_dq", "bwd_dkdv"):
        return kernel_work(label, w.B, w.H - hs, w.n, (pairs - ps) * w.B)
    return kernel_work(label, w.B, w.H, w.n, pairs * w.B)


def kernel_sources_hash() -> str:
    from factorized_block_sparse_amd import profiling
    return profiling.source_hash()


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
        key = f"{KERNEL_NAMES[label]}<{w.block_q}, {w.block_k}"  # any prefix-mask variant
    hits = [v for name, v in table.items() if key in name]
    return round(sum(hits[0])) if len(hits) == 1 else None


def cache_cold_step_ms(torch, bd, runs, K: int) -> float:
    """ms per fwd+bwd step when each step uses another of three input sets."""
    sets = []
    for r in runs:
        q, k, v, do, o, lse, grads, ws, fws, dt = r["tensors"]
        sets.append([(q, k, v, do)] + [tuple(x.clone() for x in (q, k, v, do)) for _ in range(2)])

    def step(j):
        for r, st in zip(runs, sets):
            w, lay = r["w"], r["lay"]
            q, k, v, do = st[j % 3]
            _, _, _, _, o, lse, grads, ws, fws, dt = r["tensors"]
            bd.sparse_attn_fwd(lay, q, k, v, out=o, lse=lse, workspace=fws)
            if w.backward:
                bd.sparse_attn_bwd(lay, q, k, v, o, lse, do, workspace=ws, grads=grads)

    for j in range(3):
        step(j)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for j in range(K):
        step(j)
    b.record()
    torch.cuda.synchronize()
    del sets
    return a.elapsed_time(b) / K


def two_stream_step_ms(torch, runs, K: int) -> float:
    """ms per step with each workload's launches on a stream of its own, both
    joined to the current stream at the end of every step."""
    main = torch.cuda.current_stream()
    streams = [torch.cuda.Stream() for _ in runs]

    def step():
        start = torch.cuda.Event()
        start.record(main)
        done = []
        for r, st in zip(runs, streams):
            st.wait_event(start)
            with torch.cuda.stream(st):
                for _, fn in r["calls"]:
                    fn()
            e = torch.cuda.Event()
            e.record(st)
            done.append(e)
        for e in done:
            main.wait_event(e)

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(K):
        step()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / K


def vendor_gemm_reference(torch):
    """A measured bf16 MFMA reference on this GPU: torch.matmul (the vendor GEMM
    library) of two 8192 x 8192 bf16 matrices, best of 3 timings of 10 calls."""
    try:
        n = 8192
        a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
        b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
        for _ in range(3):
            c = a @ b
        torch.cuda.synchronize()
        best = None
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(10):
                c = a @ b
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) / 10
            best = t if best is None else min(best, t)
        del a, b, c
        return {"tflops": round(2 * n ** 3 / (best * 1e-3) / 1e12, 1),
                "what": "torch.matmul bf16 8192x8192x8192, best of 3 x 10 calls"}
    except Exception:  # reference only; never fails the bench
        return None


def vendor_copy_reference(torch):
    """Measured memory references on this GPU: device-to-device copies (the
    vendor copy kernel) of 2 GiB, far more than the 256 MB Infinity Cache (HBM
    bandwidth), and of 64 MiB, which stays in it (Infinity-Cache bandwidth);
    bytes read + written per second, best of 3 timings."""
    try:
        out = {}
        for key, size, reps in (("hbm_gbs", 2 << 30, 5), ("infinity_cache_gbs", 64 << 20, 50)):
            a = torch.empty(size, device="cuda", dtype=torch.uint8)
            b = torch.empty_like(a)
            for _ in range(3):
                b.copy_(a)
            torch.cuda.synchronize()
            best = None
            for _ in range(3):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(reps):
                    b.copy_(a)
                e1.record()
                torch.cuda.synchronize()
                t = e0.elapsed_time(e1) / reps
                best = t if best is None else min(best, t)
            out[key] = round(2 * size / (best * 1e-3) / 1e9, 1)
            del a, b
        out["what"] = "device-to-device copies of 2 GiB and 64 MiB, (read + written bytes) / time, best of 3"
        return out
    except Exception:  # reference only; never fails the bench
        return None


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


def host_cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_task(args):
    key, rows, deadline = args
    if time.time() > deadline:
        return 0, 0.0
    from oracle import attention as OA
    q, k, v, do, head, n = _CPU[key]
    kf = OA.keys_fn_for(head.kind, n, head.l, head.c or None, head.sub)
    OA.fwd_rows(q, k, v, kf, rows)              # O, LSE: 4 d per key
    OA.bwd_rows_full(q, k, v, do, kf, rows=rows)  # dV, dP, dQ, dK: 8 d per key
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
            "host_cpu": host_cpu_model(), "nproc": os.cpu_count(),
            "sample": (f"{rows_done} of the {total_rows} query rows of {'+'.join(w.name for w in workloads)} "
                       f"(random order over every batch element and head) through the float64 row-gather "
                       f"oracle forward (fwd_rows) and backward (bwd_rows_full) in {wall:.1f} s of wall "
                       f"time (deadline {seconds:.0f} s); useful FLOPs 12*d*keys per row (4 d forward, 8 d "
                       f"backward)"),
            "seconds": wall}


# ----------------------------------------------------------------------------
# sweeps (separate modes; each prints one JSON line per configuration and a
# summary line)
# ----------------------------------------------------------------------------

def time_config(torch, bd, W, n: int, heads, block_q: int, block_k: int, B: int, seed: int,
                steps: int, warmup: int) -> dict:
    """Forward and forward+backward ms of one layout on seeded bf16 inputs."""
    H = len(heads)
    t0 = time.perf_counter()
    lay = bd.Layout(n, heads, block_q, block_k)
    layout_ms = 1000 * (time.perf_counter() - t0)
    inp = W.make_inputs(B, H, n, D, seed)
    q, k, v, do = (inp[x].to("cuda") for x in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, n), dtype=torch.float32, device="cuda")
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    fws = torch.empty(max(1, bd.fwd_workspace_bytes(lay, B, H)), dtype=torch.uint8, device="cuda")
    ws = torch.empty(bd.bwd_workspace_bytes(lay, B, H), dtype=torch.uint8, device="cuda")

    def fwd():
        bd.sparse_attn_fwd(lay, q, k, v, out=o, lse=lse, workspace=fws)

    def both():
        fwd()
        bd.sparse_attn_bwd(lay, q, k, v, o, lse, do, workspace=ws, grads=grads)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    fwd_ms, both_ms = timed(fwd), timed(both)
    pairs = lay.pairs_per_batch() * B
    area = lay.tiles_per_batch() * B * block_q * block_k
    useful = 12 * D * pairs
    return {"n": n, "B": B, "H": H, "tiles": [block_q, block_k], "pairs": pairs,
            "computed_tile_area": area, "tile_padding_overhead": round(area / pairs, 3),
            "fwd_ms": round(fwd_ms, 4), "fwd_bwd_ms": round(both_ms, 4),
            "useful_tflops": round(useful / (both_ms * 1e-3) / 1e12, 2),
            "layout_build_ms": round(layout_ms, 2)}


def time_workload(torch, bd, W, w, steps: int, warmup: int) -> dict:
    """Forward and forward + backward ms of one named workload on its own inputs."""
    lay = bd.Layout(w.n, w.heads, w.block_q, w.block_k)
    inp = W.workload_inputs(w)
    q, k, v, do = (inp[x].to("cuda") for x in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.n), dtype=torch.float32, device="cuda")
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    fws = torch.empty(max(1, bd.fwd_workspace_bytes(lay, w.B, w.H)), dtype=torch.uint8, device="cuda")
    ws = torch.empty(bd.bwd_workspace_bytes(lay, w.B, w.H), dtype=torch.uint8, device="cuda")

    def fwd():
        bd.sparse_attn_fwd(lay, q, k, v, out=o, lse=lse, workspace=fws)

    def both():
        fwd()
        bd.sparse_attn_bwd(lay, q, k, v, o, lse, do, workspace=ws, grads=grads)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    fwd_ms, both_ms = timed(fwd), timed(both)
    pairs = lay.pairs_per_batch() * w.B
    area = lay.tiles_per_batch() * w.B * w.block_q * w.block_k
    return {"B": w.B, "H": w.H, "n": w.n, "tiles": [w.block_q, w.block_k], "pairs": pairs,
            "tile_padding_overhead": round(area / pairs, 3), "fwd_ms": round(fwd_ms, 4),
            "ms": round(both_ms, 4),
            "useful_tflops": round(12 * D * pairs / (both_ms * 1e-3) / 1e12, 2),
            "computed_over_dense_causal": round(area / (w.B * w.H * w.n * (w.n + 1) / 2), 4)}


def scaling_report(torch, bd, W, names, runs, per_wl, steps: int, warmup: int) -> dict:
    """The strided workloads at n = 3,072 and 65,536 beside the n = 12,288 one,
    and the growth exponents of the strided pattern over n = 1,024 .. 65,536
    (H = 8 alternating local / stride heads, l = 2^round(log2 sqrt n), 64 x 64
    tiles; host-side layout counts)."""
    out = {"workloads": {}}
    for nm in names:
        out["workloads"][nm] = time_workload(torch, bd, W, W.WORKLOADS[nm], steps, warmup)
    ns = [1 << e for e in range(10, 17)]
    lays = [bd.Layout(n, W.strided_heads(8, 1 << round(math.log2(math.sqrt(n)))), 64, 64) for n in ns]
    out["exponent_pairs"] = round(fit_exponent(ns, [lay.pairs_per_batch() for lay in lays]), 3)
    out["exponent_computed_tile_area"] = round(fit_exponent(ns, [lay.tiles_per_batch() for lay in lays]), 3)
    # time per (batch, head) of the strided workloads against n
    pts = {}
    for nm, r in out["workloads"].items():
        if nm.startswith("strided_n") and "fp32" not in nm:
            pts[r["n"]] = r["ms"] / (r["B"] * r["H"])
    for r in runs:
        w = r["w"]
        if w.name.startswith("strided_n") and w.name in per_wl:
            pts[w.n] = per_wl[w.name]["ms"] / (w.B * w.H)
    if len(pts) >= 2:
        xs = sorted(pts)
        out["exponent_time_per_head_strided"] = round(fit_exponent(xs, [pts[x] for x in xs]), 3)
        out["time_per_head_ms"] = {str(x): round(pts[x], 5) for x in xs}
    out["expected_exponent"] = 1.5
    return out


def fit_exponent(xs, ys) -> float:
    """Least-squares slope of log y against log x."""
    lx = [math.log(x) for x in xs]
    ly = [math.log(y) for y in ys]
    mx, my = sum(lx) / len(lx), sum(ly) / len(ly)
    return sum((a - mx) * (b - my) for a, b in zip(lx, ly)) / sum((a - mx) ** 2 for a in lx)


def sweep_n(args) -> None:
    """O(n sqrt n) check: strided heads with l = 2^round(log2 sqrt n), 64 x 64
    tiles, n = 1,024 ... 65,536; fits the growth exponents of allowed pairs,
    computed-tile area and time."""
    import torch
    from factorized_block_sparse_amd import binding as bd
    from factorized_block_sparse_amd import workloads as W
    rows = []
    for e in range(10, 17):
        n = 1 << e
        l = 1 << round(math.log2(math.sqrt(n)))
        r = time_config(torch, bd, W, n, W.strided_heads(8, l), 64, 64, 1, 2000 + e,
                        args.steps, args.warmup)
        r.update(mode="sweep_n", l=l, dense_causal_pairs=8 * n * (n + 1) // 2)
        r["computed_over_dense_causal"] = round(r["computed_tile_area"] / r["dense_causal_pairs"], 4)
        print(json.dumps(r), flush=True)
        rows.append(r)
    ns = [r["n"] for r in rows]
    big = [r for r in rows if r["n"] >= 8192]
    print(json.dumps({
        "mode": "sweep_n_fit", "pattern": "strided, H=8 alternating local/stride, l=2^round(log2 sqrt n)",
        "exponent_pairs": round(fit_exponent(ns, [r["pairs"] for r in rows]), 3),
        "exponent_computed_tile_flops": round(fit_exponent(ns, [r["computed_tile_area"] for r in rows]), 3),
        "exponent_fwd_bwd_time": round(fit_exponent(ns, [r["fwd_bwd_ms"] for r in rows]), 3),
        "exponent_fwd_bwd_time_n_ge_8192": round(fit_exponent([r["n"] for r in big],
                                                              [r["fwd_bwd_ms"] for r in big]), 3),
        "expected": 1.5}), flush=True)


def crossover(args) -> None:
    """Dense causal attention (a local band as wide as the sequence) against the
    strided pattern (l = 2^round(log2 sqrt n)) in the same kernels, at the same
    number of tokens per call (B = max(1, 16384 / n), H = 8)."""
    import torch
    from factorized_block_sparse_amd import binding as bd
    from factorized_block_sparse_amd import workloads as W
    out = []
    for n in (512, 1024, 2048, 4096, 8192, 16384):
        B = max(1, 16384 // n)
        l = 1 << round(math.log2(math.sqrt(n)))
        dense = time_config(torch, bd, W, n, tuple(W.HeadSpec(W.LOCAL, n) for _ in range(8)), 128, 128,
                            B, 3000 + n, args.steps, args.warmup)
        sparse = min((time_config(torch, bd, W, n, W.strided_heads(8, l), t, t, B, 3000 + n,
                                  args.steps, args.warmup) for t in (32, 64)),
                     key=lambda r: r["fwd_bwd_ms"])
        r = {"mode": "crossover", "n": n, "B": B, "l": l, "dense": dense, "sparse": sparse,
             "fwd_bwd_speedup": round(dense["fwd_bwd_ms"] / sparse["fwd_bwd_ms"], 3),
             "fwd_speedup": round(dense["fwd_ms"] / sparse["fwd_ms"], 3)}
        print(json.dumps(r), flush=True)
        out.append(r)
    slower = [r["n"] for r in out if r["fwd_bwd_speedup"] < 1.0]
    print(json.dumps({"mode": "crossover_summary",
                      "n_where_dense_is_faster": slower,
                      "speedups": {r["n"]: r["fwd_bwd_speedup"] for r in out}}), flush=True)


def natural_order_tile_area(n: int, head, bq: int, bk: int) -> int:
    """Computed tile area of one summary or same-block head if its keys kept
    token order (no packing): a tile pair is computed when it holds a visible
    pair.  Host arithmetic on the head's definition, for the packing report."""
    nqt, nkt = -(-n // bq), -(-n // bk)
    l = head.l
    area = 0
    if head.kind == "sameblock":
        for qt in range(nqt):
            r0, r1 = qt * bq, min(n, (qt + 1) * bq) - 1
            lo = (r0 // l) * l
            area += (r1 // bk - lo // bk + 1) * bq * bk
        return area
    c = head.c
    s = l - ((head.sub % (l // c)) + 1) * c
    first = []  # first summary cell in each key tile (or None)
    for kt in range(nkt):
        j0, j1 = kt * bk, min(n, (kt + 1) * bk) - 1
        hit = None
        for base in range((j0 // l) * l, j1 + 1, l):
            a = max(j0, base + s)
            if a <= min(j1, base + s + c - 1):
                hit = a
                break
        first.append(hit)
    for qt in range(nqt):
        r0, r1 = qt * bq, min(n, (qt + 1) * bq) - 1
        tiles = {kt for kt in range(nkt) if first[kt] is not None and first[kt] <= r1}
        tiles |= {i // bk for i in range(r0, min(r1 + 1, s))}  # rows before the first cell read themselves
        area += len(tiles) * bq * bk
    return area


def summary_width(args) -> None:
    """Small-c summary packing: the fixed pattern at n = 12,288, l = 128,
    c = 8, 16, 32 (B = 2, H = 8 alternating same-block / summary), with the
    tile area that token order would compute beside the packed layout's."""
    import torch
    from factorized_block_sparse_amd import binding as bd
    from factorized_block_sparse_amd import workloads as W
    n, l = 12288, 128
    for c in (8, 16, 32):
        heads = W.fixed_heads(8, l, c)
        for bq, bk in ((128, 128), (128, 64)):
            r = time_config(torch, bd, W, n, heads, bq, bk, 2, 4000 + c, args.steps, args.warmup)
            natural = 2 * sum(natural_order_tile_area(n, h, bq, bk) for h in heads)
            r.update(mode="summary_width", l=l, c=c,
                     natural_order_tile_padding_overhead=round(natural / r["pairs"], 3))
            print(json.dumps(r), flush=True)


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
    ap.add_argument("--no-extra-passes", action="store_true",
                    help="skip the step-distribution, two-stream, cache-cold and GEMM passes "
                         "(for profiler runs that average per-kernel durations)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before the workloads, run one device-to-device copy of this many MiB "
                         "(a plain copy kernel of known size, for scaling HBM byte counters)")
    ap.add_argument("--preroll-ms", type=float, default=250.0,
                    help="untimed steps for this long before the warm-up steps, so that clocks and "
                         "caches settle whatever --warmup is (reported as preroll)")
    ap.add_argument("--scaling-workloads", default="strided_n3072,strided_n65536",
                    help="further workloads timed (forward and forward + backward) after the "
                         "benchmark, reported under scaling; empty to skip")
    ap.add_argument("--no-calibration", action="store_true",
                    help="skip the calibration micro-benchmarks (measured MFMA rate and clock, "
                         "VALU and LDS rates, atomic throughput)")
    ap.add_argument("--sweep-n", action="store_true",
                    help="instead of the benchmark: the O(n sqrt n) sweep, one JSON line per n")
    ap.add_argument("--crossover", action="store_true",
                    help="instead of the benchmark: dense causal vs strided, one JSON line per n")
    ap.add_argument("--summary-width", action="store_true",
                    help="instead of the benchmark: the fixed pattern at c = 8, 16, 32 with packed "
                         "summary tiles, one JSON line per (c, tiles)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported "
              "(the attention path runs on one GPU; batch elements and heads would shard across "
              "GPUs with no communication)",
              file=sys.stderr)
        sys.exit(2)

    if args.sweep_n or args.crossover or args.summary_width:
        (sweep_n if args.sweep_n else crossover if args.crossover else summary_width)(args)
        return

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
    layout_ms = {}
    for w in wls:
        t_lay = time.perf_counter()
        lay = bd.Layout(w.n, w.heads, w.block_q, w.block_k)
        layout_ms[w.name] = round(1000 * (time.perf_counter() - t_lay), 2)
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
            for label, ph in (("bwd_seg", bd.SA_BWD_SEG), ("bwd_dq", bd.SA_BWD_DQ),
                              ("bwd_dkdv", bd.SA_BWD_DKDV), ("bwd_merge", bd.SA_BWD_MERGE)):
                if label == "bwd_merge" and not (split_q or split_k):
                    continue
                if label == "bwd_seg" and lay.header.seg_len == 0:
                    continue
                calls.append((label, lambda lay=lay, q=q, k=k, v=v, o=o, lse=lse, do=do, ws=ws, grads=grads, ph=ph:
                              bd.sparse_attn_bwd(lay, q, k, v, o, lse, do, workspace=ws, grads=grads, phases=ph)))
        useful = (12 if w.backward else 4) * D * pairs
        tiles = lay.tiles_per_batch() * w.B
        runs.append(dict(w=w, lay=lay, calls=calls, pairs=pairs, useful=useful,
                         padding=tiles * w.block_q * w.block_k / pairs,
                         tensors=(q, k, v, do, o, lse, grads, ws, fws, dt)))

    flat = [(r["w"], label, fn) for r in runs for (label, fn) in r["calls"]]

    def step(evs=None):
        for i, (_, _, fn) in enumerate(flat):
            if evs is not None:
                evs[i].record()
            fn()
        if evs is not None:
            evs[len(flat)].record()

    # Pre-roll: untimed steps for a fixed wall time, then the W warm-up steps.
    # Without it a short warm-up leaves the first timed steps slower than the
    # steady state (clocks and caches still settling).
    pre_steps, t_pre = 0, time.perf_counter()
    while (time.perf_counter() - t_pre) * 1000.0 < args.preroll_ms:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
        pre_steps += 10
    preroll = {"steps": pre_steps, "ms": round((time.perf_counter() - t_pre) * 1000.0, 1)}
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

    # Step-time distribution: one event between consecutive steps (each
    # interval includes one event's cost).
    pct, two_ms, cold_ms, gemm, copy = (lambda f: None), None, None, None, None
    if not args.no_extra_passes:
        sev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
        sev[0].record()
        for s in range(K):
            step()
            sev[s + 1].record()
        torch.cuda.synchronize()
        step_ms = sorted(sev[s].elapsed_time(sev[s + 1]) for s in range(K))
        pct = lambda f: round(step_ms[min(K - 1, int(round(f * (K - 1))))], 4)

        # The workloads are independent: with each on its own stream (default
        # priority) the latency-bound strided launches overlap the fixed ones.
        # Reported beside the one-stream value, which stays the headline.
        two_ms = two_stream_step_ms(torch, runs, K) if len(runs) > 1 else None

        # Cache-cold variant: rotate three input sets (more than the 256 MB
        # Infinity Cache in total) so that a step does not find its inputs cached.
        cold_ms = cache_cold_step_ms(torch, bd, runs, K)
        gemm = vendor_gemm_reference(torch)
        copy = vendor_copy_reference(torch)

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
            fl, by = launch_work(label, w, r["lay"])
            kernels.append(dict(workload=w.name, kernel=label, ms=t, flops=fl, bytes=by))
            idx += 1
        tf = r["useful"] / (ms * 1e-3) / 1e12
        alg_bytes = algorithmic_bytes(w)
        fwd_ms = sum(k["ms"] for k in kernels[-len(r["calls"]):] if k["kernel"].startswith("fwd"))
        per_wl[w.name] = {"ms": round(ms, 4), "fwd_ms": round(fwd_ms, 4),
                          "useful_tflops": round(tf, 2),
                          "pct_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
                          "alg_hbm_bytes": alg_bytes,
                          "pct_hbm_roofline": round(100 * alg_bytes / (ms * 1e-3) / (PEAK_HBM_GBS * 1e9), 2),
                          "pct_measured_copy_bandwidth": (round(100 * alg_bytes / (ms * 1e-3) / (copy["hbm_gbs"] * 1e9), 2)
                                                          if copy else None),
                          "pairs": r["pairs"], "tile_padding_overhead": round(r["padding"], 3),
                          "layout_build_ms": layout_ms[w.name]}
    dom = max(kernels, key=lambda k: k["ms"])
    roof = roofline_entry(dom["flops"], dom["bytes"], dom["ms"] * 1e-3)
    roof.update({"traffic": measured_traffic(dom["kernel"], W.WORKLOADS[dom["workload"]]),
                 "kernel": f"{dom['kernel']} ({dom['workload']})",
                 "launch_us": round(dom["ms"] * 1e3, 2), "event_overhead_us": round(event_us, 2)})
    for k in kernels:
        k["ms"] = round(k["ms"], 4)

    calibration = None
    if not args.no_calibration:
        try:
            from factorized_block_sparse_amd import calibration as cal
            calibration = cal.run()
        except Exception as e:  # a reference only; never fails the bench
            calibration = {"error": str(e)}

    scaling = None
    extra = [x for x in args.scaling_workloads.split(",") if x]
    if extra:
        scaling = scaling_report(torch, bd, W, extra, runs, per_wl, K, max(args.warmup, 5))

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
        "pct_of_measured_gemm": round(100 * value / gemm["tflops"], 3) if gemm else None,
        "measured_gemm_reference": gemm,
        "measured_copy_reference": copy,
        "step_ms_p10_p50_p90": [pct(0.1), pct(0.5), pct(0.9)],
        "ms_per_step_cache_cold": round(cold_ms, 4) if cold_ms else None,
        "ms_per_step_two_streams": round(two_ms, 4) if two_ms else None,
        "value_two_streams": round(useful / (two_ms * 1e-3) / 1e12, 3) if two_ms else None,
        "config": {"workload": "+".join(names),
                   "shapes": {w.name: {"B": w.B, "H": w.H, "n": w.n, "d": w.d,
                                       "heads": sorted({h.kind for h in w.heads}),
                                       "tiles": [w.block_q, w.block_k]} for w in wls},
                   "per_workload": per_wl, "kernels": kernels},
        "calibration": calibration,
        "preroll": preroll,
        "length_scaling": scaling,
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernel_sources_sha256": kernel_sources_hash(),
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
