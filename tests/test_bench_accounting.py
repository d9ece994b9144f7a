"""The benchmark's accounting (host arithmetic, no GPU): useful FLOPs and
algorithmic bytes against the figures the survey of the pages states for the
n = 12,288 workloads, the roofline choice, the exponent fit, and the
token-order tile area of the packing report against a brute-force count from
the oracle's masks."""

import math

import numpy as np
import pytest

import bench
from factorized_block_sparse_amd import workloads as W
from oracle import masks as OM


def test_algorithmic_bytes_of_the_n12288_workloads():
    # Forward: Q, K, V read, O written (4 rows of 64 bf16) + LSE; backward:
    # Q, K, V, O, dO read, dQ, dK, dV written (8 rows) + LSE and D.
    # B*H = 16 rows of n = 12,288 for both workloads: 101.4 MB + 202.9 MB.
    for name in ("fixed_n12288", "strided_n12288"):
        w = W.WORKLOADS[name]
        rows = w.B * w.H * w.n
        assert rows == 196608
        assert bench.algorithmic_bytes(w) == rows * (4 * 64 * 2 + 4) + rows * (8 * 64 * 2 + 8)
    assert round(196608 * 516 / 1e6, 1) == 101.4 and round(196608 * 1032 / 1e6, 1) == 202.9


def test_useful_flops_add_up_to_the_metric():
    # 4 d per visible pair forward, 8 d backward (dQ 2 d in the query-tile
    # pass, dV, dP, dK 6 d in the key-tile pass): 12 d per pair in all.
    pairs = 157348224  # the fixed workload's visible pairs over all (b, h)
    B, H, n = 2, 8, 12288
    total = sum(bench.kernel_work(k, B, H, n, pairs)[0] for k in ("fwd", "bwd_dq", "bwd_dkdv"))
    assert total == 12 * 64 * pairs
    assert round(total / 1e9, 1) == 120.8  # the survey's C3 total, GFLOP
    assert bench.kernel_work("bwd_merge", B, H, n, pairs) == (0, 0)
    with pytest.raises(ValueError):
        bench.kernel_work("nope", B, H, n, pairs)


def test_roofline_entry_picks_the_binding_resource():
    ridge = bench.PEAK_BF16_TFLOPS * 1e12 / (bench.PEAK_HBM_GBS * 1e9)
    assert ridge == pytest.approx(312.5)
    r = bench.roofline_entry(flops=400e9, nbytes=1e9, seconds=1e-3)  # 400 flop/B: MFMA side
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["achieved"] == pytest.approx(400.0) and r["frac"] == pytest.approx(400.0 / 2500.0)
    r = bench.roofline_entry(flops=44e9, nbytes=1e9, seconds=1e-3)  # 44 flop/B: HBM side
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["achieved"] == pytest.approx(1000.0) and r["frac"] == pytest.approx(1000.0 / 8000.0)


def test_fit_exponent_recovers_power_laws():
    xs = [1024 * 2 ** i for i in range(7)]
    for e in (1.0, 1.5, 2.0):
        assert bench.fit_exponent(xs, [3.0 * x ** e for x in xs]) == pytest.approx(e)
    # The sweep's strided heads (l = 2^round(log2 sqrt n)) over n = 1,024 ..
    # 65,536: the visible pairs of the layouts grow as n sqrt n.
    from factorized_block_sparse_amd import binding as bd
    pairs = [bd.Layout(n, W.strided_heads(8, 1 << round(math.log2(math.sqrt(n)))), 64, 64).pairs_per_batch()
             for n in xs]
    assert bench.fit_exponent(xs, pairs) == pytest.approx(1.497, abs=2e-3)


def _brute_tile_area(n, kind, l, c, sub, bq, bk):
    m = OM.head_mask(n, kind, l, c, sub)  # token order, self-if-empty included
    nqt, nkt = -(-n // bq), -(-n // bk)
    area = 0
    for qt in range(nqt):
        for kt in range(nkt):
            if m[qt * bq:(qt + 1) * bq, kt * bk:(kt + 1) * bk].any():
                area += bq * bk
    return area


@pytest.mark.parametrize("n,l,c,sub,bq,bk", [(512, 64, 8, 0, 64, 64), (768, 128, 32, 1, 128, 64),
                                            (640, 64, 16, 2, 128, 128), (300, 32, 4, 3, 32, 32)])
def test_token_order_tile_area_matches_brute_force(n, l, c, sub, bq, bk):
    head = W.HeadSpec(W.SUMMARY, l, c, sub)
    assert bench.natural_order_tile_area(n, head, bq, bk) == _brute_tile_area(n, OM.SUMMARY, l, c, sub, bq, bk)
    same = W.HeadSpec(W.SAMEBLOCK, l)
    assert bench.natural_order_tile_area(n, same, bq, bk) == _brute_tile_area(n, OM.SAMEBLOCK, l, None, 0, bq, bk)


def test_kernel_bytes_count_every_tensor_the_kernel_moves():
    """bwd_dq reads Q, K, V, O, dO and writes dQ (six rows of 64 bf16) plus LSE
    and D; bwd_dkdv reads Q, K, V, dO and writes dK, dV (six rows) plus LSE and
    D: 152.6 MB each at n = 12,288 with B * H = 16."""
    rows = 2 * 8 * 12288
    assert bench.kernel_work("bwd_dq", 2, 8, 12288, 1)[1] == rows * (6 * 64 * 2 + 8)
    assert bench.kernel_work("bwd_dkdv", 2, 8, 12288, 1)[1] == rows * (6 * 64 * 2 + 8)
    assert round(rows * 776 / 1e6, 1) == 152.6
    assert bench.kernel_work("fwd", 2, 8, 12288, 1)[1] == rows * (4 * 64 * 2 + 4)


def test_cpu_baseline_task_runs_what_it_counts(monkeypatch):
    """The CPU leg counts 12 d FLOPs per visible key (4 d forward, 8 d backward),
    so each task must run both the oracle's forward and its backward."""
    import time
    from oracle import attention as OA
    calls = []
    real_f, real_b = OA.fwd_rows, OA.bwd_rows_full
    monkeypatch.setattr(OA, "fwd_rows", lambda *a, **k: calls.append("fwd") or real_f(*a, **k))
    monkeypatch.setattr(OA, "bwd_rows_full", lambda *a, **k: calls.append("bwd") or real_b(*a, **k))
    n = 64
    rng = np.random.default_rng(0)
    q, k, v, do = (rng.standard_normal((n, 64)) for _ in range(4))
    head = W.HeadSpec(W.LOCAL, 5)
    bench._CPU[("t", 0, 0)] = (q, k, v, do, head, n)
    rows = [0, 3, 40]
    done, fl = bench._cpu_task((("t", 0, 0), rows, time.time() + 60))
    assert sorted(calls) == ["bwd", "fwd"] and done == 3
    assert fl == 12 * 64 * sum(OM.row_keys(OM.LOCAL, i, n, 5).size for i in rows)


def test_segment_pass_takes_its_heads_out_of_the_tile_passes():
    """Strided n = 12,288: the segment pass carries the eight stride heads (8 d per
    pair), the dQ and dK/dV passes the eight local heads; the useful FLOPs still add
    up to 12 d per visible pair."""
    from factorized_block_sparse_amd import binding as bd
    w = W.WORKLOADS["strided_n12288"]
    lay = bd.Layout(w.n, w.heads, w.block_q, w.block_k)
    hs, ps = bench.segment_heads(lay)
    assert hs == 8 and lay.header.seg_len == 8 * 128 and lay.header.seg_tiles == 3
    stride_pairs = sum(OM.row_keys(OM.STRIDE, i, w.n, 128).size for i in range(w.n))
    assert ps == 8 * stride_pairs
    total = sum(bench.launch_work(k, w, lay)[0] for k in ("fwd", "bwd_seg", "bwd_dq", "bwd_dkdv"))
    assert total == 12 * 64 * lay.pairs_per_batch() * w.B
    rows = w.B * 8 * w.n
    assert bench.launch_work("bwd_seg", w, lay)[1] == rows * (8 * 64 * 2 + 4)
    assert bench.launch_work("bwd_dq", w, lay)[1] == rows * (6 * 64 * 2 + 8)
    off = bd.Layout(w.n, w.heads, w.block_q, w.block_k, segment_pass=False)
    assert bench.segment_heads(off) == (0, 0)
    assert bench.launch_work("bwd_dq", w, off) == bench.kernel_work("bwd_dq", w.B, w.H, w.n,
                                                                   off.pairs_per_batch() * w.B)


def test_bench_line_has_no_duplicate_keys():
    """The JSON line is one dict literal: a repeated key would silently replace a
    contract field (e.g. "scaling": "weak")."""
    import ast
    import os
    src = open(os.path.join(os.path.dirname(bench.__file__), "bench.py")).read()
    found = 0
    for node in ast.walk(ast.parse(src)):
        if isinstance(node, ast.Assign) and any(getattr(t, "id", None) == "line" for t in node.targets) \
                and isinstance(node.value, ast.Dict):
            keys = [k.value for k in node.value.keys if isinstance(k, ast.Constant)]
            assert len(keys) == len(set(keys)), sorted(k for k in keys if keys.count(k) > 1)
            assert {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                    "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                    "roofline", "cpu_baseline"} <= set(keys)
            found += 1
    assert found == 1
