"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Small cases compare every element (several tiles, ragged tails, every head
kind, all tile shapes).  The longest sequence the kernels address compares
sampled rows and keys that the oracle computes one by one, plus invariants
that hold at any size.
"""

import zlib

import numpy as np
import pytest
import torch

from factorized_block_sparse_amd import binding as bd
from factorized_block_sparse_amd import workloads as W
from factorized_block_sparse_amd.binding import HeadPattern, Layout
from oracle import attention as OA
from oracle import masks as OM
from tests.parity_util import (BF16_MAX_ABS, BF16_REL_RMS, FP32_MAX_ABS, LSE_ABS, assert_close,
                               oracle_dense_head, run_gpu, to64)

pytestmark = pytest.mark.gpu

SMALL = [
    # name, B, n, block_q, block_k, heads
    ("strided_tiles64", 2, 512, 64, 64, [HeadPattern("local", 32), HeadPattern("stride", 32)]),
    ("strided_straddle", 1, 576, 64, 64, [HeadPattern("local", 24), HeadPattern("stride", 24)]),
    ("fixed_c32", 1, 768, 64, 64, [HeadPattern("sameblock", 128), HeadPattern("summary", 128, 32, 0),
                                   HeadPattern("summary", 128, 32, 1), HeadPattern("summary", 128, 32, 3)]),
    ("fixed_c8_q128", 1, 640, 128, 64, [HeadPattern("sameblock", 64), HeadPattern("summary", 64, 8, 0),
                                        HeadPattern("summary", 64, 16, 2)]),
    ("ragged_all_kinds", 2, 333, 64, 32, [HeadPattern("local", 17), HeadPattern("stride", 17),
                                          HeadPattern("sameblock", 20), HeadPattern("summary", 20, 3, 1)]),
    ("ragged_q32_k64", 1, 301, 32, 64, [HeadPattern("stride", 10), HeadPattern("summary", 10, 1, 4)]),
    ("tiles32", 1, 256, 32, 32, [HeadPattern("local", 16), HeadPattern("stride", 16)]),
    ("degenerate", 1, 130, 64, 64, [HeadPattern("local", 1000), HeadPattern("stride", 1000),
                                    HeadPattern("summary", 8, 8, 0), HeadPattern("stride", 1)]),
    ("single_row", 1, 1, 64, 64, [HeadPattern("local", 4), HeadPattern("summary", 4, 2, 0)]),
    # rows reading more than 1024 keys: forward / dQ chunks, combine and reduce launches
    ("split_k32", 2, 1500, 64, 32, [HeadPattern("local", 1400), HeadPattern("stride", 1)], 1024),
    ("split_q128_k64", 1, 2200, 128, 64, [HeadPattern("summary", 64, 32, 0), HeadPattern("local", 2100),
                                          HeadPattern("sameblock", 2048)], 1024),
    ("split_default_caps", 1, 3500, 64, 64, [HeadPattern("local", 3300), HeadPattern("summary", 64, 16, 2)]),
    # heads whose rows read a key prefix besides an interval (merged fixed; local + global tokens)
    ("merged_global_tiles64", 2, 700, 64, 64, [HeadPattern("fixed_merged", 128, 32, 0),
                                               HeadPattern("fixed_merged", 128, 32, 3),
                                               HeadPattern("local_global", 64, 16),
                                               HeadPattern("local_global", 100, 0)]),
    ("merged_global_ragged", 1, 333, 64, 32, [HeadPattern("fixed_merged", 20, 3, 1),
                                              HeadPattern("fixed_merged", 8, 8, 0),
                                              HeadPattern("local_global", 17, 5),
                                              HeadPattern("local_global", 3, 64)]),
    ("merged_global_q128_k64", 1, 640, 128, 64, [HeadPattern("fixed_merged", 64, 8, 1),
                                                 HeadPattern("local_global", 32, 40)]),
    ("merged_global_tiles32", 1, 300, 32, 32, [HeadPattern("fixed_merged", 10, 1, 4),
                                               HeadPattern("local_global", 500, 2),
                                               HeadPattern("local_global", 1, 1000)]),
    ("split_merged_global", 1, 2300, 64, 64, [HeadPattern("fixed_merged", 128, 32, 2),
                                              HeadPattern("local_global", 256, 300)], 512),
    # merged strided heads: stride part first, band part starting from its state
    ("strided_merged_tiles64", 2, 700, 64, 64, [HeadPattern("strided_merged", 32),
                                                HeadPattern("local", 32),
                                                HeadPattern("strided_merged", 24),
                                                HeadPattern("summary", 64, 16, 1)]),
    ("strided_merged_ragged", 1, 333, 64, 32, [HeadPattern("strided_merged", 7),
                                               HeadPattern("strided_merged", 1),
                                               HeadPattern("stride", 7),
                                               HeadPattern("strided_merged", 500)]),
    ("strided_merged_tiles32", 1, 300, 32, 32, [HeadPattern("strided_merged", 10),
                                                HeadPattern("fixed_merged", 20, 4, 1)]),
    ("strided_merged_q128_k64", 1, 640, 128, 64, [HeadPattern("strided_merged", 40)]),
    ("split_strided_merged", 1, 2300, 64, 64, [HeadPattern("strided_merged", 1100),
                                               HeadPattern("strided_merged", 16)], 512),
    # stride heads in the segment pass: classes of 125 / 112 rows (four sub-tiles), 78 and
    # 59 rows (three and two), ragged last sub-tiles
    ("stride_segments_4", 2, 1000, 64, 64, [HeadPattern("stride", 8), HeadPattern("local", 8),
                                            HeadPattern("stride", 9)]),
    ("stride_segments_3", 1, 700, 32, 32, [HeadPattern("stride", 9), HeadPattern("stride", 12)]),
    # 128-row query tiles over 32-key tiles (one-wave dK/dV workgroups in two 64-row steps)
    ("tiles128x32", 1, 400, 128, 32, [HeadPattern("local", 40), HeadPattern("stride", 40),
                                      HeadPattern("sameblock", 50), HeadPattern("summary", 64, 8, 1),
                                      HeadPattern("fixed_merged", 32, 4, 2), HeadPattern("strided_merged", 9),
                                      HeadPattern("local_global", 30, 7)]),
    ("split_tiles128x32", 2, 2200, 128, 32, [HeadPattern("local", 2100), HeadPattern("summary", 64, 32, 0),
                                             HeadPattern("fixed_merged", 64, 16, 1)], 1024),
    # 128-key tiles (four waves of 32 keys in the dK/dV pass)
    ("fixed_tiles128", 1, 768, 128, 128, [HeadPattern("sameblock", 128), HeadPattern("summary", 128, 32, 0),
                                          HeadPattern("summary", 128, 32, 3), HeadPattern("local", 100)]),
    ("ragged_tiles128", 1, 333, 128, 128, [HeadPattern("local", 17), HeadPattern("stride", 17),
                                           HeadPattern("sameblock", 20), HeadPattern("summary", 20, 3, 1),
                                           HeadPattern("fixed_merged", 20, 3, 1),
                                           HeadPattern("local_global", 17, 5),
                                           HeadPattern("strided_merged", 7)]),
    ("split_tiles128", 1, 2200, 128, 128, [HeadPattern("summary", 64, 32, 0), HeadPattern("local", 2100),
                                           HeadPattern("sameblock", 2048)], 1024),
    ("split_merged_tiles128", 1, 2300, 128, 128, [HeadPattern("fixed_merged", 128, 32, 2),
                                                  HeadPattern("local_global", 256, 300),
                                                  HeadPattern("strided_merged", 1100)], 512),
]


def _check_dense(layout, heads, B, n, inp, backward=True, fp32=False):
    out = run_gpu(layout, inp, backward)
    q, k, v, do = (to64(inp[x]) for x in ("q", "k", "v", "do"))
    for b in range(B):
        for h, head in enumerate(heads):
            o, lse, g, bar = oracle_dense_head(head, n, q[b, h], k[b, h], v[b, h],
                                               do[b, h] if backward else None, bars=True)
            tag = f"b{b} h{h} {head}"
            if fp32:
                assert_close(f"O {tag}", out["o"][b, h], o, FP32_MAX_ABS)
                assert_close(f"LSE {tag}", out["lse"][b, h], lse, 1e-5)
                continue
            assert_close(f"O {tag}", out["o"][b, h], o, bar["o"], BF16_REL_RMS, bf16_output=True)
            assert_close(f"LSE {tag}", out["lse"][b, h], lse, LSE_ABS)
            if backward:
                for nm, ref in zip(("dq", "dk", "dv"), g):
                    assert_close(f"{nm} {tag}", out[nm][b, h], ref, bar[nm], BF16_REL_RMS, bf16_output=True)
    return out


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_cases_every_element(case):
    name, B, n, bq, bk, heads = case[:6]
    lay = Layout(n, heads, bq, bk, split_keys=case[6] if len(case) > 6 else 0)
    if name.startswith("split"):
        assert lay.header.comb_sched_len > 0
    inp = W.make_inputs(B, len(heads), n, 64, seed=zlib.crc32(name.encode()) % 10000)
    _check_dense(lay, heads, B, n, inp)


STRIDE_CASES = [c for c in SMALL if any(h.kind == "stride" for h in c[5])]


@pytest.mark.parametrize("case", STRIDE_CASES, ids=[c[0] for c in STRIDE_CASES])
def test_stride_heads_through_the_tile_passes(case):
    """The same cases with the segment pass off (SA_NO_SEGMENT_PASS): stride heads run
    through the dQ and dK/dV passes; the default layouts above run them in segments."""
    name, B, n, bq, bk, heads = case[:6]
    lay = Layout(n, heads, bq, bk, split_keys=case[6] if len(case) > 6 else 0, segment_pass=False)
    assert lay.header.seg_len == 0
    inp = W.make_inputs(B, len(heads), n, 64, seed=zlib.crc32(name.encode()) % 10000)
    _check_dense(lay, heads, B, n, inp)


def _random_case(seed):
    rng = np.random.default_rng(9100 + seed)
    n = int(rng.integers(1, 1501))
    bq, bk = [(32, 32), (32, 64), (64, 32), (64, 64), (128, 32), (128, 64), (128, 128)][seed % 7]
    heads = []
    for _ in range(int(rng.integers(1, 5))):
        kind = str(rng.choice(["local", "stride", "sameblock", "summary", "fixed_merged", "local_global",
                               "strided_merged"]))
        l = int(rng.integers(1, 80))
        if kind in ("summary", "fixed_merged"):
            heads.append(HeadPattern(kind, l, int(rng.integers(1, l + 1)), int(rng.integers(0, 6))))
        elif kind == "local_global":
            heads.append(HeadPattern(kind, l, int(rng.integers(0, 40))))
        else:
            heads.append(HeadPattern(kind, l))
    caps = (int(rng.integers(32, 512)), int(rng.integers(32, 512)))
    if (seed // 7) % 2 == 1:
        caps = (0, 0)  # the default caps: few splits, stride heads in the segment pass
    return (int(rng.integers(1, 3)), n, bq, bk, heads) + caps


@pytest.mark.parametrize("seed", range(28))
def test_random_small_layouts_every_element(seed):
    """Seeded random layouts (n up to 1,500, one to four heads of any kind with random
    l, c and sub-block, every tile shape; random chunk caps so that tiles split, or the
    default caps): every element of O, LSE, dQ, dK, dV against the oracle."""
    B, n, bq, bk, heads, sk, sr = _random_case(seed)
    print(f"seed {seed}: B={B} n={n} tiles={bq}x{bk} caps={sk},{sr} heads={heads}", flush=True)
    lay = Layout(n, heads, bq, bk, split_keys=sk, split_rows=sr)
    inp = W.make_inputs(B, len(heads), n, 64, seed=9200 + seed)
    _check_dense(lay, heads, B, n, inp)


@pytest.mark.parametrize("seed", range(6))
def test_fp32_forward_random_layouts(seed):
    """float32 forward on seeded random layouts (query tiles 32, 64, 128 over 32-key
    tiles; random caps): every element of O and LSE."""
    B, n, _, _, heads, sk, _ = _random_case(100 + seed)
    # two-part heads run in bf16 only (SA_EUNSUPPORTED for float32): their stride part instead
    heads = [HeadPattern("stride", h.l) if h.kind == "strided_merged" else h for h in heads]
    bq = (32, 64, 128)[seed % 3]
    print(f"fp32 seed {seed}: B={B} n={n} tiles={bq}x32 cap={sk} heads={heads}", flush=True)
    lay = Layout(n, heads, bq, 32, split_keys=sk)
    inp = W.make_inputs(B, len(heads), n, 64, seed=9300 + seed, dtype="fp32")
    _check_dense(lay, heads, B, n, inp, backward=False, fp32=True)


def test_fp32_forward_small_ragged():
    heads = [HeadPattern("local", 9), HeadPattern("stride", 9), HeadPattern("summary", 9, 3, 0)]
    lay = Layout(200, heads, 32, 32)
    inp = W.make_inputs(1, 3, 200, 64, seed=5, dtype="fp32")
    _check_dense(lay, heads, 1, 200, inp, backward=False, fp32=True)


def test_fp32_forward_split_rows():
    heads = [HeadPattern("local", 1100), HeadPattern("stride", 2)]
    lay = Layout(1100, heads, 64, 32, split_keys=1024)
    assert lay.header.comb_sched_len > 0
    inp = W.make_inputs(1, 2, 1100, 64, seed=6, dtype="fp32")
    _check_dense(lay, heads, 1, 1100, inp, backward=False, fp32=True)


def test_fp32_forward_query_tiles128():
    """float32 forward with 128-row query tiles (four waves), ragged and split."""
    heads = [HeadPattern("local", 9), HeadPattern("stride", 9), HeadPattern("summary", 9, 3, 0),
             HeadPattern("sameblock", 100), HeadPattern("fixed_merged", 20, 4, 1),
             HeadPattern("local_global", 12, 5)]
    lay = Layout(333, heads, 128, 32)
    inp = W.make_inputs(2, len(heads), 333, 64, seed=15, dtype="fp32")
    _check_dense(lay, heads, 2, 333, inp, backward=False, fp32=True)
    heads = [HeadPattern("local", 1300), HeadPattern("summary", 64, 16, 2)]
    lay = Layout(1400, heads, 128, 32, split_keys=512)
    assert lay.header.comb_sched_len > 0
    inp = W.make_inputs(1, 2, 1400, 64, seed=16, dtype="fp32")
    _check_dense(lay, heads, 1, 1400, inp, backward=False, fp32=True)


def test_workload_strided_n1024_fp32_full():
    """Strided pattern, forward only, float32, 32x32 tiles: every element."""
    w = W.WORKLOADS["strided_n1024_fp32"]
    lay = Layout(w.n, w.heads, w.block_q, w.block_k)
    _check_dense(lay, w.heads, w.B, w.n, W.workload_inputs(w), backward=False, fp32=True)


def test_workload_strided_n3072_full():
    """Strided pattern n = 3072, B = 4, H = 8: every element of every (b, h)."""
    w = W.WORKLOADS["strided_n3072"]
    lay = Layout(w.n, w.heads, w.block_q, w.block_k)
    _check_dense(lay, w.heads, w.B, w.n, W.workload_inputs(w))


def test_empty_batch_is_a_no_op():
    heads = [HeadPattern("local", 8), HeadPattern("stride", 8)]
    lay = Layout(64, heads, 64, 64)
    q = torch.zeros((0, 2, 64, 64), dtype=torch.bfloat16, device="cuda:0")
    o, lse = bd.sparse_attn_fwd(lay, q, q, q)
    dq, dk, dv = bd.sparse_attn_bwd(lay, q, q, q, o, lse, q)
    torch.cuda.synchronize()
    assert o.numel() == 0 and dq.numel() == 0


def test_binding_rejects_mismatched_outputs_before_any_launch():
    """Outputs, LSE and workspaces are written through raw pointers: the binding
    refuses tensors of the wrong shape, dtype or device instead of launching."""
    heads = [HeadPattern("local", 8), HeadPattern("stride", 8)]
    lay = Layout(64, heads, 64, 64)
    dev = torch.device("cuda:0")
    q = torch.zeros((1, 2, 64, 64), dtype=torch.bfloat16, device=dev)
    lse = torch.zeros((1, 2, 64), dtype=torch.float32, device=dev)
    bad = [dict(out=torch.zeros((1, 2, 32, 64), dtype=torch.bfloat16, device=dev)),
           dict(out=torch.zeros((1, 2, 64, 64), dtype=torch.float32, device=dev)),
           dict(lse=torch.zeros((1, 2, 32), dtype=torch.float32, device=dev)),
           dict(lse=torch.zeros((1, 2, 64), dtype=torch.bfloat16, device=dev)),
           dict(workspace=torch.zeros(64, dtype=torch.float32, device=dev))]
    for kw in bad:
        with pytest.raises(ValueError):
            bd.sparse_attn_fwd(lay, q, q, q, **kw)
    with pytest.raises(ValueError):
        bd.sparse_attn_bwd(lay, q, q, q, q, lse, q, grads=(q, q, q[:, :, :32]))
    with pytest.raises(ValueError):
        bd.sparse_attn_bwd(lay, q, q, q, q, lse[:, :1], q)
    with pytest.raises(ValueError):
        bd.sparse_attn_bwd(lay, q, q, q, q, lse, q, workspace=torch.zeros(8, dtype=torch.int32, device=dev))
    torch.cuda.synchronize()


def test_repeat_calls_are_bitwise_deterministic():
    """No atomics; split tiles are merged in chunk order: forward and backward reproduce
    bit for bit, with the same workspaces reused across calls."""
    heads = [HeadPattern("sameblock", 64), HeadPattern("summary", 64, 16, 0)]
    lay = Layout(4096, heads, 64, 64, split_keys=512)
    h = lay.header
    assert h.num_slots > 0 and h.num_qslots > 0  # split key and query tiles
    inp = W.make_inputs(1, 2, 4096, 64, seed=77)
    dev = torch.device("cuda:0")
    q, k, v, do = (inp[x].to(dev) for x in ("q", "k", "v", "do"))
    fws = torch.empty(bd.fwd_workspace_bytes(lay, 1, 2), dtype=torch.uint8, device=dev)
    bws = torch.empty(bd.bwd_workspace_bytes(lay, 1, 2), dtype=torch.uint8, device=dev)
    runs = []
    for _ in range(3):
        o, lse = bd.sparse_attn_fwd(lay, q, k, v, workspace=fws)
        grads = bd.sparse_attn_bwd(lay, q, k, v, o, lse, do, workspace=bws)
        torch.cuda.synchronize()
        runs.append([to64(t) for t in (o, lse, *grads)])
    for r in runs[1:]:
        for name, x, y in zip(("o", "lse", "dq", "dk", "dv"), runs[0], r):
            assert np.array_equal(x, y), name


def test_unsplit_long_tile_lists_every_element():
    """Splitting off: CSR and CSC lists of well over 64 tiles (the kernels walk them
    through 64-entry register windows)."""
    heads = [HeadPattern("local", 4800), HeadPattern("summary", 64, 16, 0)]
    n = 5000
    lay = Layout(n, heads, 32, 32, split_keys=1 << 30, split_rows=1 << 30)
    h = lay.header
    assert h.comb_sched_len == 0 and h.red_sched_len == 0
    fs, bs = lay.fwd_schedule(), lay.bwd_schedule()
    assert max(fs[:, 3] - fs[:, 2]) > 128 and max(bs[:, 3] - bs[:, 2]) > 128
    inp = W.make_inputs(1, len(heads), n, 64, seed=9090)
    _check_dense(lay, heads, 1, n, inp)


def test_many_chunks_per_tile_every_element():
    """Small chunk caps: up to a dozen chunks per split tile."""
    heads = [HeadPattern("local", 600), HeadPattern("summary", 32, 8, 1), HeadPattern("stride", 3)]
    n, B = 700, 2
    lay = Layout(n, heads, 32, 32, split_keys=64, split_rows=64)
    fs, bs = lay.fwd_schedule(), lay.bwd_schedule()
    assert max(fs[:, 7]) >= 8 and max(bs[:, 7]) >= 8
    inp = W.make_inputs(B, len(heads), n, 64, seed=4242)
    _check_dense(lay, heads, B, n, inp)


def test_masked_value_perturbation_on_gpu():
    """Blog post on sliding windows, section 10: a masked key's value cannot reach a row."""
    heads = [HeadPattern("local", 8), HeadPattern("stride", 8)]
    n = 256
    lay = Layout(n, heads, 64, 64)
    inp = W.make_inputs(1, 2, n, 64, seed=3)
    base = run_gpu(lay, inp, False)
    j = 100
    inp2 = dict(inp)
    v2 = inp["v"].clone()
    v2[:, :, j] += 10000
    inp2["v"] = v2
    pert = run_gpu(lay, inp2, False)
    for h, head in enumerate(heads):
        blind = ~OM.head_mask(n, head.kind, head.l)[:, j]
        assert np.array_equal(base["o"][0, h][blind], pert["o"][0, h][blind])
        assert not np.allclose(base["o"][0, h][~blind], pert["o"][0, h][~blind])


# ----------------------------------------------------------------------------
# The longest sequence: sampled rows / keys + invariants (every element of the
# full-size workloads is in test_gpu_full_size.py)
# ----------------------------------------------------------------------------

def _compact(tokens):
    """Sorted token universe and a map from token arrays to indices into it."""
    u = np.unique(np.concatenate([np.asarray(t, dtype=np.int64).ravel() for t in tokens]))
    return u, (lambda a: np.searchsorted(u, np.asarray(a, dtype=np.int64)))


@pytest.mark.skipif(not torch.cuda.is_available() or
                    torch.cuda.get_device_properties(0).total_memory < (120 << 30),
                    reason="needs a GPU with 120 GB for 8 tensors of 8.6 GB")
def test_longest_bf16_sequence_sampled():
    """n = 2^25 - 64, the longest bf16 sequence the kernels address (a (b, h)
    slice spans just under 4 GB of 32-bit byte offsets): sampled rows and keys
    at both ends against the oracle, on gathered rows, plus the gradient
    invariants over every row on the GPU."""
    n = (1 << 25) - 64
    heads = [HeadPattern("local", 16), HeadPattern("stride", 1 << 20)]
    lay = Layout(n, heads, 64, 64)
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(25)
    shape = (1, 2, n, 64)
    q, k, v, do = (torch.randn(shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
                   for _ in range(4))
    o, lse = bd.sparse_attn_fwd(lay, q, k, v)
    dq, dk, dv = bd.sparse_attn_bwd(lay, q, k, v, o, lse, do)
    torch.cuda.synchronize()
    for h, head in enumerate(heads):
        args = (head.kind, n, head.l)
        rows = [0, 1, 17, n // 2, (1 << 24) + 5, n - 65, n - 2, n - 1]
        keys = [0, 5, n - 40, n - 17, n - 1]
        rkeys = {i: OM.row_keys(head.kind, i, n, head.l) for i in rows}
        seers = {j: OM.rows_seeing(head.kind, j, n, head.l) for j in keys}
        skeys = {int(i): OM.row_keys(head.kind, int(i), n, head.l) for j in keys for i in seers[j]}
        u, m = _compact([rows, keys, *rkeys.values(), *seers.values(), *skeys.values()])
        ut = torch.from_numpy(u).to(dev)
        qc, kc, vc, doc = (to64(t[0, h].index_select(0, ut)) for t in (q, k, v, do))
        kf = lambda ic: m(OM.row_keys(head.kind, int(u[ic]), n, head.l))
        rf = lambda jc: m(OM.rows_seeing(head.kind, int(u[jc]), n, head.l))
        rc, kc_ids = m(rows), m(keys)
        ro, rl = OA.fwd_rows(qc, kc, vc, kf, rc)
        rdq = OA.bwd_rows_dq(qc, kc, vc, doc, kf, rc)
        rdk, rdv = OA.bwd_keys_dkdv(qc, kc, vc, doc, kf, rf, kc_ids)
        ri, ki = torch.tensor(rows, device=dev), torch.tensor(keys, device=dev)
        tag = f"n={n} h{h} {head.kind}"
        assert_close(f"O {tag}", to64(o[0, h].index_select(0, ri)), ro, BF16_MAX_ABS, BF16_REL_RMS, bf16_output=True)
        assert_close(f"LSE {tag}", to64(lse[0, h].index_select(0, ri)), rl, LSE_ABS)
        assert_close(f"dQ {tag}", to64(dq[0, h].index_select(0, ri)), rdq, BF16_MAX_ABS, BF16_REL_RMS, bf16_output=True)
        assert_close(f"dK {tag}", to64(dk[0, h].index_select(0, ki)), rdk, BF16_MAX_ABS, BF16_REL_RMS, bf16_output=True)
        assert_close(f"dV {tag}", to64(dv[0, h].index_select(0, ki)), rdv, BF16_MAX_ABS, BF16_REL_RMS, bf16_output=True)
        # every row: sum_j dK_j = 0 (scores are shift-invariant in the keys),
        # sum_j dV_j = sum_i dO_i (probability rows sum to one)
        sk = dk[0, h].float().sum(0)
        assert float(sk.abs().max()) <= 2e-2 * float(dk[0, h].float().abs().sum(0).max()) + 1e-3
        sv, sd = dv[0, h].float().sum(0), do[0, h].float().sum(0)
        assert float((sv - sd).abs().max()) <= 1e-2 * float(dv[0, h].float().abs().sum(0).max()) + 1e-2
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(dq).all())
