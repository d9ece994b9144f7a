"""Host layout builder (C ABI, no GPU): bit-exact against the oracle's token masks.

The reference tiles are derived here, in test code: the documented index
maps (identity; residue-class order for the stride head; summary cells first
for the summary and merged fixed heads) are rebuilt independently, the oracle's dense token
mask is permuted by them, and a tile is active iff any entry in it is set and
FULL iff all are.  CSR, CSC, flags, per-row intervals and per-token counts
must match bit for bit.
"""

import ctypes
import os
import subprocess
import tempfile

import numpy as np
import pytest

from oracle import masks as M
from factorized_block_sparse_amd import binding as bd
from factorized_block_sparse_amd import workloads as W
from factorized_block_sparse_amd.binding import HeadPattern, Layout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _doc_maps(kind, n, n_pad, l, c=0, sub=0):
    """Documented layout-space maps (query map, key map), -1 past n."""
    qmap = -np.ones(n_pad, dtype=np.int64)
    kmap = -np.ones(n_pad, dtype=np.int64)
    if kind in ("local", "sameblock", "local_global"):
        qmap[:n] = kmap[:n] = np.arange(n)
    elif kind == "fixed_merged":
        s = M.summary_start(l, c, sub)
        qmap[:n] = np.arange(n)
        cells = [j for j in range(n) if s <= j % l <= s + c - 1]
        kmap[:n] = cells + [j for j in range(n) if not s <= j % l <= s + c - 1]
    elif kind == "stride":
        order = sorted(range(n), key=lambda i: (i % l, i // l))
        qmap[:n] = kmap[:n] = order
    else:
        s = M.summary_start(l, c, sub)
        qmap[:n] = np.arange(n)
        cells = [j for j in range(n) if s <= j % l <= s + c - 1]
        empty = [i for i in range(n) if M.row_keys(M.SUMMARY, i, n, l, c, sub, self_if_empty=False).size == 0]
        taken = set(cells) | set(empty)
        rest = [j for j in range(n) if j not in taken]
        kmap[:n] = cells + empty + rest
    return qmap, kmap


def _ref_tiles(mp, bq, bk):
    n_pad = mp.shape[0]
    nqt, nkt = n_pad // bq, n_pad // bk
    t = mp.reshape(nqt, bq, nkt, bk)
    active = t.any(axis=(1, 3))
    full = t.all(axis=(1, 3))
    row_ptr = np.concatenate([[0], np.cumsum(active.sum(1))]).astype(np.int32)
    qt_idx, kt_idx = np.nonzero(active)  # row-major: CSR order, ascending k-tiles
    col = kt_idx.astype(np.int32)
    fflag = full[qt_idx, kt_idx].astype(np.uint8)
    col_ptr = np.concatenate([[0], np.cumsum(active.sum(0))]).astype(np.int32)
    kt2, qt2 = np.nonzero(active.T)
    return row_ptr, col, fflag, col_ptr, qt2.astype(np.int32), full.T[kt2, qt2].astype(np.uint8)


CASES = [
    # (n, block_q, block_k, heads)
    (256, 64, 64, [HeadPattern("local", 16), HeadPattern("stride", 16)]),
    (1024, 32, 32, [HeadPattern("local", 32), HeadPattern("stride", 32)]),
    (384, 64, 64, [HeadPattern("local", 64), HeadPattern("stride", 64)]),
    (576, 64, 64, [HeadPattern("local", 24), HeadPattern("stride", 24)]),   # class length 24: straddling tiles
    (512, 64, 64, [HeadPattern("sameblock", 128), HeadPattern("summary", 128, 32, 0),
                   HeadPattern("summary", 128, 32, 1), HeadPattern("summary", 128, 32, 2),
                   HeadPattern("summary", 128, 32, 3)]),
    (512, 128, 64, [HeadPattern("sameblock", 64), HeadPattern("summary", 64, 8, 0),
                    HeadPattern("summary", 64, 16, 2)]),
    (300, 64, 32, [HeadPattern("local", 17), HeadPattern("stride", 17), HeadPattern("sameblock", 20),
                   HeadPattern("summary", 20, 3, 1)]),                          # ragged everywhere
    (97, 32, 64, [HeadPattern("stride", 10), HeadPattern("summary", 10, 1, 4)]),
    (1, 32, 32, [HeadPattern("local", 1), HeadPattern("summary", 4, 2, 0)]),
    (200, 64, 64, [HeadPattern("local", 500), HeadPattern("stride", 500), HeadPattern("summary", 8, 8, 0)]),
    (512, 64, 64, [HeadPattern("fixed_merged", 128, 32, 0), HeadPattern("fixed_merged", 128, 32, 3),
                   HeadPattern("local_global", 64, 16), HeadPattern("local_global", 100, 0)]),
    (300, 64, 32, [HeadPattern("fixed_merged", 20, 3, 1), HeadPattern("fixed_merged", 8, 8, 0),
                   HeadPattern("fixed_merged", 6, 1, 5), HeadPattern("local_global", 17, 5),
                   HeadPattern("local_global", 3, 64), HeadPattern("local_global", 1, 1000)]),
    (97, 32, 64, [HeadPattern("fixed_merged", 10, 1, 4), HeadPattern("local_global", 500, 2)]),
    (1, 32, 32, [HeadPattern("fixed_merged", 4, 2, 0), HeadPattern("local_global", 4, 3)]),
]


@pytest.mark.parametrize("n,bq,bk,heads", CASES)
def test_layout_bit_exact(n, bq, bk, heads):
    lay = Layout(n, heads, bq, bk)
    h = lay.header
    t = max(bq, bk)
    n_pad = -(-n // t) * t
    assert (h.magic, h.n, h.n_pad, h.nqt, h.nkt) == (bd.SA_BLOB_MAGIC, n, n_pad, n_pad // bq, n_pad // bk)
    hp = lay.head_pattern_index()
    total_pairs = 0
    for hi_, head in enumerate(heads):
        arr = lay.pattern_arrays(int(hp[hi_]))
        rec = lay.pattern_rec(int(hp[hi_]))
        qmap, kmap = _doc_maps(head.kind, n, n_pad, head.l, head.c, head.sub)
        np.testing.assert_array_equal(arr["qmap"], qmap)
        np.testing.assert_array_equal(arr["kmap"], kmap)
        mask = M.head_mask(n, head.kind, head.l, head.c or None, head.sub)
        mp = np.zeros((n_pad, n_pad), dtype=bool)
        mp[:n, :n] = mask[np.ix_(qmap[:n], kmap[:n])]
        # Every layout row reads exactly a prefix [0, pre) and one interval
        # [lo, hi], the prefix before the interval.
        cols = np.arange(n_pad)
        lo, hi, pre = arr["lo"], arr["hi"], arr["pre"]
        interval = (cols[None, :] >= lo[:, None]) & (cols[None, :] <= hi[:, None])
        np.testing.assert_array_equal(interval | (cols[None, :] < pre[:, None]), mp)
        assert ((pre <= lo) | (lo > hi)).all()
        if head.kind not in ("fixed_merged", "local_global"):
            assert rec.pre_off == 0 and not pre.any()
        # No prefix array at all when every prefix is empty (kernels must not read one).
        assert (rec.pre_off == 0) == (not pre.any())
        np.testing.assert_array_equal(arr["count"], mask.sum(1))
        assert rec.pairs == mask.sum()
        total_pairs += int(mask.sum())
        ref = _ref_tiles(mp, bq, bk)
        for name, r in zip(("row_ptr", "col", "fflag", "col_ptr", "row", "bflag"), ref):
            np.testing.assert_array_equal(arr[name], r, err_msg=f"{head} {name}")
        assert rec.nnz == len(ref[1])
    assert lay.pairs_per_batch() == total_pairs


def _check_pattern_from_rows(lay, pi, kind, n, keys_of, qmap, kmap, bq, bk, tag):
    """One pattern of a built layout against a reference made from the oracle's
    per-row key lists (no n x n mask): maps, per-token counts, each layout row
    reading exactly its prefix and interval, active / FULL tiles, CSR and CSC."""
    h = lay.header
    n_pad, nqt, nkt = h.n_pad, h.nqt, h.nkt
    arr, rec = lay.pattern_arrays(pi), lay.pattern_rec(pi)
    np.testing.assert_array_equal(arr["qmap"], qmap, err_msg=f"{tag} qmap")
    np.testing.assert_array_equal(arr["kmap"], kmap, err_msg=f"{tag} kmap")
    kpos = np.empty(n, dtype=np.int64)
    kpos[kmap[:n]] = np.arange(n)
    count = np.zeros(n, dtype=np.int64)
    tiles = np.zeros((nqt, nkt), dtype=np.int64)
    lo, hi, pre = arr["lo"].astype(np.int64), arr["hi"].astype(np.int64), arr["pre"].astype(np.int64)
    pairs = 0
    for qt in range(nqt):
        kts = []
        for p in range(qt * bq, (qt + 1) * bq):
            t = int(qmap[p])
            if t < 0:
                assert pre[p] == 0 and lo[p] > hi[p], f"{tag} padding row {p}"
                continue
            kp = np.sort(kpos[keys_of(t)])
            count[t] = kp.size
            pairs += kp.size
            a, b, c0 = int(lo[p]), int(hi[p]), int(pre[p])
            span = np.arange(a, b + 1) if a <= b else np.zeros(0, dtype=np.int64)
            expect = np.concatenate([np.arange(c0), span])
            assert kp.size == expect.size and (kp == expect).all(), f"{tag} row {p} (token {t})"
            kts.append(kp // bk)
        if kts:
            tiles[qt] = np.bincount(np.concatenate(kts), minlength=nkt)
    np.testing.assert_array_equal(arr["count"], count, err_msg=f"{tag} count")
    assert rec.pairs == pairs and rec.kind == kind
    active, full = tiles > 0, tiles == bq * bk
    row_ptr = np.concatenate([[0], np.cumsum(active.sum(1))])
    qi, ki = np.nonzero(active)
    col_ptr = np.concatenate([[0], np.cumsum(active.sum(0))])
    kj, qj = np.nonzero(active.T)
    ref = {"row_ptr": row_ptr, "col": ki, "fflag": full[qi, ki], "col_ptr": col_ptr, "row": qj,
           "bflag": full.T[kj, qj]}
    for name, r in ref.items():
        np.testing.assert_array_equal(arr[name], np.asarray(r).astype(arr[name].dtype),
                                      err_msg=f"{tag} {name}")
    assert rec.nnz == len(ki)


@pytest.mark.parametrize("wname", list(W.WORKLOADS))
def test_workload_layouts_bit_exact_from_oracle_rows(wname):
    """The layouts the benchmark and the full-size parity tests run, at their real n and
    tiles (strided n = 3,072 on 64x64, fixed n = 12,288 on 128x128, strided n = 12,288
    on 32x32, strided n = 65,536 on 64x64, and the union workloads), bit for bit
    against tiles built from the oracle's row key lists."""
    w = W.WORKLOADS[wname]
    lay = Layout(w.n, w.heads, w.block_q, w.block_k)
    h = lay.header
    n, n_pad = w.n, h.n_pad
    hp = lay.head_pattern_index()
    part, _ = lay.head_parts()
    seen = set()
    for hi_, head in enumerate(w.heads):
        c = head.c or None
        if head.kind == "strided_merged":
            # two parts with disjoint key sets: the local band, then the stride
            # members at distance >= 2 l (residue-class order)
            parts = [(int(hp[hi_]), bd.KINDS["local"], "local",
                      lambda t, l=head.l: M.row_keys(M.LOCAL, t, n, l)),
                     (int(part[hi_]), bd.SA_STRIDE_FAR, "stride",
                      lambda t, l=head.l: np.setdiff1d(M.row_keys(M.STRIDE, t, n, l),
                                                       M.row_keys(M.LOCAL, t, n, l)))]
        else:
            parts = [(int(hp[hi_]), bd.KINDS[head.kind], head.kind,
                      lambda t, hd=head, c=c: M.row_keys(hd.kind, t, n, hd.l, c, hd.sub))]
        for pi, kind, order, keys_of in parts:
            if pi in seen:
                continue
            seen.add(pi)
            qmap, kmap = _doc_maps(order, n, n_pad, head.l, head.c, head.sub)
            _check_pattern_from_rows(lay, pi, kind, n, keys_of, qmap, kmap, w.block_q, w.block_k,
                                     f"{wname} head {hi_} ({head.kind}) pattern {pi}")
    assert len(seen) == h.num_patterns


def _random_heads(rng, n_heads):
    heads = []
    for _ in range(n_heads):
        kind = str(rng.choice(["local", "stride", "sameblock", "summary", "fixed_merged", "local_global",
                               "strided_merged"]))
        l = int(rng.integers(1, 80))
        if kind in ("summary", "fixed_merged"):
            c = int(rng.integers(1, l + 1))
            heads.append(HeadPattern(kind, l, c, int(rng.integers(0, 6))))
        elif kind == "local_global":
            heads.append(HeadPattern(kind, l, int(rng.integers(0, 40))))
        else:
            heads.append(HeadPattern(kind, l))
    return heads


@pytest.mark.parametrize("seed", range(24))
def test_random_layouts_bit_exact(seed):
    """Seeded random layouts (any n up to 700, every head kind with random l, c and
    sub-block, every tile shape the builder accepts): bit for bit against tiles
    built from the oracle's row key lists, like the workload layouts."""
    rng = np.random.default_rng(7000 + seed)
    n = int(rng.integers(1, 701))
    bq, bk = [(32, 32), (32, 64), (64, 32), (64, 64), (128, 32), (128, 64), (128, 128)][seed % 7]
    heads = _random_heads(rng, int(rng.integers(1, 5)))
    lay = Layout(n, heads, bq, bk, split_keys=int(rng.integers(32, 2048)),
                 split_rows=int(rng.integers(32, 2048)))
    h = lay.header
    hp = lay.head_pattern_index()
    part, _ = lay.head_parts()
    seen = set()
    for hi_, head in enumerate(heads):
        c = head.c or None
        if head.kind == "strided_merged":
            parts = [(int(hp[hi_]), bd.KINDS["local"], "local",
                      lambda t, l=head.l: M.row_keys(M.LOCAL, t, n, l)),
                     (int(part[hi_]), bd.SA_STRIDE_FAR, "stride",
                      lambda t, l=head.l: np.setdiff1d(M.row_keys(M.STRIDE, t, n, l),
                                                       M.row_keys(M.LOCAL, t, n, l)))]
        else:
            parts = [(int(hp[hi_]), bd.KINDS[head.kind], head.kind,
                      lambda t, hd=head, c=c: M.row_keys(hd.kind, t, n, hd.l, c, hd.sub))]
        for pi, kind, order, keys_of in parts:
            if pi in seen:
                continue
            seen.add(pi)
            qmap, kmap = _doc_maps(order, n, h.n_pad, head.l, head.c, head.sub)
            _check_pattern_from_rows(lay, pi, kind, n, keys_of, qmap, kmap, bq, bk,
                                     f"seed {seed} head {hi_} {head}")
    assert len(seen) == h.num_patterns
    # every split chunk of the schedules covers its tile's list exactly once
    for sched, ptr_name in ((lay.fwd_schedule(), "row_ptr"), (lay.bwd_schedule(), "col_ptr")):
        cover = {}
        for head, tile, e0, e1, *_ in sched.tolist():
            cover.setdefault((head, tile), []).append((e0, e1))
        for (head, tile), runs in cover.items():
            ptr = lay.pattern_arrays(int(hp[head]))[ptr_name]
            runs.sort()
            assert runs[0][0] == ptr[tile] and runs[-1][1] == ptr[tile + 1]
            assert all(a[1] == b[0] for a, b in zip(runs, runs[1:]))


def test_patterns_are_shared_between_equal_heads():
    heads = [HeadPattern("local", 8), HeadPattern("stride", 8)] * 4 + [HeadPattern("summary", 8, 2, 5)]
    lay = Layout(64, heads, 32, 32)
    assert lay.num_patterns == 3
    assert lay.head_pattern_index().tolist() == [0, 1] * 4 + [2]
    # sub is taken mod l / c: sub 5 == sub 1
    assert lay.pattern_rec(2).sub == 1 and lay.pattern_rec(2).s == 4


def test_schedules_cover_every_tile_heaviest_first():
    heads = [HeadPattern("sameblock", 64), HeadPattern("summary", 64, 16, 0)]
    lay = Layout(1000, heads, 64, 64)
    h = lay.header
    fs, bs = lay.fwd_schedule(), lay.bwd_schedule()
    fwork, bwork = [], []
    hp = lay.head_pattern_index()
    for head, qt, e0, e1, slot, pat, slot0, nch, first in fs:
        assert (pat, slot0, nch) == (hp[head], -1, 1)
        a = lay.pattern_arrays(int(lay.head_pattern_index()[head]))
        assert (e0, e1, slot) == (a["row_ptr"][qt], a["row_ptr"][qt + 1], -1)  # no split at n=1000
        assert first == (a["col"][e0] << 1) | a["fflag"][e0]
        fwork.append(e1 - e0)
    for head, kt, e0, e1, slot, pat, slot0, nch, first in bs:
        assert pat == hp[head]
        a = lay.pattern_arrays(int(hp[head]))
        assert first == ((a["row"][e0] << 1) | a["bflag"][e0] if e0 < e1 else -1)
        bwork.append(e1 - e0)
    assert all(w > 0 for w in fwork)
    assert fwork == sorted(fwork, reverse=True) and bwork == sorted(bwork, reverse=True)
    assert sorted(tuple(r[:2]) for r in fs.tolist()) == [(hh, q) for hh in range(2)
                                                        for q in range(h.nqt) if q * 64 < 1000]
    assert sorted({(int(r[0]), int(r[1])) for r in bs}) == [(hh, k) for hh in range(2)
                                                           for k in range(h.nkt) if k * 64 < 1000]


@pytest.mark.parametrize("n,bq,bk,heads", [
    (12288, 128, 64, [HeadPattern("sameblock", 128), HeadPattern("summary", 128, 32, 0)] * 4),
    (3072, 64, 64, [HeadPattern("local", 64), HeadPattern("stride", 64)] * 4),
    (100, 32, 32, [HeadPattern("local", 5)]),
])
def test_xcd_lists_cover_every_schedule_entry_once(n, bq, bk, heads):
    """Per-XCD lists: a permutation of the schedule (plus -1 padding), heaviest first per list,
    each list a contiguous run of the (head, tile) natural order."""
    lay = Layout(n, heads, bq, bk)
    for which, sched in (("fwd", lay.fwd_schedule()), ("bwd", lay.bwd_schedule())):
        xl = lay.xcd_lists(which)
        assert xl.shape[0] == bd.SA_XCDS
        items = lay.xcd_items(which)  # the named entries, in list order
        for x in range(bd.SA_XCDS):
            for j, idx in enumerate(xl[x]):
                expect = sched[idx] if idx >= 0 else np.full(bd.SA_SCHED_FIELDS, -1)
                np.testing.assert_array_equal(items[x, j], expect)
        flat = xl[xl >= 0]
        assert sorted(flat.tolist()) == list(range(len(sched)))
        keys = [tuple(int(x) for x in sched[i][:3]) for i in range(len(sched))]
        natural = sorted(range(len(sched)), key=lambda i: keys[i])
        rank = {i: r for r, i in enumerate(natural)}
        prev_max = -1
        for row in xl:
            ids = [int(i) for i in row if i >= 0]
            assert ids == sorted(ids)  # heaviest first = ascending schedule index
            if ids:
                rs = sorted(rank[i] for i in ids)
                assert rs == list(range(rs[0], rs[0] + len(rs)))  # contiguous run
                assert rs[0] > prev_max
                prev_max = rs[-1]


def _segment_heads(lay) -> set:
    items = lay.xcd_items("seg").reshape(-1, bd.SA_SCHED_FIELDS)
    return {int(r[0]) for r in items if r[0] >= 0}


@pytest.mark.parametrize("n,bq,bk,heads", [
    (12288, 64, 64, [HeadPattern("sameblock", 128), HeadPattern("summary", 128, 32, 0),
                     HeadPattern("summary", 128, 32, 3)]),
    (5000, 32, 32, [HeadPattern("summary", 64, 4, 1), HeadPattern("local", 3000)]),
    (3072, 64, 64, [HeadPattern("local", 64), HeadPattern("stride", 64)]),
])
def test_dkdv_chunks_partition_every_csc_column(n, bq, bk, heads):
    """Each key tile's CSC list is covered exactly once, in chunks of at most the split cap."""
    lay = Layout(n, heads, bq, bk)
    h = lay.header
    assert h.split_rows == 1536
    cap = max(1, h.split_rows // bq)
    bs, rs = lay.bwd_schedule(), lay.reduce_schedule()
    slots = sorted(int(r[4]) for r in bs if r[4] >= 0)
    assert slots == list(range(h.num_slots))
    red = {(int(r[0]), int(r[1])): (int(r[2]), int(r[3])) for r in rs}
    seg = _segment_heads(lay)
    for head in range(len(heads)):
        a = lay.pattern_arrays(int(lay.head_pattern_index()[head]))
        if head in seg:  # the segment pass runs this head's backward
            assert not any(r[0] == head for r in bs)
            continue
        for kt in range(h.nkt):
            if kt * bk >= n:
                continue
            rows = sorted((int(r[2]), int(r[3]), int(r[4])) for r in bs if r[0] == head and r[1] == kt)
            c0, c1 = a["col_ptr"][kt], a["col_ptr"][kt + 1]
            assert rows[0][0] == c0 and rows[-1][1] == c1
            assert all(x[1] == y[0] for x, y in zip(rows, rows[1:]))
            assert all(e1 - e0 <= cap for e0, e1, _ in rows)
            if c1 - c0 <= cap:
                assert rows == [(c0, c1, -1)] and (head, kt) not in red
            else:
                s0, nch = red[(head, kt)]
                assert [r[2] for r in rows] == list(range(s0, s0 + nch))
                grp = {(int(r[5]), int(r[6]), int(r[7])) for r in bs if r[0] == head and r[1] == kt}
                assert grp == {(int(lay.head_pattern_index()[head]), s0, nch)}
    if n == 12288:
        assert h.red_sched_len > 0 and h.num_slots > h.red_sched_len


@pytest.mark.parametrize("n,bq,bk,heads", [
    (12288, 128, 64, [HeadPattern("sameblock", 128), HeadPattern("summary", 128, 32, 0),
                      HeadPattern("summary", 128, 32, 3)]),
    (12288, 64, 64, [HeadPattern("local", 128), HeadPattern("stride", 128)]),
    (5000, 32, 32, [HeadPattern("summary", 64, 4, 1), HeadPattern("local", 3000)]),
    (3072, 64, 64, [HeadPattern("local", 64), HeadPattern("stride", 64)]),
])
def test_query_chunks_partition_every_csr_row(n, bq, bk, heads):
    """Each query tile's CSR list is covered exactly once by forward / dQ items, in
    contiguous chunks of at most split_keys (default 3072) keys; split tiles own
    consecutive slots that the merge schedule lists."""
    lay = Layout(n, heads, bq, bk)
    h = lay.header
    assert h.split_keys == 3072
    qcap = max(1, h.split_keys // bk)
    fs, cs = lay.fwd_schedule(), lay.combine_schedule()
    slots = sorted(int(r[4]) for r in fs if r[4] >= 0)
    assert slots == list(range(h.num_qslots))
    comb = {(int(r[0]), int(r[1])): (int(r[2]), int(r[3])) for r in cs}
    assert len(comb) == len(cs) == h.comb_sched_len
    for head in range(len(heads)):
        a = lay.pattern_arrays(int(lay.head_pattern_index()[head]))
        for qt in range(h.nqt):
            r0, r1 = int(a["row_ptr"][qt]), int(a["row_ptr"][qt + 1])
            rows = sorted((int(r[2]), int(r[3]), int(r[4])) for r in fs if r[0] == head and r[1] == qt)
            if r1 == r0:
                assert rows == [] and (head, qt) not in comb
                continue
            assert rows[0][0] == r0 and rows[-1][1] == r1
            assert all(x[1] == y[0] for x, y in zip(rows, rows[1:]))
            assert all(0 < e1 - e0 <= qcap for e0, e1, _ in rows)
            if r1 - r0 <= qcap:
                assert rows == [(r0, r1, -1)] and (head, qt) not in comb
            else:
                s0, nch = comb[(head, qt)]
                assert nch == -(-(r1 - r0) // qcap)
                assert [r[2] for r in rows] == list(range(s0, s0 + nch))
                grp = {(int(r[5]), int(r[6]), int(r[7])) for r in fs if r[0] == head and r[1] == qt}
                assert grp == {(int(lay.head_pattern_index()[head]), s0, nch)}
    if n == 12288:
        # summary heads read up to 3072 keys per row (the default cap), strided heads
        # stay within one class: nothing is split
        assert h.comb_sched_len == 0


@pytest.mark.parametrize("split_keys,split_rows", [(256, 320), (96, 64), (1 << 30, 1 << 30)])
def test_chunk_caps_are_layout_parameters(split_keys, split_rows):
    """Caller-chosen caps: every chunk within them (at least one tile), and caps at
    least n split nothing."""
    heads = [HeadPattern("summary", 64, 16, 0), HeadPattern("local", 700), HeadPattern("stride", 3)]
    n, bq, bk = 900, 64, 32
    lay = Layout(n, heads, bq, bk, split_keys=split_keys, split_rows=split_rows)
    h = lay.header
    assert (h.split_keys, h.split_rows) == (split_keys, split_rows)
    qcap, cap = max(1, split_keys // bk), max(1, split_rows // bq)
    fs, bs = lay.fwd_schedule(), lay.bwd_schedule()
    assert all(0 < r[3] - r[2] <= qcap for r in fs)
    assert all(0 <= r[3] - r[2] <= cap for r in bs)  # unread key tiles: zero dK, dV
    if split_keys >= n:
        assert h.comb_sched_len == h.num_qslots == 0 and h.red_sched_len == h.num_slots == 0
    else:
        assert h.comb_sched_len > 0 and h.red_sched_len > 0
    ref = Layout(n, heads, bq, bk)
    for i in range(ref.num_patterns):  # the caps change schedules only
        for key, arr in ref.pattern_arrays(i).items():
            np.testing.assert_array_equal(lay.pattern_arrays(i)[key], arr)


@pytest.mark.parametrize("n,bq,bk,heads", [
    (12288, 32, 32, [HeadPattern("local", 128), HeadPattern("stride", 128)] * 2),
    (3072, 64, 64, [HeadPattern("local", 64), HeadPattern("stride", 64)]),
    (1000, 64, 32, [HeadPattern("stride", 7), HeadPattern("stride", 9), HeadPattern("summary", 8, 2, 1)]),
    (100, 32, 32, [HeadPattern("stride", 1000), HeadPattern("stride", 1)]),
    (4097, 128, 128, [HeadPattern("stride", 32), HeadPattern("stride", 31), HeadPattern("strided_merged", 64)]),
])
def test_segments_are_the_stride_classes(n, bq, bk, heads):
    """Segment pass: each qualifying stride head is listed as its residue classes -- runs of
    layout positions whose rows read only keys of the same run and whose keys only rows
    of it read (checked against the oracle's sets), each at most SA_SEGMENT_ROWS rows --
    and leaves the dQ list and the backward schedule; every other head keeps its items."""
    lay = Layout(n, heads, bq, bk)
    h = lay.header
    items = lay.xcd_items("seg").reshape(-1, bd.SA_SCHED_FIELDS)
    items = items[items[:, 0] >= 0]
    hp = lay.head_pattern_index()
    expect = {hh for hh, x in enumerate(heads) if x.kind == "stride" and -(-n // x.l) <= bd.SA_SEGMENT_ROWS}
    assert _segment_heads(lay) == expect
    assert h.seg_len == len(items)
    longest = 0
    for hh in sorted(expect):
        l = heads[hh].l
        mine = sorted((int(r[1]), int(r[3])) for r in items if r[0] == hh)
        assert all(tuple(r[[4, 6, 7, 8]]) == (l, -1, 1, -1) and r[5] == hp[hh]
                   for r in items if r[0] == hh)
        assert sorted(int(r[2]) for r in items if r[0] == hh) == list(range(min(l, n)))
        qmap = lay.pattern_arrays(int(hp[hh]))["qmap"]
        pos = 0
        res = {int(r[1]): int(r[2]) for r in items if r[0] == hh}
        for r, (start, rows) in enumerate(mine):
            assert res[start] == r
            assert start == pos and rows == len(range(r, n, l)) and 1 <= rows <= bd.SA_SEGMENT_ROWS
            toks = qmap[start:start + rows]
            np.testing.assert_array_equal(toks, np.arange(r, n, l))
            ts = set(toks.tolist())
            for i in toks[:: max(1, rows // 7)]:
                assert set(M.row_keys(M.STRIDE, int(i), n, l).tolist()) <= ts
                assert set(M.rows_seeing(M.STRIDE, int(i), n, l).tolist()) <= ts
            pos += rows
            longest = max(longest, rows)
        assert pos == n and len(mine) == min(l, n)
    assert h.seg_tiles == -(-longest // 32)
    fwd = lay.xcd_items("fwd").reshape(-1, bd.SA_SCHED_FIELDS)
    dq = lay.xcd_items("dq").reshape(-1, bd.SA_SCHED_FIELDS)
    want = sorted(tuple(r) for r in fwd.tolist() if r[0] >= 0 and r[0] not in expect)
    assert sorted(tuple(r) for r in dq.tolist() if r[0] >= 0) == want
    bs = lay.bwd_schedule()
    assert {int(r[0]) for r in bs} == set(range(len(heads))) - expect
    # Without the pass: no segments, the dQ list is the forward's, every head in the schedule.
    off = Layout(n, heads, bq, bk, segment_pass=False)
    assert off.header.seg_len == off.header.seg_tiles == off.header.seg_xl_len == 0
    f2, d2 = (off.xcd_items(x).reshape(-1, bd.SA_SCHED_FIELDS) for x in ("fwd", "dq"))
    assert sorted(map(tuple, f2.tolist())) == sorted(map(tuple, d2.tolist()))
    assert {int(r[0]) for r in off.bwd_schedule()} == set(range(len(heads)))


def test_segment_pass_skips_heads_with_split_tiles():
    """A stride head whose tiles are split (caps below its lists) keeps the tile passes."""
    heads = [HeadPattern("stride", 8), HeadPattern("local", 8)]
    assert _segment_heads(Layout(1000, heads, 32, 32)) == {0}
    assert _segment_heads(Layout(1000, heads, 32, 32, split_keys=32)) == set()
    assert _segment_heads(Layout(1000, heads, 32, 32, split_rows=32)) == set()


def test_padding_overhead_closed_form_12288():
    """Computed-tile area per allowed pair for the 12,288-token heads with 64x64 tiles."""
    lay = Layout(12288, [HeadPattern("local", 128), HeadPattern("stride", 128)], 64, 64)
    a0, a1 = lay.pattern_arrays(0), lay.pattern_arrays(1)
    assert lay.pattern_rec(0).pairs == 1576896 and lay.pattern_rec(1).pairs == 595968
    # local band l=128: q-tile i >= 2 touches k-tiles i-2, i-1, i (the first only partly)
    assert len(a0["col"]) == 1 + 2 + 3 * (192 - 2)
    # stride head: 128 classes of 96 tokens; every tile pair touched stays inside a class
    assert (lay.tiles_per_batch() * 64 * 64) / lay.pairs_per_batch() < 2.0


# ----------------------------------------------------------------------------
# errors, flags, ABI surface
# ----------------------------------------------------------------------------

def _raw_layout(n, heads, bq=64, bk=64, flags=1):
    lib = bd.load_library()
    arr = (bd.CHeadPattern * max(1, len(heads)))(*heads)
    desc = bd.CLayoutDesc(n, bq, bk, len(heads), arr, flags)
    size = ctypes.c_size_t(0)
    return lib.sparse_attn_layout(ctypes.byref(desc), None, ctypes.byref(size)), size.value


@pytest.mark.parametrize("n,heads,bq,bk,flags,expect", [
    (0, [(0, 4, 0, 0)], 64, 64, 1, bd.SA_EINVAL),
    (-5, [(0, 4, 0, 0)], 64, 64, 1, bd.SA_EINVAL),
    (64, [(0, 0, 0, 0)], 64, 64, 1, bd.SA_EINVAL),          # l = 0
    (64, [(3, 8, 0, 0)], 64, 64, 1, bd.SA_EINVAL),          # c = 0
    (64, [(3, 8, 9, 0)], 64, 64, 1, bd.SA_EINVAL),          # c > l
    (64, [(3, 8, 2, -1)], 64, 64, 1, bd.SA_EINVAL),         # sub < 0
    (64, [(7, 8, 0, 0)], 64, 64, 1, bd.SA_EINVAL),          # unknown kind
    (64, [(0, 8, 0, 0)], 48, 64, 1, bd.SA_EUNSUPPORTED),    # tile not 32/64/128
    (64, [(0, 8, 0, 0)], 64, 256, 1, bd.SA_EUNSUPPORTED),
    (64, [(0, 8, 0, 0)], 64, 64, 6, bd.SA_EINVAL),          # unknown flag
    (64, [(3, 8, 2, 0)], 64, 64, 0, bd.SA_EINVAL),          # empty rows without self-if-empty
    (64, [], 64, 64, 1, bd.SA_EINVAL),                      # no heads
    ((1 << 26) + 1, [(0, 8, 0, 0)], 64, 64, 1, bd.SA_EINVAL),
])
def test_layout_rejects_bad_descriptors(n, heads, bq, bk, flags, expect):
    rc, _ = _raw_layout(n, [bd.CHeadPattern(*h) for h in heads], bq, bk, flags)
    assert rc == expect


def test_layout_rejects_negative_chunk_caps():
    lib = bd.load_library()
    arr = (bd.CHeadPattern * 1)(bd.CHeadPattern(0, 8, 0, 0))
    size = ctypes.c_size_t(0)
    for ks, rs in ((-1, 0), (0, -64)):
        desc = bd.CLayoutDesc(64, 64, 64, 1, arr, 1, ks, rs)
        assert lib.sparse_attn_layout(ctypes.byref(desc), None, ctypes.byref(size)) == bd.SA_EINVAL


def test_layout_without_self_if_empty_when_no_row_is_empty():
    rc, size = _raw_layout(64, [bd.CHeadPattern(3, 8, 8, 0), bd.CHeadPattern(1, 8, 0, 0)], flags=0)
    assert rc == bd.SA_OK and size > 0


def test_layout_buffer_too_small_and_check():
    lib = bd.load_library()
    heads = (bd.CHeadPattern * 1)(bd.CHeadPattern(0, 8, 0, 0))
    desc = bd.CLayoutDesc(128, 64, 64, 1, heads, 1)
    size = ctypes.c_size_t(0)
    assert lib.sparse_attn_layout(ctypes.byref(desc), None, ctypes.byref(size)) == 0
    need = size.value
    small = np.zeros(need - 64, dtype=np.uint8)
    size2 = ctypes.c_size_t(small.size)
    assert lib.sparse_attn_layout(ctypes.byref(desc), small.ctypes.data_as(ctypes.c_void_p),
                                  ctypes.byref(size2)) == bd.SA_ESIZE
    assert size2.value == need
    blob = np.zeros(need, dtype=np.uint8)
    size3 = ctypes.c_size_t(need)
    assert lib.sparse_attn_layout(ctypes.byref(desc), blob.ctypes.data_as(ctypes.c_void_p),
                                  ctypes.byref(size3)) == 0
    assert lib.sparse_attn_layout_check(blob.ctypes.data, need) == 0
    assert lib.sparse_attn_layout_check(blob.ctypes.data, need - 1) == bd.SA_ESIZE
    bad = blob.copy()
    bad[0] ^= 0xFF
    assert lib.sparse_attn_layout_check(bad.ctypes.data, need) == bd.SA_EINVAL
    assert lib.sparse_attn_layout_check(None, need) == bd.SA_EINVAL


def test_layout_check_rejects_bad_segment_fields():
    """The segment pass's header fields are checked like the others: sub-tile count in
    1..4 exactly when there are segments, lists inside the blob."""
    lib = bd.load_library()
    lay = Layout(1000, [HeadPattern("stride", 8), HeadPattern("local", 8)], 64, 64)
    h = lay.header
    assert h.seg_len == 8 and h.seg_tiles == 4
    assert lib.sparse_attn_layout_check(lay.blob.ctypes.data, lay.blob.size) == 0

    def patched(**fields):
        hdr = bd.CBlobHeader.from_buffer_copy(lay.blob[: ctypes.sizeof(bd.CBlobHeader)].tobytes())
        for k, v in fields.items():
            setattr(hdr, k, v)
        blob = lay.blob.copy()
        blob[: ctypes.sizeof(hdr)] = np.frombuffer(bytes(hdr), dtype=np.uint8)
        return lib.sparse_attn_layout_check(blob.ctypes.data, blob.size)

    assert patched() == 0
    assert patched(seg_tiles=5) == bd.SA_EINVAL
    assert patched(seg_tiles=0) == bd.SA_EINVAL
    assert patched(seg_len=-1) == bd.SA_EINVAL
    assert patched(seg_xitem_off=int(lay.blob.size)) == bd.SA_EINVAL
    assert patched(dq_xl_len=1 << 20) == bd.SA_EINVAL
    off = Layout(1000, [HeadPattern("stride", 8)], 64, 64, segment_pass=False)
    assert off.header.seg_len == 0 and off.header.seg_tiles == 0


def test_library_exports_every_declared_symbol():
    lib = bd.load_library()
    with open(os.path.join(ROOT, "include", "sparse_attn.h")) as f:
        text = f.read()
    import re
    declared = set(re.findall(r"\b(sparse_attn_[a-z_]+)\s*\(", text))
    assert declared == set(bd.EXPORTED)
    for name in declared:
        assert hasattr(lib, name)
    assert lib.sparse_attn_strerror(0) == b"success"
    assert lib.sparse_attn_strerror(-2) == b"unsupported configuration"
    assert lib.sparse_attn_strerror(99) == b"unknown status"


def test_probe_library_exports_its_header():
    """The calibration library exports what include/sa_probes.h declares, and the
    ctypes result struct matches the C one (loaded without a GPU: nothing runs)."""
    import re
    from factorized_block_sparse_amd import calibration as cal
    text = open(os.path.join(ROOT, "include", "sa_probes.h")).read()
    declared = set(re.findall(r"\b(sa_probe_[a-z_]+)\s*\(", text))
    assert declared == {"sa_probe_run"}
    lib = ctypes.CDLL(os.path.join(os.path.dirname(bd.library_path()), cal.LIB_NAME))
    assert all(hasattr(lib, nm) for nm in declared)
    fields = re.findall(r"double\s+(\w+);", text)
    assert tuple(fields) == cal.FIELDS
    assert ctypes.sizeof(cal.ProbeResults) == 8 * len(fields)


def test_ctypes_structs_match_the_c_header():
    """Sizes and offsets of the ABI structs, from a C compiler reading the header."""
    src = r"""
    #include <stdio.h>
    #include <stddef.h>
    #include "sparse_attn.h"
    int main(void) {
      printf("%zu %zu %zu %zu\n", sizeof(sa_head_pattern), sizeof(sa_layout_desc),
             sizeof(sa_pattern_rec), sizeof(sa_blob_header));
      printf("%zu %zu %zu\n", offsetof(sa_layout_desc, heads), offsetof(sa_layout_desc, flags),
             offsetof(sa_blob_header, tiles_all_heads));
      printf("%zu %zu\n", offsetof(sa_pattern_rec, bflag_off), offsetof(sa_blob_header, bwd_sched_len));
      return 0;
    }
    """
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "s.c")
        exe = os.path.join(d, "s")
        with open(c, "w") as f:
            f.write(src)
        subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()
    got = list(map(int, out))
    assert got == [ctypes.sizeof(bd.CHeadPattern), ctypes.sizeof(bd.CLayoutDesc),
                   ctypes.sizeof(bd.CPatternRec), ctypes.sizeof(bd.CBlobHeader),
                   bd.CLayoutDesc.heads.offset, bd.CLayoutDesc.flags.offset,
                   bd.CBlobHeader.tiles_all_heads.offset, bd.CPatternRec.bflag_off.offset,
                   bd.CBlobHeader.bwd_sched_len.offset]


def test_fwd_bwd_argument_errors_before_any_launch():
    """Validation rejects bad arguments before touching the device (runs without a GPU)."""
    lib = bd.load_library()
    lay = Layout(128, [HeadPattern("local", 8), HeadPattern("stride", 8)], 64, 64)
    hb = lay.blob.ctypes.data
    fake = 1 << 20  # aligned non-null device-looking address; never dereferenced on these paths
    f = lambda **kw: lib.sparse_attn_fwd(kw.get("blob", hb), kw.get("dev", fake), kw.get("B", 1),
                                         kw.get("H", 2), kw.get("d", 64), kw.get("dt", 0), fake,
                                         fake, fake, kw.get("o", fake), fake, kw.get("ws", fake),
                                         kw.get("wsb", 1 << 30), kw.get("scale", 0.0), None)
    assert f(blob=None) == bd.SA_EINVAL
    assert f(H=3) == bd.SA_EINVAL
    assert f(B=-1) == bd.SA_EINVAL
    assert f(d=128) == bd.SA_EUNSUPPORTED
    assert f(dt=7) == bd.SA_EINVAL
    assert f(o=None) == bd.SA_EINVAL
    assert f(o=fake + 2) == bd.SA_EINVAL
    assert f(dev=fake + 8) == bd.SA_EINVAL
    assert f(scale=float("nan")) == bd.SA_EINVAL
    assert f(B=0) == bd.SA_OK  # empty batch: nothing to do
    size = ctypes.c_size_t(1)
    assert lib.sparse_attn_fwd_workspace(hb, 2, 2, 64, 0, ctypes.byref(size)) == 0
    assert size.value == 0  # no query tile is split at n=128
    assert lib.sparse_attn_fwd_workspace(hb, 2, 2, 128, 0, ctypes.byref(size)) == bd.SA_EUNSUPPORTED
    big = Layout(12288, [HeadPattern("sameblock", 128), HeadPattern("summary", 128, 32, 0)], 64, 64,
                 split_keys=2048)
    assert big.header.num_qslots > 0
    assert lib.sparse_attn_fwd_workspace(big.blob.ctypes.data, 3, 2, 64, 0, ctypes.byref(size)) == 0
    rows = 3 * big.header.num_qslots * 64
    rnd = lambda x: -(-x // 256) * 256
    # partial O, partial max, partial sum
    assert size.value == rnd(rows * 64 * 4) + 2 * rnd(rows * 4)
    hbig = big.blob.ctypes.data
    assert lib.sparse_attn_fwd(hbig, fake, 3, 2, 64, 0, fake, fake, fake, fake, fake, fake,
                               size.value - 1, 0.0, None) == bd.SA_ESIZE
    size = ctypes.c_size_t(0)
    assert lib.sparse_attn_bwd_workspace(hb, 2, 2, 64, 0, ctypes.byref(size)) == 0
    assert lay.header.num_slots == 0
    assert size.value == -(-2 * 2 * 128 * 4 // 256) * 256  # D only: no split key tiles
    assert lib.sparse_attn_bwd_workspace(hb, 2, 2, 64, 1, ctypes.byref(size)) == bd.SA_EUNSUPPORTED
    g = lambda **kw: lib.sparse_attn_bwd(hb, fake, kw.get("B", 1), 2, 64, kw.get("dt", 0), fake, fake,
                                         fake, fake, fake, fake, fake, fake, fake, fake,
                                         kw.get("ws", 1 << 30), 0.0, None)
    assert g(ws=16) == bd.SA_ESIZE
    assert g(dt=1) == bd.SA_EUNSUPPORTED
    assert g(B=0) == bd.SA_OK
    gp = lambda ph: lib.sparse_attn_bwd_phases(hb, fake, 1, 2, 64, 0, fake, fake, fake, fake, fake, fake,
                                               fake, fake, fake, fake, 1 << 30, 0.0, ph, None)
    assert gp(0) == bd.SA_EINVAL and gp(16) == bd.SA_EINVAL
    fp = lambda ph: lib.sparse_attn_fwd_phases(hb, fake, 1, 2, 64, 0, fake, fake, fake, fake, fake,
                                               fake, 1 << 30, 0.0, ph, None)
    assert fp(0) == bd.SA_EINVAL and fp(4) == bd.SA_EINVAL
    # split key and query tiles: D, dK/dV partials, dQ partials
    assert lib.sparse_attn_bwd_workspace(hbig, 3, 2, 64, 0, ctypes.byref(size)) == 0
    hdr = big.header
    assert hdr.red_sched_len > 0 and hdr.comb_sched_len > 0
    assert size.value == (rnd(3 * 2 * 12288 * 4) + rnd(3 * hdr.num_slots * 2 * 64 * 64 * 4)
                          + rnd(3 * hdr.num_qslots * 64 * 64 * 4))


def test_layout_refuses_tile_counts_past_int32():
    """CSR / CSC entries are int32: a pattern whose active tiles could pass INT32_MAX
    (a local band as long as n = 2^21 on 32 x 32 tiles: 65,536 * 65,537 / 2 tiles) is
    refused by the size-only pass before anything is built."""
    lib = bd.load_library()
    n = 1 << 21
    heads = (bd.CHeadPattern * 1)(bd.CHeadPattern(bd.KINDS["local"], n, 0, 0))
    desc = bd.CLayoutDesc(n, 32, 32, 1, heads, bd.SA_SELF_IF_EMPTY, 0, 0)
    size = ctypes.c_size_t(0)
    assert lib.sparse_attn_layout(ctypes.byref(desc), None, ctypes.byref(size)) == bd.SA_EUNSUPPORTED
    # 64 x 64 tiles: a quarter of the tiles, within range (size query only)
    desc = bd.CLayoutDesc(1 << 16, 64, 64, 1, heads, bd.SA_SELF_IF_EMPTY, 0, 0)
    assert lib.sparse_attn_layout(ctypes.byref(desc), None, ctypes.byref(size)) == bd.SA_OK
    assert lib.sparse_attn_strerror(bd.SA_ENOMEM) == b"out of host memory"


def test_static_backward_checks_before_any_launch():
    """sparse_attn_bwd_static validates like sparse_attn_bwd and refuses sizes past its
    static array with SA_ESIZE before touching the device (runs without a GPU)."""
    lib = bd.load_library()
    lay = Layout(4096, [HeadPattern("local", 8), HeadPattern("stride", 8)], 64, 64)
    hb = lay.blob.ctypes.data
    fake = 1 << 20
    s = lambda B, H=2, d=64, dt=0, blob=hb: lib.sparse_attn_bwd_static(
        blob, fake, B, H, d, dt, fake, fake, fake, fake, fake, fake, fake, fake, fake, 0.0, None)
    big_b = bd.SA_STATIC_SCRATCH_BYTES // (2 * 4096 * 4) + 1  # D alone overflows the array
    assert s(big_b) == bd.SA_ESIZE
    assert s(1, blob=None) == bd.SA_EINVAL
    assert s(1, H=3) == bd.SA_EINVAL
    assert s(1, d=128) == bd.SA_EUNSUPPORTED
    assert s(1, dt=1) == bd.SA_EUNSUPPORTED
    assert s(0) == bd.SA_OK  # empty batch: nothing to do, no device lookup


def test_profile_summaries_parse_and_track_the_sources(tmp_path):
    """The committed counter summary lists the bench kernels; a summary whose source hash
    differs from the current kernels is ignored (its traffic would describe other code)."""
    from factorized_block_sparse_amd import profiling
    path = os.path.join(ROOT, "profiles", "n12288_fixed_strided_hbm_traffic.txt")
    recorded, table = profiling.read_traffic(path)
    assert recorded is not None and len(recorded) == 64
    w = W.WORKLOADS["fixed_n12288"]
    assert any(f"bwd_dkdv_kernel<{w.block_q}, {w.block_k}" in k for k in table)
    assert all(f > 0 and w > 0 for f, w in table.values())
    stale = tmp_path / "t.txt"
    stale.write_text(open(path).read().replace(recorded, "0" * 64))
    rec2, _ = profiling.read_traffic(str(stale))
    assert rec2 != profiling.source_hash()


def test_source_hash_follows_code_not_comments():
    """Counter summaries stay valid across comment edits and go stale on code edits."""
    from factorized_block_sparse_amd import profiling
    a = "int f(int x) {  // twice\n  return 2 * x; /* doubled */ }\n"
    b = "/* a new remark */\nint f(int x) {\n  return 2 * x;  // the double\n}"
    assert profiling.code_text(a) == profiling.code_text(b) == "int f(int x) { return 2 * x; }"
    assert profiling.code_text(a) != profiling.code_text(a.replace("2 * x", "3 * x"))
    for rel in profiling.SOURCES:  # no comment markers inside string literals
        text = open(os.path.join(ROOT, rel), encoding="utf-8").read()
        for line in text.splitlines():
            code = line.split("//")[0]
            assert code.count('"') % 2 == 0 or "//" not in line, (rel, line)


@pytest.mark.parametrize("n,bq,bk,l", [(300, 64, 32, 7), (1024, 32, 32, 32), (700, 128, 64, 24),
                                       (97, 32, 64, 10), (40, 64, 64, 1), (130, 64, 64, 500)])
def test_strided_merged_parts_are_disjoint_layouts_of_the_union(n, bq, bk, l):
    """A merged strided head runs as its local band (a local pattern) plus the
    stride members at distance >= 2l (residue-class order): disjoint, their
    union is the oracle's merged set, each part bit-exact like any pattern."""
    heads = [HeadPattern("strided_merged", l), HeadPattern("local", l), HeadPattern("strided_merged", l)]
    lay = Layout(n, heads, bq, bk)
    h = lay.header
    t = max(bq, bk)
    n_pad = -(-n // t) * t
    hp = lay.head_pattern_index()
    part, merged = lay.head_parts()
    assert part.tolist()[1] == -1 and merged.tolist() == [0, -1, 1] and h.num_merged == 2
    assert hp[0] == hp[1] == hp[2] and part[0] == part[2]  # shared band and part patterns
    band = M.head_mask(n, M.LOCAL, l)
    far = M.head_mask(n, M.STRIDE, l) & ~band
    np.testing.assert_array_equal(band | far, M.head_mask(n, M.STRIDED_MERGED, l))
    rec = lay.pattern_rec(int(part[0]))
    assert (rec.kind, rec.l, rec.pre_off) == (bd.SA_STRIDE_FAR, l, 0)
    arr = lay.pattern_arrays(int(part[0]))
    qmap, kmap = _doc_maps("stride", n, n_pad, l)
    np.testing.assert_array_equal(arr["qmap"], qmap)
    np.testing.assert_array_equal(arr["kmap"], kmap)
    mp = np.zeros((n_pad, n_pad), dtype=bool)
    mp[:n, :n] = far[np.ix_(qmap[:n], kmap[:n])]
    cols = np.arange(n_pad)
    interval = (cols[None, :] >= arr["lo"][:, None]) & (cols[None, :] <= arr["hi"][:, None])
    np.testing.assert_array_equal(interval, mp)
    np.testing.assert_array_equal(arr["count"], far.sum(1))
    assert rec.pairs == far.sum()
    ref = _ref_tiles(mp, bq, bk)
    for name, r in zip(("row_ptr", "col", "fflag", "col_ptr", "row", "bflag"), ref):
        np.testing.assert_array_equal(arr[name], r, err_msg=name)
    assert lay.pairs_per_batch() == 2 * int(band.sum() + far.sum()) + int(band.sum())
    # Second-part schedules: every tile holding a token, unsplit, in the part's lists.
    fp, bp = lay.part_schedules()
    nq = [q for q in range(h.nqt) if q * bq < n]
    nk = [k for k in range(h.nkt) if k * bk < n]
    assert sorted((int(r[0]), int(r[1])) for r in fp) == [(hh, q) for hh in (0, 2) for q in nq]
    assert sorted((int(r[0]), int(r[1])) for r in bp) == [(hh, k) for hh in (0, 2) for k in nk]
    for sched, ptr in ((fp, arr["row_ptr"]), (bp, arr["col_ptr"])):
        for head, tile, e0, e1, slot, pf, slot0, nch, first in sched.tolist():
            assert (e0, e1, slot, slot0, nch) == (ptr[tile], ptr[tile + 1], -1, -1, 1)
            assert pf == int(part[0]) | ((merged[head] + 1) << 16)
    for which, sched in (("fwdp", fp), ("bwdp", bp)):
        items = lay.xcd_items(which).reshape(-1, bd.SA_SCHED_FIELDS)
        got = sorted(tuple(r) for r in items.tolist() if r[0] >= 0)
        assert got == sorted(tuple(r) for r in sched.tolist())
    # Main entries of two-part heads carry their index, and the first chunk of
    # each tile the start-from-part flag.
    for sched in (lay.fwd_schedule(), lay.bwd_schedule()):
        for head, tile, e0, e1, slot, pf, slot0, nch, first in sched.tolist():
            assert pf & 0xffff == hp[head]
            if merged[head] < 0:
                assert pf == hp[head]
            else:
                assert (pf >> 16) & 0x3fff == merged[head] + 1
                assert bool(pf & bd.PART_INIT) == (slot == slot0)


def test_two_part_head_workspaces_and_dtype():
    """Merged strided heads add per-token float32 state to both workspaces, and
    are bf16 only (checked before any launch, no GPU needed)."""
    lib = bd.load_library()
    n = 500
    lay = Layout(n, [HeadPattern("strided_merged", 16), HeadPattern("local", 16),
                     HeadPattern("strided_merged", 9)], 64, 64)
    h = lay.header
    assert h.num_merged == 2 and h.num_qslots == 0 and h.num_slots == 0
    rnd = lambda x: -(-x // 256) * 256
    size = ctypes.c_size_t(0)
    assert lib.sparse_attn_fwd_workspace(lay.blob.ctypes.data, 3, 3, 64, 0, ctypes.byref(size)) == 0
    assert size.value == rnd(3 * 2 * n * 64 * 4) + 2 * rnd(3 * 2 * n * 4)
    assert lib.sparse_attn_bwd_workspace(lay.blob.ctypes.data, 3, 3, 64, 0, ctypes.byref(size)) == 0
    assert size.value == rnd(3 * 3 * n * 4) + 3 * rnd(3 * 2 * n * 64 * 4)
    fake = 1 << 20
    assert lib.sparse_attn_fwd(lay.blob.ctypes.data, fake, 1, 3, 64, 1, fake, fake, fake, fake, fake,
                               fake, 1 << 30, 0.0, None) == bd.SA_EUNSUPPORTED


def test_key_tiles_of_128_need_query_tiles_of_128():
    """128-key tiles run only with 128-row query tiles (bf16); other shapes with
    128-key tiles are rejected before any launch (no GPU needed)."""
    lib = bd.load_library()
    fake = 1 << 20
    heads = [HeadPattern("local", 16), HeadPattern("stride", 16)]
    for bq, bk, want in ((64, 128, bd.SA_EUNSUPPORTED), (32, 128, bd.SA_EUNSUPPORTED)):
        lay = Layout(300, heads, bq, bk)
        hb = lay.blob.ctypes.data
        assert lib.sparse_attn_fwd(hb, fake, 1, 2, 64, 0, fake, fake, fake, fake, fake,
                                   fake, 1 << 30, 0.0, None) == want
        assert lib.sparse_attn_bwd(hb, fake, 1, 2, 64, 0, fake, fake, fake, fake, fake, fake,
                                   fake, fake, fake, fake, 1 << 30, 0.0, None) == want
    lay = Layout(300, heads, 128, 128)
    assert lib.sparse_attn_fwd(lay.blob.ctypes.data, fake, 1, 2, 64, 1, fake, fake, fake, fake, fake,
                               fake, 1 << 30, 0.0, None) == bd.SA_EUNSUPPORTED  # float32: 32-key tiles only
