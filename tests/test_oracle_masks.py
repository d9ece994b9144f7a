"""Pins of the oracle's visibility sets against what the pages fix.

Each test cites the passage it checks.  None retypes the oracle's predicate:
the expected values are printed examples, closed-form counts derived by hand
from the set definitions, brute-force graph reachability, or symmetric
relations to counts the pages print.
"""

import os

import numpy as np
import pytest

from oracle import masks as M

KINDS_SMALL = [
    (M.LOCAL, dict(l=1)), (M.LOCAL, dict(l=3)), (M.LOCAL, dict(l=8)), (M.LOCAL, dict(l=40)),
    (M.STRIDE, dict(l=1)), (M.STRIDE, dict(l=3)), (M.STRIDE, dict(l=8)), (M.STRIDE, dict(l=40)),
    (M.SAMEBLOCK, dict(l=1)), (M.SAMEBLOCK, dict(l=5)), (M.SAMEBLOCK, dict(l=8)),
    (M.SUMMARY, dict(l=8, c=2, sub=0)), (M.SUMMARY, dict(l=8, c=2, sub=1)),
    (M.SUMMARY, dict(l=8, c=2, sub=3)), (M.SUMMARY, dict(l=8, c=3, sub=0)),
    (M.SUMMARY, dict(l=8, c=8, sub=0)), (M.SUMMARY, dict(l=6, c=1, sub=2)),
    (M.FIXED_MERGED, dict(l=8, c=2, sub=0)), (M.FIXED_MERGED, dict(l=8, c=2, sub=3)),
    (M.FIXED_MERGED, dict(l=6, c=1, sub=2)), (M.FIXED_MERGED, dict(l=5, c=5, sub=0)),
    (M.LOCAL_GLOBAL, dict(l=2, c=1)), (M.LOCAL_GLOBAL, dict(l=3, c=0)),
    (M.LOCAL_GLOBAL, dict(l=4, c=7)), (M.LOCAL_GLOBAL, dict(l=1, c=30)),
    (M.STRIDED_MERGED, dict(l=1)), (M.STRIDED_MERGED, dict(l=3)), (M.STRIDED_MERGED, dict(l=8)),
    (M.STRIDED_MERGED, dict(l=40)),
]


def _read_golden_matrix(path):
    rows, meta = [], {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            if len(parts) == 2 and not set(parts[0]) <= {"0", "1"}:
                meta[parts[0]] = int(parts[1])
            else:
                rows.append([ch == "1" for ch in line])
    return meta, np.array(rows, dtype=bool)


def test_local_global_worked_example(golden_dir):
    """Blog post on sliding windows, section 04: the printed 8x8 table, all rows."""
    meta, expect = _read_golden_matrix(os.path.join(golden_dir, "local_global_8x8.txt"))
    got = M.local_global_mask(meta["length"], meta["window"], (meta["global"],))
    np.testing.assert_array_equal(got, expect)
    # Section 04 / 07 statements.
    assert np.flatnonzero(got[7]).tolist() == [0, 5, 6, 7]
    assert not got[3, 4]
    assert got.any(axis=1).all()
    assert got.sum(axis=1).tolist() == [1, 2, 3, 4, 4, 4, 4, 4]
    assert got.sum() == 26


def test_local_global_mask_global_token_in_the_middle():
    """Blog post on sliding windows, sections 03-04, worked by hand for a global
    token that is not the first one: n = 6, window 1, G = {3}.  Row 3 is a global
    query (its whole causal history); rows 4 and 5 add key 3 to their windows;
    rows before 3 cannot read it (causality)."""
    expect = {0: [0], 1: [0, 1], 2: [1, 2], 3: [0, 1, 2, 3], 4: [3, 4], 5: [3, 4, 5]}
    got = M.local_global_mask(6, 1, (3,))
    for i, keys in expect.items():
        assert np.flatnonzero(got[i]).tolist() == keys, i
    # Two global tokens, one of them past a row: window 0 (only itself), G = {1, 4}.
    got = M.local_global_mask(6, 0, (1, 4))
    assert [np.flatnonzero(r).tolist() for r in got] == [[0], [0, 1], [1, 2], [1, 3], [0, 1, 2, 3, 4], [1, 4, 5]]
    with pytest.raises(ValueError):
        M.local_global_mask(6, 1, (6,))


def test_local_global_rejects_bad_args():
    """Section 07 asserts length > 0 and window >= 0."""
    with pytest.raises(ValueError):
        M.local_global_mask(0, 2)
    with pytest.raises(ValueError):
        M.local_global_mask(8, -1)


def test_causal_window_exercise():
    """Blog post, section 15: L = 10, w = 2 causal window; rows 0, 1, 5, 9 and the edge total.

    The exercise prints no answer; by the definition of section 03
    (0 <= i - j <= w) row i reads max(0, i - w) .. i, so the total is
    L (w + 1) minus the w (w + 1) / 2 pairs clipped at the start.
    """
    m = M.head_mask(10, M.LOCAL, l=2)
    assert np.flatnonzero(m[0]).tolist() == [0]
    assert np.flatnonzero(m[1]).tolist() == [0, 1]
    assert np.flatnonzero(m[5]).tolist() == [3, 4, 5]
    assert np.flatnonzero(m[9]).tolist() == [7, 8, 9]
    assert m.sum() == 27 == 10 * 3 - 3
    # The same band without global tokens is the local head of the strided pattern.
    np.testing.assert_array_equal(M.local_global_mask(10, 2, ()), m)


def _parse_ranges(tokens):
    out = []
    for t in tokens:
        a, b = t.split("-")
        out.extend(range(int(a), int(b) + 1))
    return out


def test_summary_printed_example(golden_dir):
    """Report section 2.2: l = 128, c = 8, positions past 128 see 120..128, past 256 see 248..256."""
    l = c = None
    cases = []
    with open(os.path.join(golden_dir, "summary_l128_c8.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            p = line.split()
            if p[0] == "l":
                l = int(p[1])
            elif p[0] == "c":
                c = int(p[1])
            else:
                cases.append((int(p[0]), _parse_ranges(p[1:])))
    n = 512
    mask = M.head_mask(n, M.SUMMARY, l=l, c=c, sub=0)
    for i, keys in cases:
        assert np.flatnonzero(mask[i]).tolist() == keys, i
        assert M.row_keys(M.SUMMARY, i, n, l, c, 0).tolist() == keys
    # Every position past 128 reads all of 120..127; every position past 256 all of 248..255.
    assert mask[128:, 120:128].all()
    assert mask[256:, 248:256].all()
    assert not mask[:, 128:248].any()


def test_fixed_merged_worked_example(golden_dir):
    """Report sections 2.2 and 3.1 (Eq. 7): a hand-worked 8-token merged fixed head."""
    meta, expect = _read_golden_matrix(os.path.join(golden_dir, "fixed_merged_n8_l4_c1.txt"))
    n, l, c = meta["length"], meta["l"], meta["c"]
    got = M.head_mask(n, M.FIXED_MERGED, l, c, 0)
    np.testing.assert_array_equal(got, expect)
    for i in range(n):
        assert M.row_keys(M.FIXED_MERGED, i, n, l, c, 0).tolist() == np.flatnonzero(expect[i]).tolist()
    assert got.sum() == 24


def test_fixed_merged_totals_and_special_cases():
    """Closed-form totals of the merged fixed head; c = l reads every j <= i."""
    n, l, c = 12288, 128, 32
    mb = n // l
    total = mb * l * (l + 1) // 2 + c * l * mb * (mb - 1) // 2
    assert total == 19470336
    for sub in (0, 3):
        got = sum(M.row_keys(M.FIXED_MERGED, i, n, l, c, sub).size for i in range(n))
        assert got == total
    # With c = l every position is a summary cell: dense causal.
    m = M.head_mask(40, M.FIXED_MERGED, 8, 8, 0)
    np.testing.assert_array_equal(m, np.tril(np.ones((40, 40), dtype=bool)))


def test_strided_merged_worked_example(golden_dir):
    """Report sections 2.2 and 3.1 (Eq. 7): a hand-worked 8-token merged strided head."""
    meta, expect = _read_golden_matrix(os.path.join(golden_dir, "strided_merged_n8_l2.txt"))
    n, l = meta["length"], meta["l"]
    got = M.head_mask(n, M.STRIDED_MERGED, l)
    np.testing.assert_array_equal(got, expect)
    for i in range(n):
        assert M.row_keys(M.STRIDED_MERGED, i, n, l).tolist() == np.flatnonzero(expect[i]).tolist()
    assert got.sum() == 27
    # The union covers every j <= i within one hop of the row itself or of a
    # stride member (report section 2.1): with l = 1 it is dense causal.
    np.testing.assert_array_equal(M.head_mask(30, M.STRIDED_MERGED, 1),
                                  np.tril(np.ones((30, 30), dtype=bool)))


def test_strided_merged_total_12288():
    """Closed-form total of the merged strided head at n = 12,288, l = 128."""
    n, l = 12288, 128
    band = l * (l + 1) // 2 + (n - l) * (l + 1)
    stride = l * (n // l) * (n // l + 1) // 2
    overlap = n + (n - l)  # i itself, and i - l for i >= l
    assert band + stride - overlap == 2148416
    assert sum(M.row_keys(M.STRIDED_MERGED, i, n, l).size for i in range(n)) == 2148416


def test_local_global_kind_is_the_worked_example(golden_dir):
    """Blog post section 04: window 2 plus global token 0 as the head kind (c = 1 leading token)."""
    meta, expect = _read_golden_matrix(os.path.join(golden_dir, "local_global_8x8.txt"))
    assert meta["global"] == 0
    got = M.head_mask(meta["length"], M.LOCAL_GLOBAL, meta["window"], 1)
    np.testing.assert_array_equal(got, expect)
    # Several leading global tokens agree with the dense form of arbitrary global positions.
    np.testing.assert_array_equal(M.head_mask(50, M.LOCAL_GLOBAL, 4, 6),
                                  M.local_global_mask(50, 4, tuple(range(6))))
    # No global tokens: the local head of the strided pattern.
    np.testing.assert_array_equal(M.head_mask(30, M.LOCAL_GLOBAL, 3, 0), M.head_mask(30, M.LOCAL, 3))
    np.testing.assert_array_equal(M.head_mask(30, M.LOCAL_GLOBAL, 3, None), M.head_mask(30, M.LOCAL, 3))
    with pytest.raises(ValueError):
        M.head_mask(10, M.LOCAL_GLOBAL, 3, -1)


def test_summary_start_of_sub_blocks():
    """Report section 2.2: several summary heads take different c-sized sub-blocks of the l-block."""
    assert [M.summary_start(128, 32, k) for k in range(5)] == [96, 64, 32, 0, 96]
    assert M.summary_start(128, 8, 0) == 120
    with pytest.raises(ValueError):
        M.summary_start(8, 0)
    with pytest.raises(ValueError):
        M.summary_start(8, 9)


def _closed_form_count(kind, i, l, c=None, s=None):
    """Per-row visible counts derived by hand from the set definitions."""
    if kind == M.LOCAL:
        return min(i, l) + 1
    if kind == M.STRIDE:
        return i // l + 1
    if kind == M.SAMEBLOCK:
        return i % l + 1
    if kind == M.FIXED_MERGED:
        # own block up to i, plus c cells of every earlier block (the cells of
        # the own block up to i are already in it)
        return i % l + 1 + (i // l) * c
    if kind == M.STRIDED_MERGED:
        # band min(i, l) + 1 keys, stride i // l + 1 keys; both hold i, and
        # i - l as well once i >= l
        return min(i, l) + i // l + 1 - (1 if i >= l else 0)
    if kind == M.LOCAL_GLOBAL:
        lo = max(0, i - l)
        return i - lo + 1 + min(c, lo)  # window, plus global tokens before it
    cnt = (i // l) * c + min(max(i % l - s + 1, 0), c)
    return cnt if cnt > 0 else 1


@pytest.mark.parametrize("kind,kw", KINDS_SMALL)
@pytest.mark.parametrize("n", [1, 7, 24, 61])
def test_row_counts_closed_form(kind, kw, n):
    m = M.head_mask(n, kind, **kw)
    s = M.summary_start(kw["l"], kw["c"], kw["sub"]) if kind == M.SUMMARY else None
    expect = [_closed_form_count(kind, i, kw["l"], kw.get("c"), s) for i in range(n)]
    assert m.sum(axis=1).tolist() == expect


def test_head_totals_closed_form():
    """Per-head pair totals at the 12,288-token shapes (closed forms summed by hand)."""
    n, l = 12288, 128
    mb = n // l
    local = l * (l + 1) // 2 + (n - l) * (l + 1)
    stride = l * mb * (mb + 1) // 2
    same = mb * l * (l + 1) // 2
    assert (local, stride, same) == (1576896, 595968, 792576)
    c = 32
    for sub, s in enumerate([96, 64, 32, 0]):
        total = c * l * mb * (mb - 1) // 2 + mb * (c * (c + 1) // 2 + c * (l - s - c)) + s
        got = sum(M.row_keys(M.SUMMARY, i, n, l, c, sub).size for i in range(0, n))
        assert got == total
    assert c * l * mb * (mb - 1) // 2 + mb * (c * (c + 1) // 2) + 96 == 18728544
    got_local = sum(M.row_keys(M.LOCAL, i, n, l).size for i in range(n))
    got_stride = sum(M.row_keys(M.STRIDE, i, n, l).size for i in range(n))
    assert (got_local, got_stride) == (local, stride)


@pytest.mark.parametrize("kind,kw", KINDS_SMALL)
def test_row_form_matches_dense_form(kind, kw):
    n = 53
    m = M.head_mask(n, kind, **kw)
    for i in range(n):
        assert M.row_keys(kind, i, n, **kw).tolist() == np.flatnonzero(m[i]).tolist()
    for j in range(n):
        assert M.rows_seeing(kind, j, n, **kw).tolist() == np.flatnonzero(m[:, j]).tolist()


@pytest.mark.parametrize("kind,kw", KINDS_SMALL)
def test_every_row_has_a_key_and_is_causal(kind, kw):
    """Blog post section 02: each row needs >= 1 visible key; report section 2.1: j <= i."""
    m = M.head_mask(70, kind, **kw)
    assert m.any(axis=1).all()
    assert not np.triu(m, 1).any()
    assert m[0, 0]


def test_self_if_empty_only_touches_empty_rows():
    n, l, c = 300, 16, 4
    for sub in range(4):
        s = M.summary_start(l, c, sub)
        raw = M.head_mask(n, M.SUMMARY, l, c, sub, self_if_empty=False)
        fixed = M.head_mask(n, M.SUMMARY, l, c, sub)
        empty = ~raw.any(axis=1)
        assert np.flatnonzero(empty).tolist() == list(range(s))
        assert (fixed ^ raw).sum() == s
        assert all(fixed[i, i] for i in range(s))


def test_count_connections_printed(golden_dir):
    """Numpy demo of the sparse-attention tutorial: n = 64 -> dense 4096, stripe 448, block 512.

    The demo's masks are not causal; the causal heads relate to them by
    symmetry: a symmetric non-causal mask counts 2 * (causal count) - n.
    """
    vals = {}
    with open(os.path.join(golden_dir, "count_connections_n64.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, v = line.split()
                vals[k] = int(v)
    n = vals["n"]
    assert n * n == vals["dense"]
    block = M.head_mask(n, M.SAMEBLOCK, l=8).sum()
    assert 2 * block - n == vals["block_b8"]
    stripe = M.head_mask(n, M.LOCAL, l=3).sum()
    assert 2 * stripe - n == vals["stripe_w3_unclipped"] - 3 * 4
    assert vals["stripe_w3_unclipped"] == n * (2 * 3 + 1)


def _two_hop_covers_causal(union):
    n = union.shape[0]
    u = union.astype(np.int64)
    reach = (u + u @ u) > 0
    lower = np.tril(np.ones((n, n), dtype=bool))
    return bool((reach | ~lower).all())


@pytest.mark.parametrize("n", [16, 30, 64, 100, 256])
def test_strided_union_two_hop(n):
    """Report section 2.1 (any j <= i reachable within p = 2 steps) for the strided pair, l ~ sqrt(n)."""
    for l in sorted({max(1, int(round(np.sqrt(n)))), max(1, int(np.sqrt(n)) - 1), int(np.sqrt(n)) + 2}):
        u = M.head_mask(n, M.LOCAL, l) | M.head_mask(n, M.STRIDE, l)
        assert _two_hop_covers_causal(u), (n, l)


@pytest.mark.parametrize("n,l", [(64, 8), (100, 10), (256, 16), (96, 12)])
def test_fixed_union_two_hop(n, l):
    """Same property for same-block + summary (first summary sub-block), c = 1, 2, 3."""
    for c in (1, 2, 3):
        u = M.head_mask(n, M.SAMEBLOCK, l) | M.head_mask(n, M.SUMMARY, l, c, 0)
        assert _two_hop_covers_causal(u), (n, l, c)


def test_off_by_one_summary_range_fails_two_hop():
    """Pins the reading of the garbled range {t..l}: shifting it down by one breaks reachability."""
    n, l, c = 64, 8, 2
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    shifted = (j <= i) & (j % l >= l - c - 1) & (j % l <= l - 2)
    u = M.head_mask(n, M.SAMEBLOCK, l) | shifted
    assert not _two_hop_covers_causal(u)
    ok = M.head_mask(n, M.SAMEBLOCK, l) | M.head_mask(n, M.SUMMARY, l, c, 0)
    assert _two_hop_covers_causal(ok)


def test_stride_head_is_grid_column_attention():
    """Comparison article, section 2: the stride head is column attention on an (n/l) x l grid."""
    n, l = 96, 8
    m = M.head_mask(n, M.STRIDE, l)
    grid = np.arange(n).reshape(n // l, l)  # row = i // l, column = i % l
    expect = np.zeros((n, n), dtype=bool)
    for col in range(l):
        pos = grid[:, col]
        for a in range(len(pos)):
            expect[pos[a], pos[: a + 1]] = True
    np.testing.assert_array_equal(m, expect)


def test_degenerate_parameters():
    n = 20
    causal = np.tril(np.ones((n, n), dtype=bool))
    np.testing.assert_array_equal(M.head_mask(n, M.LOCAL, l=n), causal)
    np.testing.assert_array_equal(M.head_mask(n, M.LOCAL, l=5 * n), causal)
    np.testing.assert_array_equal(M.head_mask(n, M.STRIDE, l=1), causal)
    np.testing.assert_array_equal(M.head_mask(n, M.SAMEBLOCK, l=n), causal)
    np.testing.assert_array_equal(M.head_mask(n, M.SUMMARY, l=4, c=4), causal)
    np.testing.assert_array_equal(M.head_mask(n, M.STRIDE, l=n), np.eye(n, dtype=bool))
    with pytest.raises(ValueError):
        M.head_mask(n, M.LOCAL, l=0)
    with pytest.raises(ValueError):
        M.head_mask(0, M.LOCAL, l=1)
