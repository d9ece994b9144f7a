"""Token-level visibility sets of the factorized attention heads (oracle).

TEST INFRASTRUCTURE ONLY: never imported by the product path.

Every head is causal: a query at position i may only read keys j <= i
("Sparse Transformers 深度解读报告", section 2.1: each head's set is a subset
of {j : j <= i}).  The four head kinds are the two factorizations of section
2.2 of the same report:

* strided, head 1 (``local``):    A_i = {max(0, i - l), ..., i}
* strided, head 2 (``stride``):   A_i = {j <= i : (i - j) mod l == 0}
* fixed, head 1 (``sameblock``):  A_i = {j <= i : floor(j / l) == floor(i / l)}
* fixed, head 2 (``summary``):    A_i = {j <= i : s <= j mod l <= s + c - 1}
  with s = l - c for the first summary head.

Readings where the page is garbled or silent, each with its reason:

* The summary range is printed as {t, ..., l} with t = l - c; since
  j mod l never equals l, the range taken is the c residues l - c ... l - 1.
  The printed example (l = 128, c = 8: positions past 128 see 120..128,
  past 256 see 248..256) is read as half-open ranges [120, 128) and
  [248, 256), which holds exactly c = 8 cells each.
* Several summary heads use different c-wide sub-blocks of the l-block
  (report, section 2.2, tuning notes); the k-th summary head uses
  s = l - (k' + 1) c with k' = k mod (l // c).  Only k = 0 is printed:
  parity of k >= 1 is unpinned beyond that reading.
* A query row whose set is empty would make the softmax undefined (NaN);
  the blog post on sliding windows and block sparsity (section 02) requires
  at least one visible key per row.  Only summary heads produce such rows
  (positions i < s of the first l-block).  Reading: such a row sees itself
  and nothing else ("self-if-empty"); every non-empty row is unchanged.

The local + global-token pattern of the same blog post (sections 04, 07 and
09) is here as well, because its 8-token worked example pins the causal
local band.

Two further head kinds combine sets in one head:

* ``strided_merged``: one head reads the union of the two strided-pattern
  sets, A_i = local_i | stride_i (the same merged integration of report
  section 3.1, Eq. 7, applied to the strided pattern).
* ``fixed_merged``: one head reads the union of the two fixed-pattern sets,
  A_i = same-block_i | summary_i (the merged integration of report section
  3.1, Eq. 7, which the Enwik8 model used; report section 4).  No row is
  empty (every row reads itself through its own block).
* ``local_global``: the causal window of width l plus the first c positions
  as global tokens (blog post sections 03 and 04): A_i = {j <= i : i - j <= l
  or j < c}.  A global query (i < c) reads every j <= i, as section 04 asks.
  Reading: the head kind puts the global tokens at the front; the dense
  ``local_global_mask`` keeps arbitrary global positions.
"""

from __future__ import annotations

import numpy as np

LOCAL = "local"
STRIDE = "stride"
SAMEBLOCK = "sameblock"
SUMMARY = "summary"
FIXED_MERGED = "fixed_merged"
LOCAL_GLOBAL = "local_global"
STRIDED_MERGED = "strided_merged"
KINDS = (LOCAL, STRIDE, SAMEBLOCK, SUMMARY, FIXED_MERGED, LOCAL_GLOBAL, STRIDED_MERGED)


def summary_start(l: int, c: int, sub: int = 0) -> int:
    """First residue s of the c-wide summary sub-block used by summary head ``sub``.

    Report section 2.2: the summary cells are the last c positions of each
    l-block (s = l - c); with several summary heads each attends to a
    different c-sized sub-block.  Head ``sub`` takes the (sub mod (l // c))-th
    sub-block counted from the end of the l-block.
    """
    if not (1 <= c <= l):
        raise ValueError("summary width c must satisfy 1 <= c <= l")
    nsub = l // c
    k = sub % nsub
    return l - (k + 1) * c


def visible(kind: str, i, j, l: int, c: int | None = None, sub: int = 0):
    """Vectorised predicate "query i reads key j" before the self-if-empty rule.

    ``i`` and ``j`` broadcast against each other (numpy integer arrays).
    Report section 2.2 for the four sets; every set is intersected with the
    causal condition j <= i of section 2.1.
    """
    i = np.asarray(i, dtype=np.int64)
    j = np.asarray(j, dtype=np.int64)
    if l < 1:
        raise ValueError("l must be >= 1")
    causal = (j <= i) & (j >= 0)
    if kind == LOCAL:
        return causal & (i - j <= l)
    if kind == STRIDE:
        return causal & (np.mod(i - j, l) == 0)
    if kind == SAMEBLOCK:
        return causal & (j // l == i // l)
    if kind == SUMMARY:
        s = summary_start(l, c, sub)
        r = np.mod(j, l)
        return causal & (r >= s) & (r <= s + c - 1)
    if kind == FIXED_MERGED:
        return visible(SAMEBLOCK, i, j, l) | visible(SUMMARY, i, j, l, c, sub)
    if kind == STRIDED_MERGED:
        return visible(LOCAL, i, j, l) | visible(STRIDE, i, j, l)
    if kind == LOCAL_GLOBAL:
        g = 0 if c is None else c  # None: no global tokens
        if g < 0:
            raise ValueError("need a number of global tokens c >= 0")
        return causal & ((i - j <= l) | (j < g))
    raise ValueError(f"unknown head kind {kind!r}")


def head_mask(n: int, kind: str, l: int, c: int | None = None, sub: int = 0,
              self_if_empty: bool = True) -> np.ndarray:
    """Dense boolean adjacency M[i, j] (True = query i reads key j), shape [n, n].

    The adjacency-matrix view of the blog post on sliding windows and block
    sparsity, section 02.  With ``self_if_empty`` a row with no visible key
    gets its own diagonal entry and nothing else.
    """
    if n <= 0:
        raise ValueError("n must be positive")
    idx = np.arange(n, dtype=np.int64)
    m = visible(kind, idx[:, None], idx[None, :], l, c, sub)
    if self_if_empty:
        empty = ~m.any(axis=1)
        m[idx[empty], idx[empty]] = True
    return m


def row_keys(kind: str, i: int, n: int, l: int, c: int | None = None,
             sub: int = 0, self_if_empty: bool = True) -> np.ndarray:
    """Sorted key positions read by query ``i`` (row-gather form).

    Enumerates each set of report section 2.2 directly instead of testing all
    j, so that long rows stay cheap.  Must agree with :func:`head_mask` row by
    row (checked exhaustively on small n by the tests).
    """
    if not (0 <= i < n):
        raise ValueError("row out of range")
    if kind == LOCAL:
        keys = np.arange(max(0, i - l), i + 1, dtype=np.int64)
    elif kind == STRIDE:
        keys = np.arange(i % l, i + 1, l, dtype=np.int64)
    elif kind == SAMEBLOCK:
        keys = np.arange((i // l) * l, i + 1, dtype=np.int64)
    elif kind == SUMMARY:
        s = summary_start(l, c, sub)
        blocks = np.arange(i // l + 1, dtype=np.int64)
        keys = (blocks[:, None] * l + s + np.arange(c, dtype=np.int64)[None, :]).ravel()
        keys = keys[keys <= i]
    elif kind == FIXED_MERGED:
        keys = np.union1d(row_keys(SAMEBLOCK, i, n, l),
                          row_keys(SUMMARY, i, n, l, c, sub, self_if_empty=False))
    elif kind == STRIDED_MERGED:
        keys = np.union1d(row_keys(LOCAL, i, n, l), row_keys(STRIDE, i, n, l))
    elif kind == LOCAL_GLOBAL:
        g = 0 if c is None else c
        if g < 0:
            raise ValueError("need a number of global tokens c >= 0")
        keys = np.union1d(np.arange(0, min(g, i + 1), dtype=np.int64),
                          np.arange(max(0, i - l), i + 1, dtype=np.int64))
    else:
        raise ValueError(f"unknown head kind {kind!r}")
    if keys.size == 0 and self_if_empty:
        keys = np.array([i], dtype=np.int64)
    return keys


def rows_seeing(kind: str, j: int, n: int, l: int, c: int | None = None,
                sub: int = 0, self_if_empty: bool = True) -> np.ndarray:
    """Sorted query rows whose set contains key ``j`` (the transpose of :func:`row_keys`)."""
    if not (0 <= j < n):
        raise ValueError("key out of range")
    rows = np.arange(j, n, dtype=np.int64)
    hit = visible(kind, rows, j, l, c, sub)
    if self_if_empty and not hit[0]:
        # Row j reads key j through the self-if-empty rule only when row j's
        # own set is empty.
        if row_keys(kind, j, n, l, c, sub, self_if_empty=False).size == 0:
            hit[0] = True
    return rows[hit]


def local_global_mask(n: int, window: int, global_tokens=(0,)) -> np.ndarray:
    """Causal sliding window plus global tokens, as a set per query row.

    Blog post on sliding windows, sections 03 and 04: query i reads key j iff
    j <= i and at least one of (a) i - j <= window (the causal window),
    (b) j is a global token, (c) i is a global token (a global query reads
    its whole causal history).  Section 07 states the argument checks
    (length > 0, window >= 0).
    """
    if not (n > 0 and window >= 0):
        raise ValueError("need n > 0 and window >= 0")
    g = np.unique(np.asarray(list(global_tokens), dtype=np.int64))
    if g.size and (g[0] < 0 or g[-1] >= n):
        raise ValueError("global tokens must lie in [0, n)")
    pos = np.arange(n, dtype=np.int64)
    in_g = np.isin(pos, g)
    i, j = pos[:, None], pos[None, :]
    return (j <= i) & ((i - j <= window) | in_g[None, :] | in_g[:, None])
