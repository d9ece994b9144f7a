"""Masked softmax attention, forward and backward, in float64 (oracle).

TEST INFRASTRUCTURE ONLY: never imported by the product path.

Definition (blog post on sliding windows and block sparsity, section 02, and
its section 01 for the score scaling): with S_ij = scale * q_i . k_j and a
boolean adjacency M,

    A_ij = exp(S_ij) M_ij / sum_{k : M_ik} exp(S_ik),     o_i = sum_j A_ij v_j.

scale defaults to 1 / sqrt(d).  The per-row log-sum-exp
LSE_i = log sum_{j : M_ij} exp(S_ij) is returned too: it is what the
recomputation-based backward needs ("Sparse Transformers 深度解读报告",
section 3.4: attention weights are not kept from the forward pass, they are
rebuilt in the backward pass).

Backward of the same scalar with upstream gradient dO (standard softmax
calculus, written out):

    dV_j  = sum_i A_ij dO_i
    dP_ij = dO_i . v_j
    D_i   = sum_j A_ij dP_ij
    dS_ij = A_ij (dP_ij - D_i)
    dQ_i  = scale * sum_j dS_ij k_j
    dK_j  = scale * sum_i dS_ij q_i

Two modes: dense (an [n, n] mask, for n up to a few thousand) and row-gather
(each row's visible keys are enumerated, gathered and reduced; any n).
Every row must have at least one visible key (the same section 02: an empty
row would give NaN); both modes raise otherwise.
"""

from __future__ import annotations

import math
from typing import Callable, Iterable

import numpy as np

from . import masks as _masks


def _scale(d: int, scale: float | None) -> float:
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def _as64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------
# dense-mask mode (one [n, d] head at a time)
# --------------------------------------------------------------------------

def probs_dense(q, k, mask, scale: float | None = None):
    """Row-normalised attention matrix A [n, n] and LSE [n] for one head."""
    q = _as64(q)
    k = _as64(k)
    mask = np.asarray(mask, dtype=bool)
    if not mask.any(axis=1).all():
        raise ValueError("every query row needs at least one visible key")
    sc = _scale(q.shape[-1], scale)
    s = sc * (q @ k.T)
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    z = e.sum(axis=1)
    return e / z[:, None], m + np.log(z)


def fwd_dense(q, k, v, mask, scale: float | None = None):
    """Forward for one head: returns (O [n, d], LSE [n])."""
    p, lse = probs_dense(q, k, mask, scale)
    return p @ _as64(v), lse


def bwd_dense(q, k, v, mask, do, scale: float | None = None):
    """Backward for one head: returns (dQ, dK, dV), each [n, d]."""
    q, k, v, do = map(_as64, (q, k, v, do))
    sc = _scale(q.shape[-1], scale)
    p, _ = probs_dense(q, k, mask, scale)
    dv = p.T @ do
    dp = do @ v.T
    dd = (p * dp).sum(axis=1)
    ds = p * (dp - dd[:, None])
    dq = sc * (ds @ k)
    dk = sc * (ds.T @ q)
    return dq, dk, dv


# --------------------------------------------------------------------------
# row-gather mode
# --------------------------------------------------------------------------

KeysFn = Callable[[int], np.ndarray]


def keys_fn_for(kind: str, n: int, l: int, c: int | None = None, sub: int = 0,
                self_if_empty: bool = True) -> KeysFn:
    """Row -> visible key positions for one head pattern (report section 2.2)."""
    def f(i: int) -> np.ndarray:
        return _masks.row_keys(kind, i, n, l, c, sub, self_if_empty)
    return f


def _row_probs(q, k, i: int, keys: np.ndarray, sc: float):
    if keys.size == 0:
        raise ValueError(f"query row {i} has no visible key")
    s = sc * (k[keys] @ q[i])
    m = s.max()
    e = np.exp(s - m)
    z = e.sum()
    return e / z, m + math.log(z)


def fwd_rows(q, k, v, keys_fn: KeysFn, rows: Iterable[int] | None = None,
             scale: float | None = None):
    """Forward for the listed rows of one head: returns (O [r, d], LSE [r])."""
    q, k, v = map(_as64, (q, k, v))
    n, d = q.shape
    sc = _scale(d, scale)
    rows = range(n) if rows is None else list(rows)
    out = np.empty((len(rows), d))
    lse = np.empty(len(rows))
    for t, i in enumerate(rows):
        keys = keys_fn(i)
        p, lse[t] = _row_probs(q, k, i, keys, sc)
        out[t] = p @ v[keys]
    return out, lse


def bwd_rows_full(q, k, v, do, keys_fn: KeysFn, scale: float | None = None,
                  rows: Iterable[int] | None = None):
    """Backward over all rows (or a subset) of one head: (dQ, dK, dV), each [n, d].

    With ``rows`` given, only those query rows contribute (dQ of other rows
    stays 0 and dK/dV hold partial sums): used to time a bounded sample.
    """
    q, k, v, do = map(_as64, (q, k, v, do))
    n, d = q.shape
    sc = _scale(d, scale)
    dq = np.zeros((n, d))
    dk = np.zeros((n, d))
    dv = np.zeros((n, d))
    for i in (range(n) if rows is None else rows):
        keys = keys_fn(i)
        p, _ = _row_probs(q, k, i, keys, sc)
        dp = v[keys] @ do[i]
        dd = p @ dp
        ds = p * (dp - dd)
        dv[keys] += np.outer(p, do[i])
        dq[i] = sc * (ds @ k[keys])
        dk[keys] += sc * np.outer(ds, q[i])
    return dq, dk, dv


def bwd_rows_dq(q, k, v, do, keys_fn: KeysFn, rows: Iterable[int],
                scale: float | None = None):
    """dQ for the listed rows only: each needs nothing but its own row."""
    q, k, v, do = map(_as64, (q, k, v, do))
    sc = _scale(q.shape[1], scale)
    rows = list(rows)
    out = np.empty((len(rows), q.shape[1]))
    for t, i in enumerate(rows):
        keys = keys_fn(i)
        p, _ = _row_probs(q, k, i, keys, sc)
        dp = v[keys] @ do[i]
        ds = p * (dp - p @ dp)
        out[t] = sc * (ds @ k[keys])
    return out


def bwd_keys_dkdv(q, k, v, do, keys_fn: KeysFn, rows_seeing_fn: KeysFn,
                  key_ids: Iterable[int], scale: float | None = None):
    """dK and dV for the listed keys only: (dK [r, d], dV [r, d]).

    Key j collects from every query row that reads it; each such row's full
    softmax is rebuilt from that row's own keys.
    """
    q, k, v, do = map(_as64, (q, k, v, do))
    sc = _scale(q.shape[1], scale)
    key_ids = list(key_ids)
    dk = np.zeros((len(key_ids), q.shape[1]))
    dv = np.zeros((len(key_ids), q.shape[1]))
    for t, j in enumerate(key_ids):
        for i in rows_seeing_fn(j):
            keys = keys_fn(int(i))
            p, _ = _row_probs(q, k, int(i), keys, sc)
            dp = v[keys] @ do[i]
            dd = p @ dp
            pos = int(np.searchsorted(keys, j))
            if pos >= keys.size or keys[pos] != j:
                raise AssertionError("rows_seeing and row_keys disagree")
            pij = p[pos]
            dv[t] += pij * do[i]
            dk[t] += sc * pij * (dp[pos] - dd) * q[i]
    return dk, dv


def rows_seeing_fn_for(kind: str, n: int, l: int, c: int | None = None, sub: int = 0,
                       self_if_empty: bool = True) -> KeysFn:
    """Key -> query rows that read it, for one head pattern."""
    def f(j: int) -> np.ndarray:
        return _masks.rows_seeing(kind, j, n, l, c, sub, self_if_empty)
    return f
