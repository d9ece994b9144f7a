"""Pins of the oracle's masked softmax attention (forward and backward).

Independent checks: torch's scaled_dot_product_attention in float64 on the
CPU (a library routine that computes the same masked softmax: the blog post
on sliding windows, section 08, uses it as the dense correctness baseline),
autograd through it, central finite differences, closed forms and exact
invariants.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention as A
from oracle import masks as M


def _rand(n, d, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((n, d)) for _ in range(4)]


def _sdpa(q, k, v, mask=None, causal=False):
    t = [torch.tensor(x, dtype=torch.float64) for x in (q, k, v)]
    am = None if mask is None else torch.tensor(mask)
    return F.scaled_dot_product_attention(*t, attn_mask=am, is_causal=causal).numpy()


HEADS = [(M.LOCAL, dict(l=5)), (M.STRIDE, dict(l=6)), (M.SAMEBLOCK, dict(l=7)),
         (M.SUMMARY, dict(l=8, c=3, sub=0)), (M.SUMMARY, dict(l=8, c=2, sub=2))]


def test_all_ones_mask_is_dense_attention():
    q, k, v, _ = _rand(40, 16, 0)
    o, _ = A.fwd_dense(q, k, v, np.ones((40, 40), dtype=bool))
    np.testing.assert_allclose(o, _sdpa(q, k, v), rtol=0, atol=1e-12)


@pytest.mark.parametrize("case", ["causal", "local_l_ge_n", "sameblock_l_ge_n", "summary_c_eq_l", "stride_l1"])
def test_degenerate_heads_are_causal_attention(case):
    n, d = 37, 8
    q, k, v, _ = _rand(n, d, 1)
    mask = {
        "causal": np.tril(np.ones((n, n), dtype=bool)),
        "local_l_ge_n": M.head_mask(n, M.LOCAL, l=n + 3),
        "sameblock_l_ge_n": M.head_mask(n, M.SAMEBLOCK, l=n),
        "summary_c_eq_l": M.head_mask(n, M.SUMMARY, l=6, c=6),
        "stride_l1": M.head_mask(n, M.STRIDE, l=1),
    }[case]
    o, _ = A.fwd_dense(q, k, v, mask)
    np.testing.assert_allclose(o, _sdpa(q, k, v, causal=True), rtol=0, atol=1e-12)


@pytest.mark.parametrize("kind,kw", HEADS)
def test_masked_forward_matches_sdpa_with_bool_mask(kind, kw):
    n, d = 50, 8
    q, k, v, _ = _rand(n, d, 2)
    mask = M.head_mask(n, kind, **kw)
    o, lse = A.fwd_dense(q, k, v, mask)
    np.testing.assert_allclose(o, _sdpa(q, k, v, mask), rtol=0, atol=1e-12)
    # LSE by its definition, summed with math.fsum row by row.
    s = (q @ k.T) / math.sqrt(d)
    for i in range(n):
        ref = math.log(math.fsum(math.exp(x) for x in s[i, mask[i]]))
        assert abs(lse[i] - ref) < 1e-12


def test_stride_head_longer_than_sequence_is_identity():
    """Stride l >= n: each row reads only itself, so O_i = v_i and LSE_i = S_ii."""
    n, d = 20, 8
    q, k, v, _ = _rand(n, d, 3)
    o, lse = A.fwd_dense(q, k, v, M.head_mask(n, M.STRIDE, l=n))
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, (q * k).sum(1) / math.sqrt(d), rtol=0, atol=1e-14)


def test_stride_head_equals_column_causal_attention():
    """Comparison article, section 2: stride head = causal attention down each grid column."""
    n, l, d = 96, 8, 8
    q, k, v, _ = _rand(n, d, 4)
    o, _ = A.fwd_dense(q, k, v, M.head_mask(n, M.STRIDE, l))
    expect = np.empty_like(o)
    for col in range(l):
        pos = np.arange(col, n, l)
        expect[pos] = _sdpa(q[pos], k[pos], v[pos], causal=True)
    np.testing.assert_allclose(o, expect, rtol=0, atol=1e-12)


@pytest.mark.parametrize("kind,kw", HEADS)
def test_probability_rows_sum_to_one(kind, kw):
    n = 64
    q, k, _, _ = _rand(n, 8, 5)
    p, _ = A.probs_dense(q, k, M.head_mask(n, kind, **kw))
    np.testing.assert_allclose(p.sum(1), 1.0, rtol=0, atol=1e-12)
    assert (p[~M.head_mask(n, kind, **kw)] == 0).all()


def test_empty_row_is_rejected():
    q, k, v, _ = _rand(8, 4, 6)
    m = M.head_mask(8, M.SUMMARY, l=4, c=1, self_if_empty=False)
    with pytest.raises(ValueError):
        A.fwd_dense(q, k, v, m)


def test_masked_value_perturbation_recipe():
    """Blog post section 10: add 10,000 to the value of a masked key; rows that cannot read it are unchanged."""
    q, k, v, _ = _rand(8, 4, 7)
    mask = M.local_global_mask(8, 2)
    assert not mask[7, 3]
    o1, _ = A.fwd_dense(q, k, v, mask)
    v2 = v.copy()
    v2[3] += 10_000
    o2, _ = A.fwd_dense(q, k, v2, mask)
    blind = ~mask[:, 3]
    np.testing.assert_array_equal(o1[blind], o2[blind])
    assert not np.allclose(o1[~blind], o2[~blind])


@pytest.mark.parametrize("kind,kw", HEADS)
def test_backward_matches_autograd_through_sdpa(kind, kw):
    n, d = 45, 8
    q, k, v, do = _rand(n, d, 8)
    mask = M.head_mask(n, kind, **kw)
    dq, dk, dv = A.bwd_dense(q, k, v, mask, do)
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v)]
    out = F.scaled_dot_product_attention(*t, attn_mask=torch.tensor(mask))
    out.backward(torch.tensor(do))
    for got, ref in zip((dq, dk, dv), t):
        np.testing.assert_allclose(got, ref.grad.numpy(), rtol=0, atol=1e-12)


def test_backward_finite_differences():
    """Blog post section 10: compare gradients of the same scalar, L = 8 / d = 4 first (here n = 12)."""
    n, d = 12, 4
    q, k, v, do = _rand(n, d, 9)
    mask = M.head_mask(n, M.LOCAL, 3) | M.head_mask(n, M.STRIDE, 3)
    dq, dk, dv = A.bwd_dense(q, k, v, mask, do)

    def loss(qq, kk, vv):
        o, _ = A.fwd_dense(qq, kk, vv, mask)
        return float((o * do).sum())

    h = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        for idx in [(0, 0), (5, 1), (11, 3), (7, 2)]:
            args = [q.copy(), k.copy(), v.copy()]
            args[which][idx] += h
            up = loss(*args)
            args[which][idx] -= 2 * h
            dn = loss(*args)
            assert abs((up - dn) / (2 * h) - grad[idx]) < 1e-7


@pytest.mark.parametrize("kind,kw", HEADS)
def test_backward_invariants(kind, kw):
    """sum_j dK_j = 0 (scores shift with a common key offset); sum_j dV_j = sum_i dO_i (rows of A sum to 1)."""
    n = 60
    q, k, v, do = _rand(n, 8, 10)
    dq, dk, dv = A.bwd_dense(q, k, v, M.head_mask(n, kind, **kw), do)
    np.testing.assert_allclose(dk.sum(0), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(0), do.sum(0), atol=1e-12)


@pytest.mark.parametrize("kind,kw", HEADS)
def test_row_gather_mode_matches_dense_mode(kind, kw):
    n, d = 70, 8
    q, k, v, do = _rand(n, d, 11)
    mask = M.head_mask(n, kind, **kw)
    kf = A.keys_fn_for(kind, n, **kw)
    rf = A.rows_seeing_fn_for(kind, n, **kw)
    o, lse = A.fwd_dense(q, k, v, mask)
    o2, lse2 = A.fwd_rows(q, k, v, kf)
    np.testing.assert_allclose(o2, o, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, atol=1e-12)
    dq, dk, dv = A.bwd_dense(q, k, v, mask, do)
    g = A.bwd_rows_full(q, k, v, do, kf)
    for a, b in zip(g, (dq, dk, dv)):
        np.testing.assert_allclose(a, b, atol=1e-12)
    rows = [0, 3, 33, 69]
    np.testing.assert_allclose(A.bwd_rows_dq(q, k, v, do, kf, rows), dq[rows], atol=1e-12)
    dk2, dv2 = A.bwd_keys_dkdv(q, k, v, do, kf, rf, rows)
    np.testing.assert_allclose(dk2, dk[rows], atol=1e-12)
    np.testing.assert_allclose(dv2, dv[rows], atol=1e-12)


def test_scale_argument():
    q, k, v, _ = _rand(16, 4, 12)
    mask = np.tril(np.ones((16, 16), dtype=bool))
    o, _ = A.fwd_dense(q, k, v, mask, scale=1.0)
    o2, _ = A.fwd_dense(q * 2.0, k, v, mask)  # 1/sqrt(4) = 0.5 cancels the factor 2
    np.testing.assert_allclose(o, o2, atol=1e-12)
