"""The element-wise bf16 bars of the GPU parity tests (host arithmetic, no GPU).

A kernel that runs its products on bf16 MFMA rounds the probability operand
(P, dS) to bf16 before each product.  Modelled here on the CPU from the
oracle's own probabilities: round that operand to bf16, sum exactly, round
the result to bf16.  A key that every row reads with weight about 1/7 (two
global tokens under a 4-wide window) then misses the flat 2e-2 bar on dV
while the model stays inside the bar that adds the operand rounding; on
ordinary heads the added term stays small, and a dropped term still fails.
"""

import numpy as np
import pytest
import torch

from factorized_block_sparse_amd import workloads as W
from oracle import attention as OA
from oracle import masks as OM
from tests.parity_util import BF16_MAX_ABS, bf16_bar, half_ulp_bf16, operand_rounding_error


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).to(torch.float64).numpy()


def _model(kind, l, c, n, seed, heads=1, h=0):
    """Kernel-style results (bf16 operands and outputs, exact sums), the
    oracle's, and the operand-rounding term of the bar."""
    inp = W.make_inputs(1, heads, n, 64, seed=seed)
    q, k, v, do = (inp[x][0, h].to(torch.float64).numpy() for x in ("q", "k", "v", "do"))
    mask = OM.head_mask(n, kind, l, c)
    p, _ = OA.probs_dense(q, k, mask)
    dq, dk, dv = OA.bwd_dense(q, k, v, mask, do)
    o_b = _bf16(_bf16(p) @ v)
    dp = do @ v.T
    ds_b = _bf16(p * (dp - (do * o_b).sum(axis=1, keepdims=True)))
    got = {"o": o_b, "dv": _bf16(_bf16(p).T @ do), "dk": _bf16(ds_b.T @ q / 8.0), "dq": _bf16(ds_b @ k / 8.0)}
    ref = {"o": p @ v, "dq": dq, "dk": dk, "dv": dv}
    return got, ref, operand_rounding_error(q, k, v, do, mask), (q, k, v, do, mask, p)


# The first case is head 0 of a seeded two-head input at n = 607.
@pytest.mark.parametrize("kind,l,c,n,seed,heads", [("local_global", 4, 2, 607, 9205, 2),
                                                   ("local_global", 1, 3, 1500, 0, 1),
                                                   ("local_global", 4, 1, 1500, 1, 1)])
def test_heavy_key_columns_need_the_operand_rounding(kind, l, c, n, seed, heads):
    got, ref, oe, _ = _model(kind, l, c, n, seed, heads)
    err = np.abs(got["dv"] - ref["dv"])
    half = half_ulp_bf16(ref["dv"])
    assert (err > BF16_MAX_ABS + half).any()
    for nm in ("o", "dq", "dk", "dv"):
        err = np.abs(got[nm] - ref[nm])
        assert (err <= bf16_bar(oe[nm]) + half_ulp_bf16(ref[nm])).all(), nm


@pytest.mark.parametrize("kind,l,c", [("local", 32, None), ("stride", 32, None), ("sameblock", 64, None),
                                      ("summary", 64, 8), ("fixed_merged", 64, 8), ("local_global", 64, 16),
                                      ("strided_merged", 24, None)])
def test_ordinary_heads_stay_near_the_flat_bar(kind, l, c):
    got, ref, oe, _ = _model(kind, l, c, 700, 7)
    for nm in ("o", "dq", "dk", "dv"):
        assert oe[nm].max() < 0.75 * BF16_MAX_ABS, nm
        err = np.abs(got[nm] - ref[nm])
        assert (err <= BF16_MAX_ABS + half_ulp_bf16(ref[nm])).all(), nm


def test_a_dropped_row_still_fails_on_a_heavy_key():
    """dV of a global key with one reading row left out: outside the bar."""
    got, ref, oe, (q, k, v, do, mask, p) = _model("local_global", 4, 2, 607, 9205, 2)
    i = int(np.argmax(p[:, 0] * np.abs(do[:, 0])))
    wrong = ref["dv"][0] - p[i, 0] * do[i]
    assert (np.abs(wrong - ref["dv"][0]) > bf16_bar(oe["dv"][0]) + half_ulp_bf16(ref["dv"][0])).any()
