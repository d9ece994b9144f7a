"""Shared helpers of the GPU parity tests: run the HIP path, run the oracle, compare.

Tolerances (bf16 data, fp32 accumulation): relative RMS
(||x - ref||_2 / ||ref||_2) <= 1e-2 and, element by element,
|x - ref| <= 2e-2 + ulp_bf16(ref) / 2 on O, dQ, dK, dV.  The half-ULP term is
the rounding of the bf16 output itself: at |ref| >= 8 it alone exceeds 2e-2,
so the 2e-2 bar is read as the error beyond the output's own rounding.  LSE
(float32 from exactly the same bf16 inputs) to 1e-3 absolute.  float32 data:
max |err| <= 1e-4 on O.

The element-wise bar also carries the rounding the products' operands take.
Each product runs on bf16 MFMA, so its probability operand (P for O = P V
and dV = P^T dO, dS for dQ = dS K and dK = dS^T Q) is rounded to bf16 first.
An entry summing terms a_i b_i then moves by e = sum_i (bf16(a_i) - a_i) b_i
before any accumulation error (dS also takes D = rowsum(dO O) from the O
the forward stored, bf16(bf16(P) V)); a key that hundreds of rows read with weight
about 1/7 (a global token under a narrow window) makes |e| alone exceed 2e-2.
The bar is 2e-2 + |e| + ulp_bf16(ref) / 2, with e computed from the
oracle's own fp64 probabilities: 2e-2 is read as the error beyond the
rounding of the operands and of the output.
"""

from __future__ import annotations

import numpy as np
import torch

from oracle import attention as OA
from oracle import masks as OM

BF16_MAX_ABS = 2e-2
BF16_REL_RMS = 1e-2
LSE_ABS = 1e-3
FP32_MAX_ABS = 1e-4


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def rel_rms(got: np.ndarray, ref: np.ndarray) -> float:
    den = float(np.linalg.norm(ref))
    return float(np.linalg.norm(got - ref)) / (den if den > 0 else 1.0)


def half_ulp_bf16(ref: np.ndarray) -> np.ndarray:
    """Half the spacing of bfloat16 numbers at |ref| (8 significant bits)."""
    a = np.maximum(np.abs(ref), 2.0 ** -126)
    return 0.5 * np.exp2(np.floor(np.log2(a)) - 7)


def assert_close(name: str, got: np.ndarray, ref: np.ndarray, max_abs: float,
                 rel: float | None = None, bf16_output: bool = False):
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    if not got.size:
        return
    diff = np.abs(got - ref)
    bound = max_abs + (half_ulp_bf16(ref) if bf16_output else 0.0)
    worst = int(np.argmax(diff - bound))
    assert (diff <= bound).all(), (f"{name}: |err| {diff.flat[worst]:.3e} > bound "
                                   f"{np.broadcast_to(bound, diff.shape).flat[worst]:.3e} "
                                   f"at ref {ref.flat[worst]:+.4f} (max |err| {diff.max():.3e})")
    if rel is not None:
        r = rel_rms(got, ref)
        assert r <= rel, f"{name}: rel RMS {r:.3e} > {rel:.1e}"


def operand_rounding_error(q, k, v, do, mask, scale=None) -> dict:
    """|e| per output entry of O, dQ, dK, dV: what rounding the probability
    operand of each product to bf16 alone changes, from the oracle's values.

    The products are those of the oracle's backward (blog post on sliding
    windows and block sparsity, section 02, and the softmax calculus written
    out in the oracle): O = P v, dV = P^T dO, dK = scale dS^T q and
    dQ = scale dS k, with dS = P (dP - D), dP = dO v^T, D = rowsum(P dP).
    The rounded dS takes D from O as the forward stores it, bf16(bf16(P) v).
    """
    p, _ = OA.probs_dense(q, k, mask, scale)
    sc = 1.0 / np.sqrt(q.shape[1]) if scale is None else scale
    dp = do @ v.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    ep = _bf16(p) - p
    # The backward reads O as the forward stored it, bf16(bf16(P) v): D = rowsum(dO O).
    ds_b = _bf16(p * (dp - (do * _bf16(p @ v + ep @ v)).sum(axis=1, keepdims=True)))
    eds = ds_b - ds
    return {"o": np.abs(ep @ v), "dv": np.abs(ep.T @ do),
            "dk": sc * np.abs(eds.T @ q), "dq": sc * np.abs(eds @ k)}


def _bf16(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).to(torch.float64).numpy()


def bf16_bar(operand_error: np.ndarray) -> np.ndarray:
    """Element-wise absolute bar before the output's own half-ULP."""
    return BF16_MAX_ABS + operand_error


def head_args(h):
    return dict(kind=h.kind, l=h.l, c=(h.c or None), sub=h.sub)


def oracle_dense_head(h, n, q, k, v, do=None, bars=False):
    """Oracle forward (and backward when do is given) for one head, dense mode.

    With ``bars`` a fourth item gives the element-wise bf16 bars of O, dQ, dK,
    dV (``bf16_bar`` of ``operand_rounding_error``)."""
    mask = OM.head_mask(n, h.kind, h.l, h.c or None, h.sub)
    o, lse = OA.fwd_dense(q, k, v, mask)
    g = None if do is None else OA.bwd_dense(q, k, v, mask, do)
    if not bars:
        return o, lse, g
    err = operand_rounding_error(q, k, v, do if do is not None else np.zeros_like(q), mask)
    return o, lse, g, {nm: bf16_bar(x) for nm, x in err.items()}


def run_gpu(layout, inp: dict, backward: bool, device="cuda:0"):
    from factorized_block_sparse_amd import binding as bd
    q, k, v = (inp[x].to(device) for x in ("q", "k", "v"))
    o, lse = bd.sparse_attn_fwd(layout, q, k, v)
    out = {"o": o, "lse": lse}
    if backward:
        do = inp["do"].to(device)
        dq, dk, dv = bd.sparse_attn_bwd(layout, q, k, v, o, lse, do)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {kk: to64(vv) for kk, vv in out.items()}
