"""Shared helpers of the GPU parity tests: run the HIP path, run the oracle, compare.

Tolerances (bf16 data, fp32 accumulation): relative RMS
(||x - ref||_2 / ||ref||_2) <= 1e-2 and, element by element,
|x - ref| <= 2e-2 + ulp_bf16(ref) / 2 on O, dQ, dK, dV.  The half-ULP term is
the rounding of the bf16 output itself: at |ref| >= 8 it alone exceeds 2e-2,
so the 2e-2 bar is read as the error beyond the output's own rounding.  LSE
(float32 from exactly the same bf16 inputs) to 1e-3 absolute.  float32 data:
max |err| <= 1e-4 on O.
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


def head_args(h):
    return dict(kind=h.kind, l=h.l, c=(h.c or None), sub=h.sub)


def oracle_dense_head(h, n, q, k, v, do=None):
    """Oracle forward (and backward when do is given) for one head, dense mode."""
    mask = OM.head_mask(n, h.kind, h.l, h.c or None, h.sub)
    o, lse = OA.fwd_dense(q, k, v, mask)
    if do is None:
        return o, lse, None
    return (o, lse, OA.bwd_dense(q, k, v, mask, do))


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
