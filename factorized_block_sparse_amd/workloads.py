"""Seeded synthetic workloads shaped like the pages' experiments.

This module holds no attention arithmetic: it names the head patterns of
each workload and draws the input tensors.  It is the only code shared by the
HIP path's callers and the oracle's callers (the tests hand the same tensors
to both).

The pages measure on Enwik8 (context 12,288), CIFAR-10 (context 3,072) and
raw audio (length 65,536) ("Sparse Transformers 深度解读报告", sections 4.1,
4.2 and 4.4).  Those datasets are not used: seeded Gaussian tensors of the
same sequence lengths stand in for their activations.

Recipe for every workload: ``torch.Generator('cpu').manual_seed(seed)``;
draw Q, K, V, dO in that order as float32 ``randn`` of shape [B, H, n, d];
optionally add the shared sinusoid to Q and K; cast to the workload dtype
(bfloat16 by round-to-nearest-even).  The same bytes go to the GPU and,
upcast to float64, to the oracle.

Head assignment within one call: heads alternate between the two kinds of a
pattern (report, section 3.1, the multi-head integration): even heads use the
first kind (local band / same block), odd heads the second (stride / summary
columns); the k-th summary head uses the k-th c-wide sub-block.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

LOCAL = "local"
STRIDE = "stride"
STRIDED_MERGED = "strided_merged"
SAMEBLOCK = "sameblock"
SUMMARY = "summary"
FIXED_MERGED = "fixed_merged"
LOCAL_GLOBAL = "local_global"


@dataclass(frozen=True)
class HeadSpec:
    kind: str
    l: int
    c: int = 0
    sub: int = 0


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    n: int
    d: int
    heads: tuple
    dtype: str            # "bf16" or "fp32"
    block_q: int
    block_k: int
    seed: int
    backward: bool = True
    sinusoid: bool = False
    note: str = field(default="", compare=False)


def strided_heads(H: int, l: int) -> tuple:
    """Alternating local-band / stride heads (report section 2.2, strided attention)."""
    return tuple(HeadSpec(LOCAL, l) if h % 2 == 0 else HeadSpec(STRIDE, l) for h in range(H))


def merged_heads(H: int, l: int, c: int) -> tuple:
    """Merged fixed heads (report section 3.1, Eq. 7): head k reads its block and sub-block k's cells."""
    return tuple(HeadSpec(FIXED_MERGED, l, c, h) for h in range(H))


def fixed_heads(H: int, l: int, c: int) -> tuple:
    """Alternating same-block / summary heads; summary head k uses sub-block k."""
    return tuple(HeadSpec(SAMEBLOCK, l) if h % 2 == 0 else HeadSpec(SUMMARY, l, c, h // 2)
                 for h in range(H))


WORKLOADS = {
    w.name: w for w in (
        Workload("strided_n1024_fp32", 1, 2, 1024, 64, strided_heads(2, 32), "fp32", 32, 32,
                 1001, backward=False,
                 note="strided pattern, forward only, float32, 32x32 tiles"),
        Workload("strided_n3072", 4, 8, 3072, 64, strided_heads(8, 64), "bf16", 64, 64, 1002,
                 note="strided pattern at the CIFAR-10 context length"),
        Workload("fixed_n12288", 2, 8, 12288, 64, fixed_heads(8, 128, 32), "bf16", 128, 128, 1003,
                 note="fixed pattern at the Enwik8 context length, l=128, c=32"),
        Workload("strided_n12288", 1, 16, 12288, 64, strided_heads(16, 128), "bf16", 32, 32, 1004,
                 sinusoid=True,
                 note="strided pattern at 12,288 with a shared period-128 sinusoid in Q and K; "
                      "32x32 tiles (the 96-token residue classes of the stride head fill whole "
                      "tiles; fastest in a sweep of tile shapes)"),
        Workload("fixed_c8_n12288", 2, 8, 12288, 64, fixed_heads(8, 128, 8), "bf16", 128, 64, 1006,
                 note="fixed pattern with narrow summaries (l=128, c=8, the report's own example); "
                      "the summary cells of consecutive blocks are packed into dense key tiles"),
        Workload("fixed_merged_n12288", 2, 8, 12288, 64, merged_heads(8, 128, 32), "bf16", 128, 64,
                 1007, note="merged fixed heads at the Enwik8 context length (the report's Enwik8 "
                            "model: fixed pattern, l=128, c=32, merged heads), head k on sub-block k"),
        Workload("local_global_n12288", 2, 8, 12288, 64,
                 tuple(HeadSpec(LOCAL_GLOBAL, 256, 64) for _ in range(8)), "bf16", 64, 64, 1008,
                 note="causal window of 256 plus 64 leading global tokens (blog post sections 03-04)"),
        Workload("strided_merged_n12288", 1, 16, 12288, 64,
                 tuple(HeadSpec(STRIDED_MERGED, 128) for _ in range(16)), "bf16", 32, 32, 1009,
                 sinusoid=True,
                 note="merged strided heads (local band and stride in one head, l=128) at "
                      "12,288 with the shared period-128 sinusoid in Q and K"),
        Workload("strided_n65536", 1, 8, 65536, 64, strided_heads(8, 256), "bf16", 64, 64, 1005,
                 note="long strided pattern at the audio length 65,536"),
    )
}


def sinusoid(n: int, d: int, period: int = 128, amplitude: float = 0.5) -> torch.Tensor:
    """Shared periodic component a[i, f] = amplitude * sin(2 pi i / period + 2 pi f / d), float32 [n, d]."""
    i = torch.arange(n, dtype=torch.float64)[:, None]
    f = torch.arange(d, dtype=torch.float64)[None, :]
    return (amplitude * torch.sin(2 * math.pi * i / period + 2 * math.pi * f / d)).to(torch.float32)


def torch_dtype(name: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "fp32": torch.float32}[name]


def make_inputs(B: int, H: int, n: int, d: int, seed: int, dtype: str = "bf16",
                with_sinusoid: bool = False) -> dict:
    """Draw Q, K, V, dO (CPU tensors of the requested dtype) from one seeded generator."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    shape = (B, H, n, d)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    do = torch.randn(shape, generator=g, dtype=torch.float32)
    if with_sinusoid:
        a = sinusoid(n, d)
        q += a
        k += a
    t = torch_dtype(dtype)
    return {"q": q.to(t), "k": k.to(t), "v": v.to(t), "do": do.to(t)}


def workload_inputs(w: Workload, seed: int | None = None) -> dict:
    return make_inputs(w.B, w.H, w.n, w.d, w.seed if seed is None else seed, w.dtype, w.sinusoid)
