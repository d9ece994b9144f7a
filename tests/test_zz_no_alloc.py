"""The allocation-free backward (``sparse_attn_bwd_static``) against the
workspace-taking ``sparse_attn_bwd``, through the C ABI, on two calls in a row:
the second smaller, so it runs over what the first left in the library's
static device array.  Both layouts split key and query tiles, so the chunk
partials that live in that array carry results."""

import pytest
import torch

from factorized_block_sparse_amd import binding as bd
from factorized_block_sparse_amd import workloads as W
from factorized_block_sparse_amd.binding import HeadPattern, Layout
from tests.parity_util import BF16_MAX_ABS, BF16_REL_RMS, assert_close, to64

pytestmark = pytest.mark.gpu

CALLS = [
    # (B, n, heads, split_keys, split_rows, seed)
    (2, 4096, [HeadPattern("sameblock", 128), HeadPattern("summary", 128, 32, 0),
               HeadPattern("local", 300), HeadPattern("stride", 64)], 512, 256, 71),
    (1, 1000, [HeadPattern("summary", 64, 16, 1), HeadPattern("local", 900)], 256, 128, 72),
]


def test_static_backward_matches_workspace_backward_twice():
    dev = torch.device("cuda:0")
    for B, n, heads, sk, sr, seed in CALLS:
        lay = Layout(n, heads, 64, 64, split_keys=sk, split_rows=sr)
        assert lay.header.num_slots > 0 and lay.header.num_qslots > 0
        assert bd.bwd_workspace_bytes(lay, B, len(heads)) <= bd.SA_STATIC_SCRATCH_BYTES
        inp = W.make_inputs(B, len(heads), n, 64, seed=seed)
        q, k, v, do = (inp[x].to(dev) for x in ("q", "k", "v", "do"))
        o, lse = bd.sparse_attn_fwd(lay, q, k, v)
        ref = bd.sparse_attn_bwd(lay, q, k, v, o, lse, do)
        got = bd.sparse_attn_bwd_static(lay, q, k, v, o, lse, do)
        torch.cuda.synchronize()
        for nm, g, r in zip(("dq", "dk", "dv"), got, ref):
            g64, r64 = to64(g), to64(r)
            for b in range(B):
                for h in range(len(heads)):
                    assert_close(f"{nm} n={n} b{b} h{h}", g64[b, h], r64[b, h], BF16_MAX_ABS,
                                 BF16_REL_RMS, bf16_output=True)
            # both entry points run the same deterministic kernels
            assert torch.equal(g, r), nm


def test_static_backward_refuses_sizes_past_the_array():
    """D alone of this call needs more than the static array: SA_ESIZE, nothing launched."""
    dev = torch.device("cuda:0")
    heads = [HeadPattern("local", 8), HeadPattern("stride", 8)]
    n = 4096
    B = bd.SA_STATIC_SCRATCH_BYTES // (len(heads) * n * 4) + 1
    lay = Layout(n, heads, 64, 64)
    assert bd.bwd_workspace_bytes(lay, B, 2) > bd.SA_STATIC_SCRATCH_BYTES
    x = torch.zeros((B, 2, n, 64), dtype=torch.bfloat16, device=dev)
    lse = torch.zeros((B, 2, n), dtype=torch.float32, device=dev)
    with pytest.raises(bd.SparseAttnError, match="static array"):
        bd.sparse_attn_bwd_static(lay, x, x, x, x, lse, x)
    torch.cuda.synchronize()
