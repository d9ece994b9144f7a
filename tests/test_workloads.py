"""The seeded input recipe: determinism, shapes, and the shared sinusoid's closed form."""

import math

import numpy as np
import torch

from factorized_block_sparse_amd import workloads as W


def test_inputs_are_seeded_and_shaped():
    a = W.make_inputs(1, 2, 64, 64, seed=7)
    b = W.make_inputs(1, 2, 64, 64, seed=7)
    for key in ("q", "k", "v", "do"):
        assert a[key].shape == (1, 2, 64, 64) and a[key].dtype == torch.bfloat16
        assert torch.equal(a[key], b[key])
    c = W.make_inputs(1, 2, 64, 64, seed=8)
    assert not torch.equal(a["q"], c["q"])


def test_sinusoid_logit_closed_form():
    """Shared component a[i, f] = 0.5 sin(2 pi i / 128 + 2 pi f / 64) in both Q and K.

    sum_f a[i, f] a[j, f] = 0.25 * (64 / 2) cos(2 pi (i - j) / 128), so after the
    1/sqrt(64) scale the expected logit is cos(2 pi (i - j) / 128).
    """
    a = W.sinusoid(300, 64).double().numpy()
    s = (a @ a.T) / 8.0
    i = np.arange(300)
    expect = np.cos(2 * math.pi * (i[:, None] - i[None, :]) / 128)
    np.testing.assert_allclose(s, expect, atol=1e-6)


def test_workload_head_assignment():
    w = W.WORKLOADS["fixed_n12288"]
    kinds = [(h.kind, h.sub) for h in w.heads]
    assert kinds == [("sameblock", 0), ("summary", 0), ("sameblock", 0), ("summary", 1),
                     ("sameblock", 0), ("summary", 2), ("sameblock", 0), ("summary", 3)]
    w = W.WORKLOADS["strided_n12288"]
    assert w.sinusoid and [h.kind for h in w.heads[:2]] == ["local", "stride"]
