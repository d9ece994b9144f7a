"""CPU oracle for causal factorized (block-sparse) self-attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, tables or
helpers with the HIP library under ``factorized_block_sparse_amd/``.

Everything here is plain numpy in float64, written from the pages' own
definitions:

* ``masks``      token-level visibility sets of every head kind (strided:
                 local band + stride; fixed: same-block + summary columns;
                 plus the local + global-token worked example), in a dense
                 ``[n, n]`` form and a per-row form.
* ``attention``  masked softmax attention forward and backward (the
                 recomputation form of the backward), in a dense-mask mode
                 and a row-gather mode.

Sources (cited by page title and section):

* "Sparse Transformers 深度解读报告" (Generating Long Sequences with Sparse
  Transformers, deep-dive report), section 2.1 (factorized self-attention),
  section 2.2 (strided and fixed patterns), section 3.4 (recomputation),
  section 3.5 (block-sparse kernels).
* "长序列为何不必让每个 token 看见全部历史？滑动窗口、块稀疏与全局 token",
  section 02 (masked softmax over an adjacency matrix), section 03 (causal
  sliding window), section 04 (8-token worked example), section 07 (dense
  truth mask), section 10 (verification recipe), section 15 (exercise).
* "【Transformer 与注意力机制】43｜稀疏与局部注意力", section 2 (Sparse
  Transformer: grid/column view of the stride head, two-hop reachability).

Parity status: every function is pinned by a ``-m "not gpu"`` test against a
printed example, a closed form, an invariant, a library routine on a special
case, or brute force; see ``tests/test_oracle_*.py``.  One reading is
"parity unpinned" beyond its printed special case: the choice of summary
sub-block for the k-th summary head (only k = 0 is printed).
"""

from . import masks, attention  # noqa: F401
