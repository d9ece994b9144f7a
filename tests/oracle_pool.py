"""The oracle over every row of full-size workloads, on a pool of host processes.

Test helper.  Each task runs the float64 row-gather oracle (forward and
backward) over all rows of one (batch, head) and returns O, LSE, dQ, dK, dV
and which keys any row reads.  Workers are spawned (never forked from a
process that has used the GPU) and run one BLAS thread each; the pool holds
at most 16 of them.
"""

from __future__ import annotations

import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np


def _one_blas_thread():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # threading only affects speed
        pass


def head_task(kind, n, l, c, sub, q, k, v, do):
    """Oracle forward + backward over every row of one head: (O, LSE, dQ, dK, dV, read)."""
    from oracle import attention as OA
    kf = OA.keys_fn_for(kind, n, l, c, sub)
    o, lse = OA.fwd_rows(q, k, v, kf)
    dq, dk, dv = OA.bwd_rows_full(q, k, v, do, kf)
    read = np.zeros(n, dtype=bool)
    for i in range(n):
        read[kf(i)] = True
    return o, lse, dq, dk, dv, read


def make_pool(workers: int | None = None) -> ProcessPoolExecutor:
    workers = workers or min(16, os.cpu_count() or 1)
    return ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn"),
                               initializer=_one_blas_thread)
