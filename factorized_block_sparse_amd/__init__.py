"""Causal factorized block-sparse self-attention for AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library ``libsparse_attn.so`` (hand-written HIP
kernels plus a host layout builder); ``binding`` is a thin ctypes layer over
it that only marshals arguments.  Importing this package does not load the
library; the first call does, and raises if the library has not been built.
"""

from . import workloads  # noqa: F401
from .binding import (  # noqa: F401
    Layout, HeadPattern, sparse_attn_layout, sparse_attn_fwd, sparse_attn_bwd,
    library_path, load_library,
)
