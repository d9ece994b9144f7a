"""Build the C-ABI library ``libsparse_attn.so`` in-tree with hipcc for gfx950.

Usage: ``python -m factorized_block_sparse_amd.build`` (or ``build()`` from
Python).  Compiles every source under ``csrc/`` (host C++ and HIP) into one
shared library next to this file.  It always recompiles.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ_DIR = os.path.join(PKG, "_build")
LIB_NAME = "libsparse_attn.so"
ARCH = "gfx950"

SOURCES = ["layout.cpp", "fwd.hip", "bwd.hip"]
# Calibration micro-benchmarks (include/sa_probes.h), a library of their own:
# the benchmark reads the measured ceilings from it; the attention path does not.
PROBE_SOURCES = ["probes.hip"]
PROBE_LIB_NAME = "libsa_probes.so"

# Packed FP32 VALU ops are disabled for all device code: the kernels rely on
# ordinary scalar float arithmetic only.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics", "-Wall", "-Wno-unused-function",
    # MFMA accumulators in ordinary VGPRs: the softmax rescales and the
    # epilogues touch them with VALU code, which AGPRs would force through
    # copies.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in (res.stderr or "").splitlines() if noise not in line)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    return obj


def _link(objs, name: str) -> str:
    out = os.path.join(PKG, name)
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stderr}")
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Compile all sources and link the attention library (returns its path)
    and the calibration library beside it."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose), srcs)))
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB_NAME)
    return _link([objs[s] for s in SOURCES], LIB_NAME)


if __name__ == "__main__":
    print(build(verbose=True))
