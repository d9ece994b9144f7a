"""Measured ceilings of the GPU the benchmark runs on (ctypes binding of
``include/sa_probes.h``): back-to-back bf16 MFMA rate and the shader clock
under that load, VALU FMA and exp rates, LDS read instruction rates, and
fp32 atomic-add against plain-store throughput.  The library
``libsa_probes.so`` is built beside the attention library."""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libsa_probes.so"
FIELDS = ("mfma_bf16_tflops", "shader_clock_ghz", "mfma_cycles", "fma_cycles", "exp_cycles",
          "lds_b128_cycles", "lds_tr_b64_cycles", "atomic_f32_tbs", "store_f32_tbs")


class ProbeResults(ctypes.Structure):
    _fields_ = [(f, ctypes.c_double) for f in FIELDS]


def run() -> dict:
    """Run the probes on the current device; raises if the library is missing or a HIP call fails."""
    path = os.path.join(_PKG, LIB_NAME)
    if not os.path.exists(path):
        raise RuntimeError(f"{LIB_NAME} is not built ({path})")
    lib = ctypes.CDLL(path)
    lib.sa_probe_run.argtypes = [ctypes.POINTER(ProbeResults)]
    lib.sa_probe_run.restype = ctypes.c_int
    r = ProbeResults()
    rc = lib.sa_probe_run(ctypes.byref(r))
    if rc != 0:
        raise RuntimeError(f"sa_probe_run failed with status {rc}")
    return {f: round(getattr(r, f), 3) for f in FIELDS}


if __name__ == "__main__":
    import json
    print(json.dumps(run()))
