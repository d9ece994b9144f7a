"""Summaries of rocprofv3 output for the committed profiles.

Two kinds of summary, both short text files:

* kernel statistics: the ``*_kernel_stats.csv`` of a
  ``rocprofv3 --kernel-trace --stats`` run, one line per kernel;
* HBM traffic: two ``--pmc`` runs (``FETCH_SIZE``, then ``WRITE_SIZE``) of a
  command that also runs one plain device-to-device copy of known size.  The
  copy's own counter values give the scale factor of each counter (known
  bytes / counted bytes); every kernel's average per dispatch is scaled by it.
  The file records a hash of the kernel sources, so that a reader can tell
  whether the kernels changed after the counters were taken.

Usage (on the csv files a profiling run wrote):

    python -m factorized_block_sparse_amd.profiling stats <kernel_stats.csv> <out.txt> "<command>"
    python -m factorized_block_sparse_amd.profiling traffic <fetch.csv> <write.csv> <copy MiB> \\
        <out.txt> "<fetch command>" "<write command>"
"""

from __future__ import annotations

import csv
import hashlib
import os
import sys
from collections import defaultdict

_PKG = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_PKG)
SOURCES = ("factorized_block_sparse_amd/csrc/device_common.hpp",
           "factorized_block_sparse_amd/csrc/abi_common.hpp",
           "factorized_block_sparse_amd/csrc/fwd.hip",
           "factorized_block_sparse_amd/csrc/bwd.hip",
           "factorized_block_sparse_amd/csrc/layout.cpp",
           "include/sparse_attn.h")
COPY_KERNEL_MARK = "copyBuffer"  # the runtime's device-to-device copy kernel


def source_hash() -> str:
    """sha256 over the kernel and layout sources (the code the counters describe)."""
    h = hashlib.sha256()
    for rel in SOURCES:
        with open(os.path.join(_ROOT, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read() + b"\0")
    return h.hexdigest()


def write_kernel_stats(src: str, dst: str, command: str) -> str:
    rows = list(csv.DictReader(open(src)))
    lines = ["# rocprofv3 kernel statistics (one MI355X)",
             f"# command: {command}",
             f"# kernel sources sha256: {source_hash()}",
             f"{'kernel':58s} {'calls':>5s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'share%':>7s}"]
    for r in rows:
        lines.append(f"{r['Name'][:58]:58s} {int(r['Calls']):5d} {float(r['AverageNs']) / 1e3:9.2f} "
                     f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f} "
                     f"{float(r['Percentage']):7.2f}")
    text = "\n".join(lines) + "\n"
    with open(dst, "w") as f:
        f.write(text)
    return text


def _per_kernel(path: str) -> dict:
    vals = defaultdict(list)
    for r in csv.DictReader(open(path)):
        vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in vals.items()}


def write_traffic(fetch_csv: str, write_csv: str, copy_mib: int, dst: str, fetch_cmd: str,
                  write_cmd: str) -> str:
    fetch, write = _per_kernel(fetch_csv), _per_kernel(write_csv)
    copy = [k for k in fetch if COPY_KERNEL_MARK in k]
    if not copy or not any(COPY_KERNEL_MARK in k for k in write):
        raise SystemExit("no copy kernel in the counter files: run with --copy-calibration-mib")
    known_kib = copy_mib * 1024.0
    f_scale = known_kib / fetch[copy[0]][0]
    w_scale = known_kib / write[[k for k in write if COPY_KERNEL_MARK in k][0]][0]
    lines = ["# HBM traffic per dispatch from rocprofv3 counters (one MI355X)",
             f"# FETCH_SIZE command: {fetch_cmd}",
             f"# WRITE_SIZE command: {write_cmd}",
             f"# calibration: a {copy_mib} MiB device-to-device copy counts "
             f"{fetch[copy[0]][0]:.1f} KiB fetched and "
             f"{write[[k for k in write if COPY_KERNEL_MARK in k][0]][0]:.1f} KiB written;",
             f"#   scale factors fetch x{f_scale:.4f}, write x{w_scale:.4f} (known / counted)",
             f"# kernel sources sha256: {source_hash()}",
             "# kernel | dispatches | fetch_MB | write_MB  (scaled, per dispatch, 1 MB = 1e6 B)"]
    for k in sorted(fetch, key=lambda x: -fetch[x][0]):
        if COPY_KERNEL_MARK in k or k not in write or "sa::" not in k and "_ZN2sa" not in k:
            continue
        fb = fetch[k][0] * f_scale * 1024
        wb = write[k][0] * w_scale * 1024
        lines.append(f"{k} | {fetch[k][1]} | {fb / 1e6:.3f} | {wb / 1e6:.3f}")
    text = "\n".join(lines) + "\n"
    with open(dst, "w") as f:
        f.write(text)
    return text


def read_traffic(path: str) -> tuple[str | None, dict]:
    """(sources hash recorded, {kernel name: (fetch bytes, write bytes) per dispatch})."""
    recorded, table = None, {}
    if not os.path.exists(path):
        return None, {}
    for line in open(path):
        if line.startswith("# kernel sources sha256:"):
            recorded = line.split(":", 1)[1].strip()
        elif not line.startswith("#") and "|" in line:
            name, _, fmb, wmb = (x.strip() for x in line.split("|"))
            table[name] = (float(fmb) * 1e6, float(wmb) * 1e6)
    return recorded, table


def main(argv: list[str]) -> None:
    if len(argv) >= 4 and argv[0] == "stats":
        print(write_kernel_stats(argv[1], argv[2], argv[3]))
    elif len(argv) >= 7 and argv[0] == "traffic":
        print(write_traffic(argv[1], argv[2], int(argv[3]), argv[4], argv[5], argv[6]))
    else:
        print(__doc__)
        sys.exit(2)


if __name__ == "__main__":
    main(sys.argv[1:])
