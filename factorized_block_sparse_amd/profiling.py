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

* shader counters: one ``--pmc`` run of SQ counters (MFMA busy cycles, LDS
  bank conflicts, wait cycles), averaged per dispatch, with the ratios
  derived from them.

Usage (on the csv files a profiling run wrote; ``--log <stdout of the
profiled run>`` records the kernel-source hash that run's bench line printed,
otherwise the hash of the sources here):

    python -m factorized_block_sparse_amd.profiling stats <kernel_stats.csv> <out.txt> "<command>"
    python -m factorized_block_sparse_amd.profiling traffic <fetch.csv> <write.csv> <copy MiB> \\
        <out.txt> "<fetch command>" "<write command>" [<kernel_stats.csv>]
    python -m factorized_block_sparse_amd.profiling counters <counters.csv> <out.txt> "<command>"
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


def code_text(src: str) -> str:
    """C/C++ source without comments and with runs of whitespace collapsed: what
    the compiler sees of it (the sources hold no comment markers inside string
    literals)."""
    out, i, n = [], 0, len(src)
    while i < n:
        if src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        else:
            out.append(src[i])
            i += 1
    return " ".join("".join(out).split())


def source_hash() -> str:
    """sha256 over the code of the kernel and layout sources (the code the
    counters describe; comments and layout of the text do not count)."""
    h = hashlib.sha256()
    for rel in SOURCES:
        with open(os.path.join(_ROOT, rel), encoding="utf-8") as f:
            h.update(rel.encode() + b"\0" + code_text(f.read()).encode() + b"\0")
    return h.hexdigest()


def run_hash(log: str | None) -> str:
    """The kernel-source hash of the profiled run: read from the bench line in
    its log (bench.py prints it); without a log, the hash of the sources here."""
    if log:
        import json
        for line in open(log, errors="replace"):
            if line.startswith("{") and "kernel_sources_sha256" in line:
                return json.loads(line)["kernel_sources_sha256"]
        raise SystemExit(f"no bench line with kernel_sources_sha256 in {log}")
    return source_hash()


def write_kernel_stats(src: str, dst: str, command: str, log: str | None = None) -> str:
    rows = list(csv.DictReader(open(src)))
    lines = ["# rocprofv3 kernel statistics (one MI355X)",
             f"# command: {command}",
             f"# kernel sources sha256: {run_hash(log)}",
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


def _first_copy(path: str) -> float:
    """Counter value of the first dispatch of the copy kernel: the calibration
    copy, which runs before anything else copies (later copies, of other sizes,
    use the same kernel)."""
    hits = [(int(r["Dispatch_Id"]), float(r["Counter_Value"])) for r in csv.DictReader(open(path))
            if COPY_KERNEL_MARK in r["Kernel_Name"]]
    if not hits:
        raise SystemExit("no copy kernel in the counter files: run with --copy-calibration-mib")
    return min(hits)[1]


def _avg_durations_us(stats_csv: str | None) -> dict:
    if not stats_csv:
        return {}
    return {r["Name"]: float(r["AverageNs"]) / 1e3 for r in csv.DictReader(open(stats_csv))}


def write_traffic(fetch_csv: str, write_csv: str, copy_mib: int, dst: str, fetch_cmd: str,
                  write_cmd: str, stats_csv: str | None = None, log: str | None = None) -> str:
    """Per-dispatch HBM bytes; with the kernel statistics of a kernel-trace run
    of the same command, also the achieved HBM rate (bytes / average duration)."""
    fetch, write = _per_kernel(fetch_csv), _per_kernel(write_csv)
    dur = _avg_durations_us(stats_csv)
    copy_f, copy_w = _first_copy(fetch_csv), _first_copy(write_csv)
    known_kib = copy_mib * 1024.0
    f_scale = known_kib / copy_f
    w_scale = known_kib / copy_w
    lines = ["# HBM traffic per dispatch from rocprofv3 counters (one MI355X)",
             f"# FETCH_SIZE command: {fetch_cmd}",
             f"# WRITE_SIZE command: {write_cmd}",
             f"# calibration: the first dispatch of the copy kernel (a {copy_mib} MiB device-to-device "
             f"copy) counts {copy_f:.1f} KiB fetched and {copy_w:.1f} KiB written;",
             f"#   scale factors fetch x{f_scale:.4f}, write x{w_scale:.4f} (known / counted)",
             f"# kernel sources sha256: {run_hash(log)}",
             "# kernel | dispatches | fetch_MB | write_MB | achieved_GB/s  (scaled, per dispatch, "
             "1 MB = 1e6 B; GB/s = (fetch + write) / kernel-trace average duration, - if none)"]
    for k in sorted(fetch, key=lambda x: -fetch[x][0]):
        if COPY_KERNEL_MARK in k or k not in write or "sa::" not in k and "_ZN2sa" not in k:
            continue
        fb = fetch[k][0] * f_scale * 1024
        wb = write[k][0] * w_scale * 1024
        rate = f"{(fb + wb) / (dur[k] * 1e-6) / 1e9:.0f}" if k in dur else "-"
        lines.append(f"{k} | {fetch[k][1]} | {fb / 1e6:.3f} | {wb / 1e6:.3f} | {rate}")
    text = "\n".join(lines) + "\n"
    with open(dst, "w") as f:
        f.write(text)
    return text


SIMDS_PER_XCD = 128  # 32 CUs x 4 SIMDs in each of the 8 XCDs


def _per_kernel_counters(path: str) -> dict:
    vals = defaultdict(lambda: defaultdict(list))
    for r in csv.DictReader(open(path)):
        vals[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return {k: {c: (sum(v) / len(v), len(v)) for c, v in d.items()} for k, d in vals.items()}


def write_counters(src: str, dst: str, command: str, log: str | None = None) -> str:
    """Per-dispatch averages of SQ counters and three ratios:
    mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (128 x GRBM_GUI_ACTIVE), the share
    of SIMD cycles the matrix units were busy.  GRBM_GUI_ACTIVE reads about 8x
    the dispatch's duration in shader cycles here (one count per XCD), so
    128 x GRBM_GUI_ACTIVE is the SIMD-cycles of all 1,024 SIMDs; a 32x32x16
    bf16 MFMA adds 32 busy cycles (SQ_VALU_MFMA_BUSY_CYCLES = 32 x SQ_INSTS_MFMA
    in these files).
    lds_conflict = SQ_LDS_BANK_CONFLICT / SQ_INSTS_LDS, bank-conflict cycles
    per LDS instruction.
    wait = SQ_WAIT_ANY / SQ_WAVE_CYCLES, the share of wave lifetime spent
    waiting on a dependency (s_waitcnt)."""
    table = _per_kernel_counters(src)
    names = sorted({c for d in table.values() for c in d})
    lines = ["# rocprofv3 shader counters per dispatch (one MI355X)",
             f"# command: {command}",
             f"# kernel sources sha256: {run_hash(log)}",
             "# mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (128 SIMDs per XCD x GRBM_GUI_ACTIVE, "
             "which counts once per XCD); lds_conflict = SQ_LDS_BANK_CONFLICT / SQ_INSTS_LDS; "
             "wait = SQ_WAIT_ANY / SQ_WAVE_CYCLES",
             "# kernel | dispatches | mfma_busy | lds_conflict | wait | " + " | ".join(names)]
    for k in sorted(table):
        if "sa::" not in k and "_ZN2sa" not in k:
            continue
        d = table[k]
        g = lambda c: d[c][0] if c in d else float("nan")
        div = lambda a, b: a / b if b else float("nan")
        busy = div(g("SQ_VALU_MFMA_BUSY_CYCLES"), SIMDS_PER_XCD * g("GRBM_GUI_ACTIVE"))
        conf = div(g("SQ_LDS_BANK_CONFLICT"), g("SQ_INSTS_LDS"))
        wait = div(g("SQ_WAIT_ANY"), g("SQ_WAVE_CYCLES"))
        n = max(v[1] for v in d.values())
        lines.append(f"{k} | {n} | {busy:.3f} | {conf:.3f} | {wait:.3f} | "
                     + " | ".join(f"{g(c):.4g}" for c in names))
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
            name, _, fmb, wmb = (x.strip() for x in line.split("|")[:4])
            table[name] = (float(fmb) * 1e6, float(wmb) * 1e6)
    return recorded, table


def main(argv: list[str]) -> None:
    log = None
    if "--log" in argv:  # the profiled run's stdout: the hash is taken from its bench line
        i = argv.index("--log")
        log = argv[i + 1]
        argv = argv[:i] + argv[i + 2:]
    if len(argv) >= 4 and argv[0] == "stats":
        print(write_kernel_stats(argv[1], argv[2], argv[3], log))
    elif len(argv) >= 4 and argv[0] == "counters":
        print(write_counters(argv[1], argv[2], argv[3], log))
    elif len(argv) >= 7 and argv[0] == "traffic":
        print(write_traffic(argv[1], argv[2], int(argv[3]), argv[4], argv[5], argv[6],
                            argv[7] if len(argv) > 7 else None, log))
    else:
        print(__doc__)
        sys.exit(2)


if __name__ == "__main__":
    main(sys.argv[1:])
