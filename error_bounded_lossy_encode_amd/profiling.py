"""Turn rocprofv3 output into the short text summaries kept under profiles/, and read them back.

Two kinds of summary:

* kernel-trace statistics (``rocprofv3 --kernel-trace --stats``, rocpd database): count and
  average / min / max duration per codec kernel;
* HBM traffic per kernel launch from two counter runs (``--pmc FETCH_SIZE`` and ``--pmc
  WRITE_SIZE``, KiB per dispatch).  Each counter is scaled by what it reads for a plain device
  copy of known size run in the same process, so the traffic is in true bytes.

A traffic summary records the SHA-256 of the kernel sources it was measured on; the benchmark
uses it only while they are unchanged.
"""
from __future__ import annotations

import csv
import hashlib
import os
import re
import sqlite3
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = [os.path.join(HERE, "csrc", f) for f in
                  ("eblc_internal.h", "eblc_device.h", "eblc_kernels.hip", "eblc_chunk.hip")]
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def kernel_source_sha256() -> str:
    """One digest over every file the kernels are compiled from, in a fixed order."""
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def short_name(full: str) -> str:
    m = re.search(r"(\w+_kernel)\b", full)
    if m:
        return m.group(1)
    return full.split("(")[0].strip()


def trace_stats(db_path: str, pattern: str = "eblc"):
    """{kernel: (count, avg_us, min_us, max_us)} from a rocpd database."""
    con = sqlite3.connect(db_path)
    rows = con.execute("select name, count(*), avg(end-start), min(end-start), max(end-start) "
                       "from kernels group by name").fetchall()
    out = {}
    for name, cnt, avg, mn, mx in rows:
        if re.search(pattern, name):
            out[short_name(name)] = (int(cnt), avg / 1e3, mn / 1e3, mx / 1e3)
    return out


def counter_values(csv_path: str, counter: str):
    """{kernel: [value per dispatch]} for one counter of a rocprofv3 --pmc CSV."""
    vals = defaultdict(list)
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            key = COPY_KERNEL if COPY_KERNEL in name else short_name(name)
            vals[key].append((float(r["Counter_Value"]), int(r["Grid_Size"])))
    return vals


def copy_scale(vals, copy_bytes: int, counter: str) -> float:
    """Counter KiB per true KiB, from the largest plain copy in the run."""
    if COPY_KERNEL not in vals:
        raise ValueError(f"no {COPY_KERNEL} dispatch in the {counter} run")
    measured = max(v for v, _ in vals[COPY_KERNEL])
    return measured * 1024.0 / copy_bytes


def traffic_summary(fetch_csv: str, write_csv: str, copy_bytes: int, kernels, command: str,
                    workload: str) -> str:
    """Text summary of scaled FETCH_SIZE / WRITE_SIZE bytes per launch for `kernels`."""
    fv = counter_values(fetch_csv, "FETCH_SIZE")
    wv = counter_values(write_csv, "WRITE_SIZE")
    # a copy reads copy_bytes and writes copy_bytes
    f_scale = copy_scale(fv, copy_bytes, "FETCH_SIZE")
    w_scale = copy_scale(wv, copy_bytes, "WRITE_SIZE")
    lines = [
        f"# HBM traffic per launch, {workload}",
        f"command: {command}",
        f"kernel_source_sha256: {kernel_source_sha256()}",
        f"copy_bytes: {copy_bytes}",
        f"fetch_scale: {f_scale:.6f}   (FETCH_SIZE KiB of the {copy_bytes} B copy / true KiB)",
        f"write_scale: {w_scale:.6f}   (WRITE_SIZE KiB of the same copy / true KiB)",
        "kernel dispatches fetch_KiB_raw write_KiB_raw fetch_bytes write_bytes traffic_bytes",
    ]
    for k in kernels:
        if k not in fv or k not in wv:
            continue
        f = sum(v for v, _ in fv[k]) / len(fv[k])
        w = sum(v for v, _ in wv[k]) / len(wv[k])
        fb = f * 1024.0 / f_scale
        wb = w * 1024.0 / w_scale
        lines.append(f"{k} {len(fv[k])} {f:.1f} {w:.1f} {fb:.0f} {wb:.0f} {fb + wb:.0f}")
    return "\n".join(lines) + "\n"


def read_traffic(path: str):
    """{kernel: traffic bytes per launch} from a traffic summary, or None when the file is
    missing or was measured on a different kernel source."""
    if not os.path.exists(path):
        return None
    text = open(path).read().splitlines()
    sha = None
    out = {}
    in_table = False
    for line in text:
        if line.startswith("kernel_source_sha256:"):
            sha = line.split(":", 1)[1].strip()
        elif line.startswith("kernel dispatches"):
            in_table = True
        elif in_table and line.strip():
            parts = line.split()
            out[parts[0]] = float(parts[-1])
    if sha != kernel_source_sha256():
        return None
    return out


def trace_summary(db_path: str, command: str, workload: str, pattern: str = "eblc") -> str:
    stats = trace_stats(db_path, pattern)
    lines = [f"# rocprofv3 --kernel-trace --stats, {workload}",
             f"command: {command}",
             f"kernel_source_sha256: {kernel_source_sha256()}",
             "kernel calls avg_us min_us max_us"]
    for k, (cnt, avg, mn, mx) in sorted(stats.items(), key=lambda kv: -kv[1][0] * kv[1][1]):
        lines.append(f"{k} {cnt} {avg:.2f} {mn:.2f} {mx:.2f}")
    return "\n".join(lines) + "\n"
