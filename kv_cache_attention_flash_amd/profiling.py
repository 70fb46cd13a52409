"""Summaries of rocprofv3 output for the library's kernels.

    python -m kv_cache_attention_flash_amd.profiling stats  <kernel_stats.csv> <out.md> <command...>
    python -m kv_cache_attention_flash_amd.profiling stats-db <results.db> <out.md> <command...>
    python -m kv_cache_attention_flash_amd.profiling traffic <fetch_counter.csv> <write_counter.csv> \
        <out.json> <kernel-substrings> <calibration-bytes> <source-file> <command...>

``stats`` writes a Markdown table of per-kernel call counts and durations
(from the ``--output-format csv`` statistics file); ``stats-db`` makes the same
table from the SQLite database rocprofv3 writes by default.
``traffic`` turns two counter runs (FETCH_SIZE, then WRITE_SIZE, KiB per
dispatch) into HBM bytes per call of one library entry point: the sum over
its kernels (comma-separated name substrings) of each kernel's median.  Each counter is scaled by
what it reads for the plain device-to-device copy of ``calibration-bytes``
bytes that ran in the same process (the ``copyBuffer`` dispatch of that size):
on gfx950 FETCH_SIZE reads half of the bytes a copy actually fetches.  The
JSON records the sha256 prefix of the kernel's source file so that a later
change to the kernel invalidates the figure.
"""

from __future__ import annotations

import csv
import hashlib
import json
import os
import re
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))


def short_name(name: str) -> str:
    m = re.search(r"(?:\w+::)*(\w+)(?:<[^()]*>)?\(", name)
    return m.group(1) if m else name[:60]


def kernel_stats_markdown(stats_csv: str, command: str) -> str:
    rows = list(csv.DictReader(open(stats_csv)))
    out = ["| kernel | calls | average (us) | min (us) | max (us) | share |",
           "|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| `{short_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                   f"{float(r['Percentage']):.1f}% |")
    return f"Command: `{command}`\n\n" + "\n".join(out) + "\n"


def kernel_stats_markdown_db(db_path: str, command: str) -> str:
    import sqlite3
    con = sqlite3.connect(db_path)
    rows = list(con.execute("select name, count(*), avg(end - start), min(end - start), "
                            "max(end - start), sum(end - start) from kernels group by name "
                            "order by sum(end - start) desc"))
    total = sum(r[5] for r in rows) or 1
    out = ["| kernel | calls | average (us) | min (us) | max (us) | share |",
           "|---|---|---|---|---|---|"]
    for name, n, avg, mn, mx, tot in rows:
        out.append(f"| `{short_name(name)}` | {n} | {avg / 1e3:.2f} | {mn / 1e3:.2f} | "
                   f"{mx / 1e3:.2f} | {100.0 * tot / total:.1f}% |")
    return f"Command: `{command}`\n\n" + "\n".join(out) + "\n"


def _per_dispatch(counter_csv: str, counter: str):
    vals = {}
    for r in csv.DictReader(open(counter_csv)):
        if r["Counter_Name"] != counter:
            continue
        vals.setdefault((r["Kernel_Name"], r.get("Grid_Size", "")), []).append(float(r["Counter_Value"]))
    return vals


def _calibration(vals, grid_hint=None):
    """KiB the counter reported for the largest copyBuffer dispatch."""
    best = None
    for (name, grid), v in vals.items():
        if "copyBuffer" in name:
            m = statistics.median(v)
            if best is None or m > best:
                best = m
    return best


def traffic(fetch_csv, write_csv, kernel_substrs, calib_bytes, source_file):
    fv = _per_dispatch(fetch_csv, "FETCH_SIZE")
    wv = _per_dispatch(write_csv, "WRITE_SIZE")
    cf, cw = _calibration(fv), _calibration(wv)
    if not cf or not cw:
        raise SystemExit("no copy calibration dispatch found")
    scale_f = calib_bytes / (cf * 1024.0)
    scale_w = calib_bytes / (cw * 1024.0)
    per_kernel = {}
    for ks in kernel_substrs.split(","):
        kf = [x for (n, _), v in fv.items() if ks in n for x in v]
        kw = [x for (n, _), v in wv.items() if ks in n for x in v]
        if not kf or not kw:
            raise SystemExit(f"no dispatch of a kernel matching {ks!r}")
        per_kernel[ks] = {"dispatches": [len(kf), len(kw)],
                          "fetch_size_kib_median": statistics.median(kf),
                          "write_size_kib_median": statistics.median(kw),
                          "fetch_bytes": statistics.median(kf) * 1024.0 * scale_f,
                          "write_bytes": statistics.median(kw) * 1024.0 * scale_w}
    fetch_b = sum(k["fetch_bytes"] for k in per_kernel.values())
    write_b = sum(k["write_bytes"] for k in per_kernel.values())
    with open(source_file, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()[:16]
    return {"kernels": per_kernel,
            "copy_calibration_bytes": calib_bytes, "copy_fetch_kib": cf, "copy_write_kib": cw,
            "fetch_scale": scale_f, "write_scale": scale_w,
            "fetch_bytes_per_launch": fetch_b, "write_bytes_per_launch": write_b,
            "bytes_per_launch": fetch_b + write_b,
            "kernel_source": os.path.relpath(source_file, os.path.dirname(HERE)),
            "kernel_source_sha256_16": sha}


def main(argv):
    if argv[0] in ("stats", "stats-db"):
        fn = kernel_stats_markdown if argv[0] == "stats" else kernel_stats_markdown_db
        md = fn(argv[1], " ".join(argv[3:]))
        with open(argv[2], "w") as f:
            f.write(md)
        print(md)
    elif argv[0] == "traffic":
        fetch_csv, write_csv, out, kernels, calib, source = argv[1:7]
        t = traffic(fetch_csv, write_csv, kernels, float(calib), source)
        t["commands"] = " ".join(argv[7:])
        with open(out, "w") as f:
            json.dump(t, f, indent=1)
        print(json.dumps(t, indent=1))
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
