"""Turns rocprofv3 CSV output into the short text/JSON summaries kept under profiles/.

  python rocprof_summary.py stats DIR --cmd "..." > summary.txt
      per-kernel dispatch count and mean/min/max duration from DIR's *_kernel_stats.csv.

  python rocprof_summary.py traffic --fetch DIR1 --write DIR2 \
      --kernel NAME --copy-bytes B --cmd-fetch "..." --cmd-write "..." > traffic.json
      HBM bytes per dispatch of kernel NAME from a FETCH_SIZE pass and a WRITE_SIZE pass
      (KiB per dispatch), each scaled by what the same counter reads for the plain
      device-to-device copy of B bytes (the runtime's copyBuffer kernel) in the same
      pass: factor = B / counter bytes of the copy.

  python rocprof_summary.py counters DIR [DIR ...] \
      --kernel NAME --cmd "..." --title "..." > counters.txt
      mean per dispatch of every counter that the --pmc passes in the DIRs collected for
      kernel NAME (rows of one dispatch summed), with the pass's command.

  python rocprof_summary.py gaps DIR --cmd "..." [--labels a,b,c] > gaps.txt
      from DIR's *_kernel_trace.csv: the dispatches in start order, split into phases at
      each spin kernel (the head start the benchmark queues before a timed loop); per
      phase the median duration of each kernel and the median and 90th-percentile idle
      gap between consecutive kernels, by the pair (previous kernel -> next kernel).

The `stats` and `counters` summaries take --source FILE to record the kernel source's
sha256 prefix they were taken on.

Reads only CSV files (and --source); runs nothing.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import statistics
import sys

COPY_KERNEL = "copyBuffer"


def _find(d, suffix):
    out = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not out:
        raise SystemExit(f"no *{suffix} under {d}")
    return out


def short_name(name):
    name = name.replace("(anonymous namespace)::", "")
    cut = name.find("(")
    if cut > 0:
        name = name[:cut]
    return name.replace("void ", "")


def kernel_stats(d):
    rows = []
    for f in _find(d, "_kernel_stats.csv"):
        for r in csv.DictReader(open(f)):
            rows.append(dict(name=short_name(r["Name"]), calls=int(r["Calls"]),
                             avg_us=float(r["AverageNs"]) / 1e3, min_us=float(r["MinNs"]) / 1e3,
                             max_us=float(r["MaxNs"]) / 1e3, pct=float(r["Percentage"])))
    return rows


def counter_per_dispatch(d, counter):
    """{kernel short name: [value per dispatch]} for one counter (rows of one dispatch summed)."""
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    for f in _find(d, "_counter_collection.csv"):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            per[short_name(r["Kernel_Name"])][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {k: list(v.values()) for k, v in per.items()}


def _pick(table, kernel):
    hits = [k for k in table if kernel in k]
    if len(hits) != 1:
        raise SystemExit(f"kernel {kernel!r} matches {hits} in {sorted(table)}")
    return table[hits[0]]


def cmd_stats(a):
    rows = kernel_stats(a.dir)
    print(f"# rocprofv3 kernel-trace summary: {a.title}{source_note(a.source)}")
    print(f"# command: {a.cmd}")
    print("#")
    print(f"{'kernel':60s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'time%':>6s}")
    for r in sorted(rows, key=lambda r: -r["pct"]):
        print(f"{r['name'][:60]:60s} {r['calls']:6d} {r['avg_us']:9.3f} {r['min_us']:9.3f} "
              f"{r['max_us']:9.3f} {r['pct']:6.2f}")


def cmd_traffic(a):
    fetch = counter_per_dispatch(a.fetch, "FETCH_SIZE")
    write = counter_per_dispatch(a.write, "WRITE_SIZE")
    kf, kw = _pick(fetch, a.kernel), _pick(write, a.kernel)
    cf, cw = _pick(fetch, COPY_KERNEL), _pick(write, COPY_KERNEL)
    # the largest copy dispatch is the calibration copy of --copy-bytes
    ff = a.copy_bytes / (max(cf) * 1024.0)
    fw = a.copy_bytes / (max(cw) * 1024.0)
    f_kib, w_kib = statistics.mean(kf), statistics.mean(kw)
    src_hash = None
    if a.source:
        with open(a.source, "rb") as f:
            src_hash = hashlib.sha256(f.read()).hexdigest()[:16]
    out = {
        "kernel": a.kernel,
        "workload": a.workload,
        "dispatches": [len(kf), len(kw)],
        "fetch_kib_per_dispatch_raw": round(f_kib, 2),
        "write_kib_per_dispatch_raw": round(w_kib, 2),
        "copy_bytes": a.copy_bytes,
        "copy_fetch_kib_raw": round(max(cf), 2),
        "copy_write_kib_raw": round(max(cw), 2),
        "fetch_scale": round(ff, 4),
        "write_scale": round(fw, 4),
        "hbm_read_bytes_per_launch": round(f_kib * 1024.0 * ff),
        "hbm_write_bytes_per_launch": round(w_kib * 1024.0 * fw),
        "hbm_bytes_per_launch": round(f_kib * 1024.0 * ff + w_kib * 1024.0 * fw),
        "source": os.path.basename(a.source) if a.source else None,
        "source_sha256_16": src_hash,
        "command_fetch": a.cmd_fetch,
        "command_write": a.cmd_write,
    }
    if a.algorithmic_bytes:
        out["algorithmic_bytes"] = a.algorithmic_bytes
        out["traffic_over_algorithmic"] = round(out["hbm_bytes_per_launch"] / a.algorithmic_bytes, 3)
    json.dump(out, sys.stdout, indent=1)
    print()


def source_note(path):
    if not path:
        return ""
    with open(path, "rb") as f:
        return f"; source {os.path.basename(path)} sha256/16 {hashlib.sha256(f.read()).hexdigest()[:16]}"


def _pct(vals, q):
    v = sorted(vals)
    return v[min(len(v) - 1, int(round(q * (len(v) - 1))))]


def cmd_gaps(a):
    rows = []
    for f in _find(a.dir, "_kernel_trace.csv"):
        for r in csv.DictReader(open(f)):
            rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), short_name(r["Kernel_Name"])))
    rows.sort()
    labels = a.labels.split(",") if a.labels else []
    print(f"# rocprofv3 kernel-trace gaps: {a.title}")
    print(f"# command: {a.cmd}")
    print("# phases split at the spin kernels; durations and idle gaps (next start - previous end) in us")
    phases, cur = [], []
    for r in rows:
        if a.split in r[2]:
            phases.append(cur)
            cur = []
        else:
            cur.append(r)
    phases.append(cur)
    timed = [ph for ph in phases[1:] if len(ph) >= a.min]
    for i, ph in enumerate(timed):
        name = labels[i] if i < len(labels) else f"phase {i}"
        span = (ph[-1][1] - ph[0][0]) / 1e3
        print(f"## {name}: {len(ph)} dispatches over {span:.1f} us")
        durs = collections.defaultdict(list)
        for st, en, n in ph:
            durs[n].append((en - st) / 1e3)
        for n, v in durs.items():
            print(f"   kernel {n:40s} n={len(v):5d} duration p50 {statistics.median(v):8.2f}")
        gaps = collections.defaultdict(list)
        for (s0, e0, n0), (s1, e1, n1) in zip(ph[:-1], ph[1:]):
            gaps[(n0, n1)].append((s1 - e0) / 1e3)
        for (n0, n1), v in gaps.items():
            print(f"   gap {n0} -> {n1}: n={len(v)} p50 {statistics.median(v):.2f} p90 {_pct(v, 0.9):.2f}")


def cmd_counters(a):
    print(f"# rocprofv3 counter summary: {a.title}{source_note(a.source)}")
    print(f"# command (one run per pass, PASS = the counters of one directory): {a.cmd}")
    print(f"# kernel: {a.kernel}; values are means over its dispatches of the per-dispatch sums")
    print("#")
    for d in a.dirs:
        names = sorted({r["Counter_Name"] for f in _find(d, "_counter_collection.csv")
                        for r in csv.DictReader(open(f))})
        print(f"# pass {os.path.basename(os.path.normpath(d))}: {' '.join(names)}")
        for c in names:
            vals = _pick(counter_per_dispatch(d, c), a.kernel)
            print(f"{c:32s} {statistics.mean(vals):18.1f}   ({len(vals)} dispatches)")


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--cmd", required=True)
    s.add_argument("--title", default="")
    s.add_argument("--source", default="")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--workload", default="")
    t.add_argument("--source", default="")
    t.add_argument("--algorithmic-bytes", type=float, default=0.0)
    t.add_argument("--cmd-fetch", required=True)
    t.add_argument("--cmd-write", required=True)
    c = sub.add_parser("counters")
    c.add_argument("dirs", nargs="+")
    c.add_argument("--kernel", required=True)
    c.add_argument("--cmd", required=True)
    c.add_argument("--title", default="")
    c.add_argument("--source", default="")
    g = sub.add_parser("gaps")
    g.add_argument("dir")
    g.add_argument("--cmd", required=True)
    g.add_argument("--title", default="")
    g.add_argument("--labels", default="")
    g.add_argument("--split", default="spin_kernel")
    g.add_argument("--min", type=int, default=10)
    a = ap.parse_args(argv)
    {"stats": cmd_stats, "traffic": cmd_traffic, "counters": cmd_counters, "gaps": cmd_gaps}[a.what](a)


if __name__ == "__main__":
    main()
