"""Condense rocprofv3 CSV output into a short Markdown summary.

    python -m quantized_routed_moe_router_amd.profsum DIR [--match NAME ...]

DIR is a rocprofv3 output directory written with ``--output-format csv``.
Every ``*kernel_stats.csv`` found under it (from ``--kernel-trace --stats``)
becomes a table of per-kernel launch counts and durations, and every
``*counter_collection.csv`` (from ``--pmc``) a table of each counter's mean
value per dispatch, per kernel.  ``--match`` keeps only kernels whose name
contains one of the given strings.
"""
import argparse
import collections
import csv
import glob
import os
import sys


def _short(name, width=72):
    name = name.split("(")[0] if "(" in name else name
    return name if len(name) <= width else name[:width - 3] + "..."


def _keep(name, match):
    return not match or any(m in name for m in match)


def kernel_stats(path, match):
    rows = list(csv.DictReader(open(path, newline="")))
    out = ["| kernel | calls | avg us | min us | max us | % of time |", "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        name = r.get("Name") or r.get("KERNEL_NAME") or ""
        if not _keep(name, match):
            continue
        out.append("| %s | %s | %.2f | %.2f | %.2f | %.1f |" % (
            _short(name), r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    return out


def counters(path, match):
    acc = collections.defaultdict(lambda: collections.defaultdict(float))
    disp = collections.defaultdict(set)
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            if not _keep(name, match):
                continue
            acc[name][r["Counter_Name"]] += float(r["Counter_Value"])
            disp[name].add(r["Dispatch_Id"])
    names = sorted({c for d in acc.values() for c in d})
    out = ["| kernel | dispatches | " + " | ".join(names) + " |", "|---|---:|" + "---:|" * len(names)]
    for k in sorted(acc, key=lambda k: -len(disp[k])):
        n = len(disp[k])
        out.append("| %s | %d | " % (_short(k), n) + " | ".join("%.6g" % (acc[k][c] / n) for c in names) + " |")
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("dir")
    ap.add_argument("--match", nargs="*", default=[])
    a = ap.parse_args(argv)
    found = False
    for p in sorted(glob.glob(os.path.join(a.dir, "**", "*kernel_stats.csv"), recursive=True)):
        found = True
        print("kernel durations (%s):\n" % os.path.basename(p))
        print("\n".join(kernel_stats(p, a.match)) + "\n")
    for p in sorted(glob.glob(os.path.join(a.dir, "**", "*counter_collection.csv"), recursive=True)):
        found = True
        print("counters, mean per dispatch (%s):\n" % os.path.basename(p))
        print("\n".join(counters(p, a.match)) + "\n")
    if not found:
        print("no rocprofv3 CSV output under %s" % a.dir, file=sys.stderr)
        return 1
    return 0


if __name__ == "__main__":
    sys.exit(main())
