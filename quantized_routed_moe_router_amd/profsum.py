"""Condense rocprofv3 CSV output into a short Markdown summary.

    python -m quantized_routed_moe_router_amd.profsum DIR [--match NAME ...]
    python -m quantized_routed_moe_router_amd.profsum DIR --by-grid NAME

DIR is a rocprofv3 output directory written with ``--output-format csv``.
Every ``*kernel_stats.csv`` found under it (from ``--kernel-trace --stats``)
becomes a table of per-kernel launch counts and durations, and every
``*counter_collection.csv`` (from ``--pmc``) a table of each counter's mean
value per dispatch, per kernel.  ``--match`` keeps only kernels whose name
contains one of the given strings.

    python -m quantized_routed_moe_router_amd.profsum --hbm KERNEL \
        --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR --copy-bytes N

turns a FETCH_SIZE pass and a WRITE_SIZE pass over a kernel into HBM bytes
per launch.  The counters' units are fixed by the same counters read over a
plain device copy of N bytes (``bench.py --copy-calib``): bytes per counter
unit = N / (copy kernel's mean counter value).  The summary ends with
``- traffic_bytes_per_launch:`` and ``- kernel_source_sha256:`` lines, the
latter a digest of the HIP sources the counters were taken on.
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


def grid_table(path, name):
    """Durations of one kernel's dispatches grouped by grid size (workgroups)."""
    groups = collections.defaultdict(list)
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if name not in r["Kernel_Name"]:
                continue
            wg = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]) // max(
                1, int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"]))
            groups[wg].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = ["| workgroups | dispatches | avg us | min us | max us |", "|---:|---:|---:|---:|---:|"]
    for wg in sorted(groups):
        v = groups[wg]
        out.append("| %d | %d | %.2f | %.2f | %.2f |" % (wg, len(v), sum(v) / len(v), min(v), max(v)))
    return out


COPY_KERNEL = "copyBuffer"


# The sources each kernel family is compiled from (its translation unit and
# the headers it includes); other kernels use every file of csrc/.
KERNEL_SOURCES = {
    "dec_": ("common.h", "ffn_dev.h", "route_dev.h", "k_decode.hip"),
    "pf_": ("common.h", "ffn_dev.h", "k_prefill.hip"),
    "large_": ("common.h", "ffn_dev.h", "k_ffn_large.hip"),
}


def kernel_source_digest(kernel=None):
    """SHA-256 over the HIP sources the kernel is built from (csrc/), in
    file-name order: a counter summary is stale once this changes."""
    import hashlib
    h = hashlib.sha256()
    root = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
    files = sorted(os.listdir(root))
    for prefix, srcs in KERNEL_SOURCES.items():
        if kernel and kernel.startswith(prefix):
            files = sorted(srcs)
    for f in files:
        with open(os.path.join(root, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def _mean_counter(d, counter, match):
    """Mean value of ``counter`` per dispatch over kernels whose name contains ``match``."""
    tot, disp = 0.0, set()
    for p in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(p, newline="") as f:
            for r in csv.DictReader(f):
                if match in r["Kernel_Name"] and r["Counter_Name"] == counter:
                    tot += float(r["Counter_Value"])
                    disp.add((p, r["Dispatch_Id"]))
    if not disp:
        raise SystemExit("no %s values for a kernel named *%s* under %s" % (counter, match, d))
    return tot / len(disp), len(disp)


def hbm(a):
    fetch, nf = _mean_counter(a.fetch, "FETCH_SIZE", a.hbm)
    write, nw = _mean_counter(a.write, "WRITE_SIZE", a.hbm)
    cfetch, ncf = _mean_counter(a.copy_fetch, "FETCH_SIZE", COPY_KERNEL)
    cwrite, ncw = _mean_counter(a.copy_write, "WRITE_SIZE", COPY_KERNEL)
    bf, bw = a.copy_bytes / cfetch, a.copy_bytes / cwrite
    traffic = fetch * bf + write * bw
    print("HBM traffic of %s per launch, from rocprofv3 FETCH_SIZE and WRITE_SIZE passes.\n" % a.hbm)
    print("| counter | kernel mean per dispatch | dispatches | copy of %d B: mean | bytes per unit | bytes |"
          % a.copy_bytes)
    print("|---|---:|---:|---:|---:|---:|")
    print("| FETCH_SIZE | %.6g | %d | %.6g (%d) | %.2f | %.0f |" % (fetch, nf, cfetch, ncf, bf, fetch * bf))
    print("| WRITE_SIZE | %.6g | %d | %.6g (%d) | %.2f | %.0f |" % (write, nw, cwrite, ncw, bw, write * bw))
    if a.algorithmic_bytes:
        print("\nalgorithmic bytes per launch %d; traffic / algorithmic = %.4f"
              % (a.algorithmic_bytes, traffic / a.algorithmic_bytes))
    print()
    print("- traffic_bytes_per_launch: %.0f" % traffic)
    print("- kernel_source_sha256: %s" % kernel_source_digest(a.hbm))
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("dir", nargs="?")
    ap.add_argument("--match", nargs="*", default=[])
    ap.add_argument("--hbm", metavar="KERNEL", help="kernel-name substring for the HBM traffic summary")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--copy-fetch")
    ap.add_argument("--copy-write")
    ap.add_argument("--copy-bytes", type=float)
    ap.add_argument("--algorithmic-bytes", type=int, default=0)
    ap.add_argument("--by-grid", metavar="KERNEL",
                    help="durations of the kernel's dispatches grouped by workgroup count (from the kernel trace)")
    a = ap.parse_args(argv)
    if a.hbm:
        if not (a.fetch and a.write and a.copy_fetch and a.copy_write and a.copy_bytes):
            ap.error("--hbm needs --fetch, --write, --copy-fetch, --copy-write and --copy-bytes")
        return hbm(a)
    if not a.dir:
        ap.error("a rocprofv3 output directory is needed")
    found = False
    if a.by_grid:
        for p in sorted(glob.glob(os.path.join(a.dir, "**", "*kernel_trace.csv"), recursive=True)):
            found = True
            print("dispatches of %s by grid size (%s):\n" % (a.by_grid, os.path.basename(p)))
            print("\n".join(grid_table(p, a.by_grid)) + "\n")
        return 0 if found else 1
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
