"""Summarise rocprofv3 CSV output (kernel trace and counter collection).

    python -m measure.profsummary trace <run>_kernel_trace.csv
    python -m measure.profsummary pmc <run>_counter_collection.csv COUNTER [calib_kernel calib_bytes]
    python -m measure.profsummary pmctable NAME_FILTER <pass1>_counter_collection.csv [<pass2>...]
    python -m measure.profsummary sha

`trace` prints, per kernel name and grid size, the dispatch count and the
mean / min / max duration in microseconds.  `pmc` prints, per kernel name and
grid size, the mean of COUNTER per dispatch (nominally KiB for FETCH_SIZE and
WRITE_SIZE) and, given a calibration kernel (a name prefix) of known byte
count per dispatch, the factor that turns the counter into bytes and the
scaled bytes per dispatch.  The grid size (work-items) tells the shapes of one
kernel apart.  `pmctable` prints the
mean of every counter per dispatch for the kernels whose name contains
NAME_FILTER, over several counter passes.  `sha` prints the hash of the kernel sources that a counter
summary records (bench.py reports its traffic only while they match).
"""
import collections
import csv
import hashlib
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# The sources that decide what the SpMV kernels do and how they are launched.
KERNEL_SOURCES = ["nmspmv.hip", "nm_plan.h", "nm_rules.h", "nm_decode.h"]


def kernel_sources_sha256():
    """sha256 over the kernel sources (in KERNEL_SOURCES order): a counter
    summary taken from another version of them no longer describes the kernels."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "sparse_matrix_vector_amd", "csrc", name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def short(name, width=110):
    name = name.replace("(anonymous namespace)::", "")
    return name if len(name) <= width else name[:width] + "..."


def _grid(r):
    for k in ("Grid_Size", "Grid_Size_X"):
        if k in r:
            return int(r[k])
    return 0


def trace(path):
    dur = collections.defaultdict(list)
    with open(path) as fh:
        for r in csv.DictReader(fh):
            dur[(r["Kernel_Name"], _grid(r))].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    rows = sorted(dur.items(), key=lambda kv: -sum(kv[1]))
    total = sum(sum(v) for v in dur.values())
    print(f"{'calls':>7} {'grid':>9} {'mean_us':>9} {'min_us':>9} {'max_us':>9} {'share':>6}  kernel")
    for (name, grid), v in rows:
        print(f"{len(v):7d} {grid:9d} {sum(v) / len(v):9.3f} {min(v):9.3f} {max(v):9.3f} "
              f"{100 * sum(v) / total:5.1f}%  {short(name)}")


def pmc(path, counter, calib_kernel=None, calib_bytes=None):
    vals = collections.defaultdict(list)
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] == counter:
                vals[(r["Kernel_Name"], _grid(r))].append(float(r["Counter_Value"]))
    factor = None
    if calib_kernel:
        cal = [v for (k, _), vs in vals.items() if short(k, 1 << 20).startswith(calib_kernel) for v in vs]
        if cal:
            factor = float(calib_bytes) / (sum(cal) / len(cal))
            print(f"calibration: {calib_kernel} reads {sum(cal) / len(cal):.1f} {counter} units per dispatch "
                  f"for {int(calib_bytes)} bytes -> {factor:.3f} bytes per unit")
    print(f"{'calls':>7} {'grid':>9} {'mean_' + counter:>16} {'bytes/dispatch':>16}  kernel")
    for (name, grid), v in sorted(vals.items(), key=lambda kv: -sum(kv[1])):
        mean = sum(v) / len(v)
        scaled = f"{mean * factor:16.0f}" if factor else f"{'':>16}"
        print(f"{len(v):7d} {grid:9d} {mean:16.1f} {scaled}  {short(name)}")


def pmc_table(paths, name_filter="", min_calls=1):
    """Mean of every counter per dispatch, per kernel name and grid size, over
    one or more counter-collection CSVs (one pass each), for the kernels whose
    name contains name_filter."""
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    for path in paths:
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if name_filter in r["Kernel_Name"]:
                    vals[(r["Kernel_Name"], _grid(r))][r["Counter_Name"]].append(float(r["Counter_Value"]))
    counters = sorted({c for per in vals.values() for c in per})
    for (name, grid), per in sorted(vals.items(), key=lambda kv: (kv[0][0], kv[0][1])):
        calls = max(len(v) for v in per.values())
        if calls < min_calls:
            continue
        print(f"{short(name, 60)}  grid {grid}  ({calls} dispatches)")
        for c in counters:
            if c in per:
                v = per[c]
                print(f"    {c:40s} {sum(v) / len(v):16.1f}")


if __name__ == "__main__":
    if len(sys.argv) >= 3 and sys.argv[1] == "trace":
        trace(sys.argv[2])
    elif len(sys.argv) >= 4 and sys.argv[1] == "pmc":
        pmc(sys.argv[2], sys.argv[3], *(sys.argv[4:6]))
    elif len(sys.argv) >= 4 and sys.argv[1] == "pmctable":
        pmc_table(sys.argv[3:], sys.argv[2])
    elif len(sys.argv) == 2 and sys.argv[1] == "sha":
        print(kernel_sources_sha256())
    else:
        print(__doc__)
        sys.exit(2)
