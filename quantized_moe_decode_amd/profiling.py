"""Summaries of rocprofv3 output (CSV) for the profiles kept with the code.

    python -m quantized_moe_decode_amd.profiling stats <kernel_stats.csv>
    python -m quantized_moe_decode_amd.profiling traffic <fetch counter_collection.csv>
        <write counter_collection.csv> <kernel substring> <out.json>

`stats` prints the per-kernel duration table.  `traffic` turns the
FETCH_SIZE and WRITE_SIZE counters (KiB per dispatch, one rocprofv3 --pmc
run each) into HBM bytes per launch of the named kernel.  Each counter is
scaled by what it reads for a plain device copy of known size in the same
run (the 1 GiB copy bench.py --calib-copy issues), so the figure is in
bytes as the copy sees them.  The JSON records the sha256 of the one-token
kernels' sources it was taken on; bench.py reports it only while they match.
"""

import csv
import hashlib
import json
import os
import sys

CALIB_BYTES = 1 << 30


# The sources the one-token kernels are built from (the kernels of the
# counter summary): their file and every header it includes.
DIGEST_SOURCES = ("moe.hip", "hfq4_device.h", "topk_device.h", "moe_common.h", "launch.h",
                  "xchg_device.h")


def kernel_sources_digest(root):
    h = hashlib.sha256()
    csrc = os.path.join(root, "quantized_moe_decode_amd", "csrc")
    for name in DIGEST_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def stats_table(path, top=12):
    with open(path, newline="") as f:
        rows = list(csv.DictReader(f))
    key = "TotalDurationNs" if rows and "TotalDurationNs" in rows[0] else None
    rows.sort(key=lambda r: -float(r.get(key, 0) or 0))
    out = ["%-72s %7s %11s %10s %10s %10s" % ("kernel", "calls", "total_us", "avg_us", "min_us",
                                               "max_us")]
    for r in rows[:top]:
        out.append("%-72s %7s %11.1f %10.3f %10.3f %10.3f" % (
            r["Name"][:72], r["Calls"], float(r["TotalDurationNs"]) / 1e3,
            float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3))
    return "\n".join(out)


def trace_durations(path, kernel_substr, last=None):
    """Durations (us) of the dispatches of one kernel in a kernel_trace.csv,
    in dispatch order; `last` keeps only the final ones."""
    d = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if kernel_substr in r["Kernel_Name"]:
                d.append((int(r.get("Dispatch_Id", 0) or 0),
                          (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    d.sort()
    v = [x for _, x in d]
    return v[-last:] if last else v


def _per_dispatch(path, counter):
    """{dispatch_id: (kernel_name, value)} for one counter."""
    out = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") != counter:
                continue
            did = r.get("Dispatch_Id") or r.get("Correlation_Id")
            out[did] = (r["Kernel_Name"], float(r["Counter_Value"]))
    return out


def _calibration(disp):
    """Largest copy-like dispatch: (name, KiB)."""
    best = None
    for name, v in disp.values():
        if ("copy" in name.lower() or "elementwise" in name.lower()) and (best is None or v > best[1]):
            best = (name, v)
    return best


def traffic(fetch_csv, write_csv, kernel_substr):
    f = _per_dispatch(fetch_csv, "FETCH_SIZE")
    w = _per_dispatch(write_csv, "WRITE_SIZE")
    cf, cw = _calibration(f), _calibration(w)
    if cf is None or cw is None:
        raise SystemExit("no calibration copy found in the counter runs")
    kf = CALIB_BYTES / (cf[1] * 1024.0)
    kw = CALIB_BYTES / (cw[1] * 1024.0)
    fv = [v for n, v in f.values() if kernel_substr in n]
    wv = [v for n, v in w.values() if kernel_substr in n]
    if not fv or not wv:
        raise SystemExit("kernel %r not found in the counter runs" % kernel_substr)
    fetch = sum(fv) / len(fv) * 1024.0 * kf
    write = sum(wv) / len(wv) * 1024.0 * kw
    return {"kernel": kernel_substr, "dispatches": len(fv),
            "fetch_bytes_per_launch": round(fetch), "write_bytes_per_launch": round(write),
            "hbm_bytes_per_launch": round(fetch + write),
            "calibration": {"copy_kernel": cf[0], "copy_bytes": CALIB_BYTES,
                            "fetch_kib_read": cf[1], "write_kib_read": cw[1],
                            "fetch_scale": kf, "write_scale": kw}}


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        # stats <kernel_stats.csv> [rows]
        print(stats_table(sys.argv[2], int(sys.argv[3]) if len(sys.argv) > 3 else 12))
    elif sys.argv[1] == "durations":
        # durations <kernel_trace.csv> <kernel substring> <last N>
        v = trace_durations(sys.argv[2], sys.argv[3])
        n = int(sys.argv[4])
        tail = v[-n:]
        print("%s: %d dispatches, avg %.3f us; last %d: avg %.3f us, "
              "median %.3f us" % (sys.argv[3], len(v), sum(v) / len(v), len(tail),
                                  sum(tail) / len(tail), sorted(tail)[len(tail) // 2]))
    elif sys.argv[1] == "traffic":
        root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
        t = traffic(sys.argv[2], sys.argv[3], sys.argv[4])
        t["kernel_sources_sha256"] = kernel_sources_digest(root)
        with open(sys.argv[5], "w") as fo:
            json.dump(t, fo, indent=1)
        print(json.dumps(t, indent=1))
