"""HBM traffic from hardware counters, for the roofline report.

Two rocprofv3 ``--pmc`` runs (FETCH_SIZE, then WRITE_SIZE) of the benchmark give
the counters per dispatch of a kernel; two more runs of the 1 GiB copy probe
(``bench.py --calibrate-copy``, which reads and writes exactly 2^30 bytes per
launch) give the scale from counter units to bytes.  The scaled per-launch bytes
are stored in ``profiles/<kernel>_traffic.json`` together with a hash of the
kernel sources; ``stored_traffic`` returns None once the sources have changed.

    python -m ssm_recurrent_decode_amd.profiling summarize \\
        --kernel replay_append_decode --match replay_window_kernel \\
        --fetch <dir>/..._counter_collection.csv --write <...> \\
        --calib-fetch <...> --calib-write <...> --command "<how the runs were made>"
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
PROFILES = os.path.join(ROOT, "profiles")
CALIB_BYTES = 1 << 30


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")) +
                   glob.glob(os.path.join(PKG, "csrc", "*.hpp")) +
                   [os.path.join(ROOT, "include", "ssm_recurrent_decode.h")])
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _counter_rows(path: str):
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            yield row


def per_dispatch(path: str, match: str, counter: str):
    """Counter value of every dispatch whose kernel name contains ``match``
    (values of one dispatch summed over its rows, e.g. per-XCD instances)."""
    vals = {}
    for row in _counter_rows(path):
        if match not in row.get("Kernel_Name", ""):
            continue
        if row.get("Counter_Name", counter) != counter:
            continue
        key = row.get("Dispatch_Id") or row.get("Correlation_Id")
        vals[key] = vals.get(key, 0.0) + float(row["Counter_Value"])
    return [vals[k] for k in sorted(vals, key=lambda x: int(x))]


def summarize(kernel, match, fetch, write, calib_fetch, calib_write, command, out=None):
    f = per_dispatch(fetch, match, "FETCH_SIZE")
    w = per_dispatch(write, match, "WRITE_SIZE")
    cf = per_dispatch(calib_fetch, "probe_copy", "FETCH_SIZE")
    cw = per_dispatch(calib_write, "probe_copy", "WRITE_SIZE")
    if not (f and w and cf and cw):
        raise RuntimeError("missing dispatches in the counter files")
    # first copy launch also pays the cold-start page mapping; use the rest
    cfv = sorted(cf[1:] or cf)[len(cf[1:] or cf) // 2]
    cwv = sorted(cw[1:] or cw)[len(cw[1:] or cw) // 2]
    read_scale, write_scale = CALIB_BYTES / cfv, CALIB_BYTES / cwv
    rb = sum(f) / len(f) * read_scale
    wb = sum(w) / len(w) * write_scale
    res = {"kernel": kernel, "match": match, "source_hash": kernel_source_hash(),
           "dispatches": [len(f), len(w)], "read_bytes_per_launch": round(rb),
           "write_bytes_per_launch": round(wb), "traffic_bytes_per_launch": round(rb + wb),
           "fetch_counter_per_launch": sum(f) / len(f), "write_counter_per_launch": sum(w) / len(w),
           "calibration": {"kernel": "rssm_probe_copy", "bytes_each_way": CALIB_BYTES,
                           "fetch_counter": cfv, "write_counter": cwv,
                           "read_scale_bytes_per_unit": read_scale,
                           "write_scale_bytes_per_unit": write_scale},
           "command": command}
    out = out or os.path.join(PROFILES, f"{kernel}_traffic.json")
    with open(out, "w") as fh:
        json.dump(res, fh, indent=1)
        fh.write("\n")
    return res


def stored_traffic(kernel: str):
    """(traffic bytes per launch, note) from the stored counter summary, or
    (None, reason) when there is none or the kernel sources changed since."""
    path = os.path.join(PROFILES, f"{kernel}_traffic.json")
    if not os.path.exists(path):
        return None, "no counter run recorded"
    with open(path) as fh:
        res = json.load(fh)
    if res.get("source_hash") != kernel_source_hash():
        return None, "kernel sources changed since the counters were taken"
    return res["traffic_bytes_per_launch"], (
        f"FETCH_SIZE+WRITE_SIZE per launch scaled by the 1 GiB copy probe "
        f"({os.path.relpath(path, ROOT)})")


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("summarize")
    s.add_argument("--kernel", required=True)
    s.add_argument("--match", required=True)
    s.add_argument("--fetch", required=True)
    s.add_argument("--write", required=True)
    s.add_argument("--calib-fetch", required=True)
    s.add_argument("--calib-write", required=True)
    s.add_argument("--command", required=True)
    sub.add_parser("hash")
    a = ap.parse_args(argv)
    if a.cmd == "hash":
        print(kernel_source_hash())
        return 0
    res = summarize(a.kernel, a.match, a.fetch, a.write, a.calib_fetch, a.calib_write, a.command)
    print(json.dumps(res, indent=1))
    return 0


if __name__ == "__main__":
    sys.exit(main())
