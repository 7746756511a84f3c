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


def _calibration(calib_fetch: str, calib_write: str):
    """Bytes per FETCH_SIZE and per WRITE_SIZE unit, from the copy probe's runs
    (median over its launches after the first, which also maps the pages)."""
    cf = per_dispatch(calib_fetch, "probe_copy", "FETCH_SIZE")
    cw = per_dispatch(calib_write, "probe_copy", "WRITE_SIZE")
    if not (cf and cw):
        raise RuntimeError("missing copy-probe dispatches in the calibration files")
    cfv = sorted(cf[1:] or cf)[len(cf[1:] or cf) // 2]
    cwv = sorted(cw[1:] or cw)[len(cw[1:] or cw) // 2]
    return CALIB_BYTES / cfv, CALIB_BYTES / cwv


def _row_kernels(bench: dict):
    """(label, kernel-name substring, work-items, algorithmic bytes per launch
    averaged over every launch of that kernel in the run) for the rows present
    in one bench JSON line.  Rows that launch the same kernel at the same grid
    (the T = 4 verify of the verify row and of the window sweep; the GDN verify
    rounds that fill the rings before an explicit flush) are merged, weighted by
    their launch counts."""
    parts = []  # (label, match, grid, launches, total algorithmic bytes)

    def add(label, match, grid, n, avg):
        parts.append((label, match, grid, n, n * avg))

    rows = bench.get("rows", {})
    std = bench.get("standard_step")
    if std and "alg_bytes" in std:
        c = bench["config"]
        add("ssm_decode_step (standard Mamba-2 step, headline shape)", "ssm_step_kernel<64, 128>",
            c["batch"] * c["nheads"] * 256, 1, std["alg_bytes"])
    m2v, gv = "replay_window_kernel<64, 128, {T}, false, 16, false>", "gdn_verify_kernel<128, 128, {T}, 16, false>"
    g_m2, g_gdn = 512 * 32 * 256, 256 * 32 * 256
    sv = rows.get("speculative_verify")
    if sv:
        add("replay_verify_T, T = 4", m2v.format(T=4), g_m2, sv["launches"], sv["alg_bytes_avg_all_launches"])
    gs = rows.get("gdn_speculative_verify")
    if gs:
        add("gdn_replay_verify_T, T = 4", gv.format(T=4), g_gdn, gs["launches"], gs["alg_bytes_avg_all_launches"])
        st = gs["standard_step"]
        add("gdn_decode_step (standard GDN step)", "gdn_step_kernel<128, 128>", g_gdn, st["launches"], st["alg_bytes"])
    ga = rows.get("gdn_append_decode")
    if ga:
        add("gdn_replay_append_decode", "gdn_verify_kernel<128, 128, 1, 16, true>", g_gdn, ga["launches"],
            ga["alg_bytes_avg_all_launches"])
        st = ga["standard_step"]
        add("gdn_decode_step (standard GDN step)", "gdn_step_kernel<128, 128>", g_gdn, st["launches"], st["alg_bytes"])
    fl = rows.get("explicit_flush")
    if fl:
        add("replay_flush (15 entries)", "replay_flush_kernel<64, 128>", 256 * 32 * 256, fl["mamba2"]["launches"],
            fl["mamba2"]["alg_bytes"])
        g = fl["gdn"]
        add("gdn_replay_flush (12 entries)", "gdn_flush_kernel<128, 128>", g_gdn, g["launches"], g["alg_bytes"])
        n = g["buildup_verify_launches"]
        add("gdn_replay_verify_T, T = 4", gv.format(T=4), g_gdn, n, g["buildup_verify_alg_bytes_total"] / n)
    ws = rows.get("window_sweep")
    if ws:
        for fam, d, grid, gdn in (("mamba2", 64, g_m2, False), ("gdn", 128, g_gdn, True)):
            w = ws[fam]
            st = w["standard_step"]
            add("gdn_decode_step (standard GDN step)" if gdn else "ssm_decode_step (standard Mamba-2 step, B = 512)",
                f"{'gdn_step_kernel' if gdn else 'ssm_step_kernel'}<{d}, 128>", grid, st["launches"], st["alg_bytes"])
            for t in w["T"]:
                T = t["T"]
                add(f"{'gdn_replay_verify_T' if gdn else 'replay_verify_T'}, T = {T}",
                    (gv if gdn else m2v).format(T=T), grid, t["replay_launches"],
                    t["replay_alg_bytes_avg_all_launches"])
                add(f"{'gdn_snapshot_verify_T' if gdn else 'ssm_snapshot_verify_T'}, T = {T}",
                    f"snapshot_verify_kernel<{d}, 128, {T}, {'true' if gdn else 'false'}>", grid,
                    t["snapshot_launches"], t["snapshot_alg_bytes"])
    merged = {}
    for label, match, grid, n, tot in parts:
        m = merged.setdefault((match, grid), [label, 0, 0.0])
        m[1] += n
        m[2] += tot
    return [(label, match, grid, tot / n) for (match, grid), (label, n, tot) in merged.items()]


def rows_traffic(fetch, write, calib_fetch, calib_write, bench_log, command, title, out_md):
    """Measured HBM bytes (calibrated FETCH_SIZE + WRITE_SIZE, mean per dispatch)
    against the algorithmic bytes of every row kernel the bench run launched."""
    with open(bench_log) as fh:
        bench = json.loads([ln for ln in fh.read().splitlines() if ln.startswith("{")][-1])
    rs, ws = _calibration(calib_fetch, calib_write)
    f, w = per_dispatch_counters(fetch), per_dispatch_counters(write)
    lines = [f"# {title}", "", "Commands (repository root on one MI355X; `<repo>` is its path):", "", "```",
             command, "```", "",
             f"Measured = mean per dispatch of FETCH_SIZE x {rs:.1f} B plus WRITE_SIZE x {ws:.1f} B (the "
             "units of the 1 GiB copy probe, read and written once per launch); algorithmic = the "
             "traffic model's bytes, averaged over the same dispatches (every launch of the kernel in the "
             "run, warm-up and untimed passes included).  Kernels are told apart by name and grid.  "
             f"Kernel sources at the time of the runs: hash `{kernel_source_hash()}` "
             "(`python -m ssm_recurrent_decode_amd.profiling hash`).", "",
             "| kernel | work-items | dispatches | read MB | written MB | measured MB | algorithmic MB | measured / algorithmic |",
             "|---|---|---|---|---|---|---|---|"]
    res = []
    for label, match, grid, alg in _row_kernels(bench):
        fv = [d["FETCH_SIZE"] for d in f.values() if match in d["name"] and d["grid"] == grid and "FETCH_SIZE" in d]
        wv = [d["WRITE_SIZE"] for d in w.values() if match in d["name"] and d["grid"] == grid and "WRITE_SIZE" in d]
        if not fv or not wv:
            continue
        rb, wb = sum(fv) / len(fv) * rs, sum(wv) / len(wv) * ws
        res.append((label, rb + wb, alg))
        lines.append(f"| {label} | {grid} | {len(fv)} | {rb / 1e6:.1f} | {wb / 1e6:.1f} | {(rb + wb) / 1e6:.1f} | "
                     f"{alg / 1e6:.1f} | {(rb + wb) / alg:.3f} |")
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return res


MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_F32", "SQ_VALU_MFMA_BUSY_CYCLES")
BF16_COUNTER = "SQ_INSTS_VALU_MFMA_MOPS_BF16"
NUM_SIMDS = 256 * 4
CLOCK_HZ = 2.4e9
FP32_MFMA_PEAK = 157.3e12


def per_dispatch_counters(path: str):
    """{dispatch id: {"name", "grid", "dur_s", counter: value}} from a rocprofv3
    counter-collection CSV (one row per counter per dispatch, already reduced
    over the hardware instances)."""
    out = {}
    for row in _counter_rows(path):
        key = int(row.get("Dispatch_Id") or row.get("Correlation_Id"))
        d = out.setdefault(key, {"name": row.get("Kernel_Name", ""), "grid": int(row.get("Grid_Size", 0)),
                                 "dur_s": (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) * 1e-9})
        d[row["Counter_Name"]] = d.get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
    return out


def mfma_summary(path: str, kernels, command: str, out_md: str):
    """Per kernel (substring match) and grid size, split into dispatches with and
    without MFMA work: MFMA flops per dispatch (SQ_INSTS_VALU_MFMA_MOPS_F32 x 512,
    plus SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 when the run collected it),
    duration (dispatch timestamps of the counter run), achieved MFMA FLOP/s
    against the fp32 dense peak, and the MFMA busy fraction of all SIMD cycles
    (SQ_VALU_MFMA_BUSY_CYCLES summed over SIMDs / (duration x 2.4 GHz x 1024))."""
    disp = per_dispatch_counters(path)
    lines = ["# MFMA use of the decode kernels (rocprofv3 counters)", "",
             "Command (repository root on one MI355X; `<repo>` is its path):", "", "```", command, "```", "",
             "Per dispatch: MFMA flops = (`SQ_INSTS_VALU_MFMA_MOPS_F32` + `SQ_INSTS_VALU_MFMA_MOPS_BF16`) "
             "x 512 (the bf16 ones are the hi/lo split products of the verify combine and the GDN "
             "readouts); duration from the dispatch timestamps of the same run; MFMA busy = "
             "`SQ_VALU_MFMA_BUSY_CYCLES` (summed over SIMDs) / (duration x 2.4 GHz x 1024 SIMDs).  "
             "Peaks: 157.3 TFLOP/s dense fp32, 2.5 PFLOP/s dense bf16.  The kernels are HBM-bound; "
             "these figures show that the matrix-core work (the fold of a flush, the verify "
             "combine, the GDN readouts) stays far from being a bottleneck.", "",
             "| kernel | work-items (threads) | dispatches | fp32 MFMA GFLOP / dispatch | bf16 MFMA GFLOP / dispatch | us | MFMA TFLOP/s | MFMA busy |",
             "|---|---|---|---|---|---|---|---|"]
    res = {}
    for label, match in kernels:
        groups = {}
        for d in disp.values():
            if match in d["name"] and all(c in d for c in MFMA_COUNTERS):
                work = d["SQ_INSTS_VALU_MFMA_MOPS_F32"] + d.get(BF16_COUNTER, 0.0)
                kind = "with MFMA work" if work > 0 else "without"
                groups.setdefault((d["grid"], kind), []).append(d)
        for (grid, kind), ds in sorted(groups.items()):
            n = len(ds)
            f32 = sum(d["SQ_INSTS_VALU_MFMA_MOPS_F32"] for d in ds) * 512 / n
            b16 = sum(d.get(BF16_COUNTER, 0.0) for d in ds) * 512 / n
            t = sum(d["dur_s"] for d in ds) / n
            busy = sum(d["SQ_VALU_MFMA_BUSY_CYCLES"] for d in ds) / n
            rate = (f32 + b16) / t if t > 0 else 0.0
            frac_busy = busy / (t * CLOCK_HZ * NUM_SIMDS) if t > 0 else 0.0
            res[(label, grid, kind)] = {"dispatches": n, "flops_f32": f32, "flops_bf16": b16, "us": t * 1e6,
                                        "rate": rate, "busy": frac_busy}
            lines.append(f"| {label} ({kind}) | {grid} | {n} | {f32 / 1e9:.3f} | {b16 / 1e9:.3f} | {t * 1e6:.1f} | "
                         f"{rate / 1e12:.2f} | {frac_busy:.4f} |")
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return res


def trace_summary(trace_csv: str, command: str, out_md: str, title: str, match: str = "rssm",
                  segment: str = "", last: int = 0):
    """Kernel durations of a rocprofv3 --kernel-trace CSV grouped by kernel name and
    grid size (one template instance can serve several workload shapes).  With
    ``segment``, also the longest run of back-to-back dispatches of that kernel,
    or only its last ``last`` dispatches (the bench's timed pass follows its
    untimed warm-up launches without a pause)."""
    groups = {}
    for row in _counter_rows(trace_csv):
        name = row.get("Kernel_Name", "")
        if match not in name:
            continue
        grid = int(row.get("Grid_Size_X", 0)) * int(row.get("Grid_Size_Y", 1)) * int(row.get("Grid_Size_Z", 1))
        us = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) * 1e-3
        groups.setdefault((name, grid), []).append(us)
    lines = [f"# {title}", "", "Command (repository root on one MI355X; `<repo>` is its path):", "",
             "```", command, "```", "",
             "| kernel | work-items (threads) | calls | avg us | median us | min us | max us |",
             "|---|---|---|---|---|---|---|"]
    for (name, grid), v in sorted(groups.items(), key=lambda kv: (kv[0][0], kv[0][1])):
        v = sorted(v)
        lines.append(f"| {name.replace('|', '/')} | {grid} | {len(v)} | {sum(v) / len(v):.2f} | "
                     f"{v[len(v) // 2]:.2f} | {v[0]:.2f} | {v[-1]:.2f} |")
    if segment:
        # a run ends at another kernel or at an idle gap over 20 us (the bench
        # synchronises between its passes)
        runs, cur = [], []
        for row in sorted(_counter_rows(trace_csv), key=lambda r_: int(r_["Start_Timestamp"])):
            s_, e = int(row["Start_Timestamp"]), int(row["End_Timestamp"])
            if cur and (segment not in row.get("Kernel_Name", "") or s_ - cur[-1][1] > 20_000):
                runs.append(cur)
                cur = []
            if segment in row.get("Kernel_Name", ""):
                cur.append((s_, e))
        if cur:
            runs.append(cur)
        if runs:
            run = max(runs, key=len)
            n_run = len(run)
            what = "the bench's back-to-back timed pass"
            if last and last < n_run:
                run = run[-last:]
                what = f"the last {last} of a run of {n_run}, the bench's timed pass after its warm-up"
            dur = [(e - s_) * 1e-3 for s_, e in run]
            gap = (run[-1][0] - run[0][0]) * 1e-3 / max(len(run) - 1, 1)
            lines += ["", f"Consecutive `{segment}` dispatches ({what}): {len(run)} launches, average "
                          f"duration {sum(dur) / len(dur):.2f} us, average start-to-start spacing {gap:.2f} us."]
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return groups


def counter_table(csvs, match: str, command: str, title: str, out_md: str, note: str = ""):
    """Mean value per dispatch of every counter in one or more rocprofv3 --pmc
    CSVs (one per pass), for the dispatches whose kernel name contains
    ``match``, as a markdown table."""
    rows = []
    for path in csvs:
        per = {}
        for row in _counter_rows(path):
            if match not in row.get("Kernel_Name", ""):
                continue
            key = row.get("Dispatch_Id") or row.get("Correlation_Id")
            c = row["Counter_Name"]
            per.setdefault(c, {}).setdefault(key, 0.0)
            per[c][key] += float(row["Counter_Value"])
        for c, d in sorted(per.items()):
            rows.append((c, len(d), sum(d.values()) / len(d)))
    lines = [f"# {title}", "", "Commands (repository root on one MI355X; `<repo>` is its path):", "",
             "```", command, "```", "", f"Kernel: `{match}`.  Kernel sources: hash `{kernel_source_hash()}`.", ""]
    if note:
        lines += [note, ""]
    lines += ["| counter | dispatches | mean per dispatch |", "|---|---|---|"]
    lines += [f"| {c} | {n} | {v:,.0f} |" for c, n, v in rows]
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return rows


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
    s.add_argument("--out", default=None, help="output json (default profiles/<kernel>_traffic.json)")
    m = sub.add_parser("mfma")
    m.add_argument("--csv", required=True)
    m.add_argument("--out", required=True)
    m.add_argument("--command", required=True)
    t = sub.add_parser("trace")
    t.add_argument("--csv", required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--title", required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--last", type=int, default=0,
                   help="with --segment: only the last N dispatches of the longest run")
    t.add_argument("--segment", default="",
                   help="also report the longest run of consecutive dispatches of this kernel")
    rt = sub.add_parser("rows-traffic")
    rt.add_argument("--fetch", required=True)
    rt.add_argument("--write", required=True)
    rt.add_argument("--calib-fetch", required=True)
    rt.add_argument("--calib-write", required=True)
    rt.add_argument("--bench-log", required=True, help="the stdout of one of the two counter runs")
    rt.add_argument("--title", required=True)
    rt.add_argument("--command", required=True)
    rt.add_argument("--out", required=True)
    ct = sub.add_parser("counters")
    ct.add_argument("--csv", required=True, nargs="+", help="counter_collection.csv of each --pmc pass")
    ct.add_argument("--match", required=True)
    ct.add_argument("--title", required=True)
    ct.add_argument("--command", required=True)
    ct.add_argument("--note", default="")
    ct.add_argument("--out", required=True)
    sub.add_parser("hash")
    a = ap.parse_args(argv)
    if a.cmd == "hash":
        print(kernel_source_hash())
        return 0
    if a.cmd == "counters":
        counter_table(a.csv, a.match, a.command, a.title, a.out, a.note)
        print(open(a.out).read())
        return 0
    if a.cmd == "rows-traffic":
        rows_traffic(a.fetch, a.write, a.calib_fetch, a.calib_write, a.bench_log, a.command, a.title, a.out)
        print(open(a.out).read())
        return 0
    if a.cmd == "trace":
        trace_summary(a.csv, a.command, a.out, a.title, segment=a.segment, last=a.last)
        print(open(a.out).read())
        return 0
    if a.cmd == "mfma":
        kernels = [("replay_append_decode", "replay_window_kernel<64, 128, 1, true, 16, false"),
                   ("replay_append_decode_conv", "replay_window_kernel<64, 128, 1, true, 16, true"),
                   ("replay_verify_T (T=4)", "replay_window_kernel<64, 128, 4, false"),
                   ("replay_verify_T (T=6, combine on MFMA)", "replay_window_kernel<64, 128, 6, false"),
                   ("gdn_replay_verify_T (T=4)", "gdn_verify_kernel<128, 128, 4, 16, false"),
                   ("gdn_replay_append_decode", "gdn_verify_kernel<128, 128, 1, 16, true"),
                   ("ssm_decode_step", "ssm_step_kernel")]
        mfma_summary(a.csv, kernels, a.command, a.out)
        print(open(a.out).read())
        return 0
    res = summarize(a.kernel, a.match, a.fetch, a.write, a.calib_fetch, a.calib_write, a.command, a.out)
    print(json.dumps(res, indent=1))
    return 0


if __name__ == "__main__":
    sys.exit(main())
