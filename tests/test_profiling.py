"""The counter and trace summaries that write profiles/, on small hand-made
rocprofv3-style CSV files: counter units scaled by the copy probe's calibration
(its first, cold launch ignored), kernels selected by name and grid, rows that
share a kernel merged by launch count, stale summaries refused."""
import csv
import json
import os

from ssm_recurrent_decode_amd import profiling as pf

APPEND = "void rssm::replay_window_kernel<64, 128, 1, true, 16, false>(rssm::ReplayParams)"
VERIFY = "void rssm::gdn_verify_kernel<128, 128, 4, 16, false>(rssm::GdnReplayParams)"
COPY = "rssm::probe_copy_kernel(rssm::CopyParams)"
G_GDN = 256 * 32 * 256


def _counters(path, rows):
    """rows: (dispatch id, kernel, grid, counter, value, start ns, end ns)."""
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value",
                    "Start_Timestamp", "End_Timestamp"])
        for r in rows:
            w.writerow(r)


def _calibration(tmp_path):
    cf, cw = tmp_path / "cf.csv", tmp_path / "cw.csv"
    # first launch cold (ignored), then 2^30 bytes = 524,288 fetch units of 2 KiB
    _counters(cf, [(1, COPY, 1 << 20, "FETCH_SIZE", 600_000, 0, 1)] +
              [(i, COPY, 1 << 20, "FETCH_SIZE", 524_288, 0, 1) for i in range(2, 6)])
    _counters(cw, [(1, COPY, 1 << 20, "WRITE_SIZE", 900_000, 0, 1)] +
              [(i, COPY, 1 << 20, "WRITE_SIZE", 1_048_576, 0, 1) for i in range(2, 6)])
    return str(cf), str(cw)


def test_summarize_scales_and_selects(tmp_path):
    cf, cw = _calibration(tmp_path)
    fe, wr = tmp_path / "f.csv", tmp_path / "w.csv"
    # two per-instance rows per dispatch are summed; another kernel is ignored
    _counters(fe, [(1, APPEND, 8192, "FETCH_SIZE", 60_000, 0, 1), (1, APPEND, 8192, "FETCH_SIZE", 40_000, 0, 1),
                   (2, APPEND, 8192, "FETCH_SIZE", 120_000, 0, 1), (3, COPY, 1, "FETCH_SIZE", 7, 0, 1)])
    _counters(wr, [(1, APPEND, 8192, "WRITE_SIZE", 1_000, 0, 1), (2, APPEND, 8192, "WRITE_SIZE", 3_000, 0, 1)])
    out = tmp_path / "t.json"
    res = pf.summarize("replay_append_decode", "replay_window_kernel<64, 128, 1, true, 16, false>", str(fe),
                       str(wr), cf, cw, "cmd", str(out))
    assert res["dispatches"] == [2, 2]
    assert res["read_bytes_per_launch"] == 110_000 * 2048
    assert res["write_bytes_per_launch"] == 2_000 * 1024
    assert json.load(open(out))["source_hash"] == pf.kernel_source_hash()


def test_stored_traffic_refuses_stale_counters(tmp_path, monkeypatch):
    monkeypatch.setattr(pf, "PROFILES", str(tmp_path))
    assert pf.stored_traffic("k")[0] is None
    rec = {"source_hash": pf.kernel_source_hash(), "traffic_bytes_per_launch": 123}
    (tmp_path / "k_traffic.json").write_text(json.dumps(rec))
    assert pf.stored_traffic("k")[0] == 123
    rec["source_hash"] = "0" * 16
    (tmp_path / "k_traffic.json").write_text(json.dumps(rec))
    val, why = pf.stored_traffic("k")
    assert val is None and "changed" in why


def test_rows_traffic_merges_rows_that_share_a_kernel(tmp_path):
    cf, cw = _calibration(tmp_path)
    bench = {"config": {"batch": 256, "nheads": 32},
             "rows": {"gdn_speculative_verify": {"launches": 3, "alg_bytes_avg_all_launches": 2048 * 1000,
                                                 "standard_step": {"launches": 1, "alg_bytes": 5}},
                      "explicit_flush": {"mamba2": {"launches": 1, "alg_bytes": 1},
                                         "gdn": {"launches": 1, "alg_bytes": 1, "buildup_verify_launches": 1,
                                                 "buildup_verify_alg_bytes_total": 2048 * 2000}}}}
    log = tmp_path / "bench.log"
    log.write_text("progress line\n" + json.dumps(bench) + "\n")
    fe, wr = tmp_path / "f.csv", tmp_path / "w.csv"
    # four launches of the GDN verify at its grid, one more at another grid (not counted)
    _counters(fe, [(i, VERIFY, G_GDN, "FETCH_SIZE", 1_250, 0, 1) for i in range(4)] +
              [(9, VERIFY, 1024, "FETCH_SIZE", 99_999, 0, 1)])
    _counters(wr, [(i, VERIFY, G_GDN, "WRITE_SIZE", 0, 0, 1) for i in range(4)])
    out = tmp_path / "rows.md"
    res = pf.rows_traffic(str(fe), str(wr), cf, cw, str(log), "cmd", "title", str(out))
    got = {label: (meas, alg) for label, meas, alg in res}
    meas, alg = got["gdn_replay_verify_T, T = 4"]
    assert meas == 1_250 * 2048
    assert alg == 2048 * (3 * 1000 + 2000) / 4      # launch-weighted over both rows
    assert f"| gdn_replay_verify_T, T = 4 | {G_GDN} | 4 |" in out.read_text()


def test_trace_groups_by_kernel_and_grid(tmp_path):
    tr = tmp_path / "trace.csv"
    with open(tr, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z", "Start_Timestamp", "End_Timestamp"])
        w.writerows([(APPEND, 2097152, 1, 1, 0, 50_000), (APPEND, 2097152, 1, 1, 0, 54_000),
                     (APPEND, 8388608, 1, 1, 0, 190_000), ("other", 1, 1, 1, 0, 5)])
    out = tmp_path / "t.md"
    groups = pf.trace_summary(str(tr), "cmd", str(out), "title")
    assert sorted(groups[(APPEND, 2097152)]) == [50.0, 54.0] and groups[(APPEND, 8388608)] == [190.0]
    assert len(groups) == 2 and "| 2 | 52.00 |" in out.read_text()


def test_mfma_summary_counts_both_precisions(tmp_path):
    p = tmp_path / "m.csv"
    dur = 100_000  # ns
    rows = []
    for i, (f32, b16) in enumerate([(8, 16), (8, 16), (0, 0)]):
        for name, val in (("SQ_INSTS_VALU_MFMA_MOPS_F32", f32), ("SQ_INSTS_VALU_MFMA_MOPS_BF16", b16),
                          ("SQ_VALU_MFMA_BUSY_CYCLES", 2.4e9 * 1e-4 * 1024 * 0.5 if f32 else 0)):
            rows.append((i, VERIFY, G_GDN, name, val, 0, dur))
    _counters(p, rows)
    res = pf.mfma_summary(str(p), [("gdn verify", "gdn_verify_kernel<128, 128, 4")], "cmd", str(tmp_path / "m.md"))
    w = res[("gdn verify", G_GDN, "with MFMA work")]
    assert w["dispatches"] == 2 and w["flops_f32"] == 8 * 512 and w["flops_bf16"] == 16 * 512
    assert abs(w["busy"] - 0.5) < 1e-9 and abs(w["us"] - 100.0) < 1e-9
    assert res[("gdn verify", G_GDN, "without")]["dispatches"] == 1
    assert os.path.exists(tmp_path / "m.md")


def test_trace_reports_the_longest_back_to_back_run(tmp_path):
    tr = tmp_path / "trace.csv"
    rows = [("conv", 0, 5), (APPEND, 10, 60), ("conv", 61, 66), (APPEND, 70, 120)]      # eager: interleaved
    rows += [(APPEND, 200 + 55 * i, 250 + 55 * i) for i in range(4)]                   # timed pass
    rows += [("other", 1000, 1001)]
    with open(tr, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z", "Start_Timestamp", "End_Timestamp"])
        w.writerows([(n, 1, 1, 1, s * 1000, e * 1000) for n, s, e in rows])
    out = tmp_path / "t.md"
    pf.trace_summary(str(tr), "cmd", str(out), "title", match="", segment="replay_window_kernel")
    text = out.read_text()
    assert "4 launches, average duration 50.00 us, average start-to-start spacing 55.00 us" in text


def test_trace_can_keep_the_last_dispatches_of_the_run(tmp_path):
    tr = tmp_path / "trace.csv"
    rows = [(APPEND, 55 * i, 55 * i + 80) for i in range(3)]                        # warm-up, slower
    rows += [(APPEND, 165 + 55 * i, 165 + 55 * i + 50) for i in range(4)]          # timed pass
    with open(tr, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z", "Start_Timestamp", "End_Timestamp"])
        w.writerows([(n, 1, 1, 1, s * 1000, e * 1000) for n, s, e in rows])
    out = tmp_path / "t.md"
    pf.trace_summary(str(tr), "cmd", str(out), "title", match="", segment="replay_window_kernel", last=4)
    text = out.read_text()
    assert "the last 4 of a run of 7" in text
    assert "4 launches, average duration 50.00 us, average start-to-start spacing 55.00 us" in text
