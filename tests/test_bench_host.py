"""Host-side parts of bench.py that run without a GPU: the one-GPU guard and the
two CPU-oracle legs (single process, and the batch split over spawned processes).
The rates themselves are not checked, only that each leg runs the oracle over the
stated sample and reports what it used."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_cpu_baseline_single_core():
    res = bench._cpu_baseline(1)
    assert res["kind"] == "oracle" and res["cores"] == 1 and res["unit"] == "tokens/s"
    assert res["value"] > 0 and "256" in res["sample"]
    assert res["cpu_model"] and res["cores_available"] == len(os.sched_getaffinity(0))


@pytest.mark.timeout(300)
def test_cpu_baseline_all_cores_splits_the_batch():
    res = bench._cpu_baseline_all_cores(1, max_workers=2)
    assert res["kind"] == "oracle" and res["unit"] == "tokens/s"
    assert res["cores"] == min(2, len(os.sched_getaffinity(0)))
    assert res["value"] > 0 and f"over {res['cores']} processes" in res["sample"]
    assert res["cores_available"] == len(os.sched_getaffinity(0))
    assert f"{res['cores']} of the {res['cores_available']} cores" in res["sample"]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("cfg_id", [2, 4])
def test_cpu_spec_baseline_runs_the_oracle(cfg_id):
    res = bench._cpu_spec_baseline(cfg_id, 2, rounds=2)
    assert res["kind"] == "oracle" and res["cores"] == 1 and res["unit"] == "verified positions/s"
    assert res["value"] > 0 and res["accepted_tokens_per_s"] >= 0
    assert "requests 0..1" in res["sample"] and "2 verify rounds" in res["sample"]


@pytest.mark.timeout(300)
def test_cpu_standard_baseline_runs_one_ring_cycle():
    res = bench._cpu_standard_baseline(3, 2, capacity=4)
    assert res["kind"] == "oracle" and res["cores"] == 1 and res["unit"] == "tokens/s"
    assert res["value"] > 0 and "requests 0..1 of 256 (128 heads)" in res["sample"]
    assert "4 decode steps" in res["sample"]


def test_a_failing_row_is_recorded_and_the_rest_skipped(monkeypatch):
    def boom(*args, **kwargs):
        raise ValueError("planted")

    monkeypatch.setattr(bench, "_row_verify", boom)
    out = bench._rows(None, None, None, None, None, None, None,
                      ["speculative_verify", "gdn_speculative_verify", "max_concurrency"])
    assert out["speculative_verify"] == {"error": "ValueError: planted"}
    assert out["gdn_speculative_verify"] == {"skipped": "row speculative_verify failed"}
    assert out["max_concurrency"] == {"skipped": "row speculative_verify failed"}
