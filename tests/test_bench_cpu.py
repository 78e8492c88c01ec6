"""Host-side checks of bench.py: the committed counter summaries it reports
are tied to the kernel source they were measured on, and a request for more
than one GPU is refused before anything touches a device."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("kernel,wid", [("cmp_mfma_kernel", 3), ("gqa_cmp_kernel", 4)])
def test_stored_summaries_follow_the_kernel_source(kernel, wid, tmp_path, monkeypatch):
    # summaries written for the current source are reported; the same files
    # under any other source hash are not
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    h = bench.kernel_source_hash(kernel)
    with open(bench.traffic_path(kernel, wid), "w") as fh:
        json.dump({"source_sha256": h, "traffic_bytes": 123.0}, fh)
    with open(bench.mfma_path(kernel, wid), "w") as fh:
        json.dump({"source_sha256": h, "mfma_busy_frac": 0.4, "executed_tflop": 3.4, "executed_tflops": 800.0,
                   "clock_ghz": 1.8, "launches": 6}, fh)
    assert bench.stored_traffic(kernel, wid) == 123.0
    assert bench.stored_mfma(kernel, wid)["mfma_busy_frac"] == 0.4
    monkeypatch.setattr(bench, "kernel_source_hash", lambda k: "0" * 64)
    assert bench.stored_traffic(kernel, wid) is None
    assert bench.stored_mfma(kernel, wid) is None


def test_missing_summary_reports_none(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.stored_traffic("cmp_mfma_kernel", 5) is None
    assert bench.stored_mfma("cmp_mfma_kernel", 5) is None


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120, cwd=ROOT)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
