"""bench.py's host-side contract, checked without a GPU: it refuses more than one GPU with a
message, and the traffic figure it reports is read from the committed counter summary only while
that summary matches the kernel source."""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_is_read_only_for_the_matching_kernel_source(tmp_path, monkeypatch):
    summary = tmp_path / "traffic.md"
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(summary))
    assert bench.read_traffic(1.0) is None                      # no summary
    summary.write_text("- kernel_source_sha256: %s\n- hbm_bytes_per_launch: 1.5e9\n" % bench.kernel_source_hash())
    assert bench.read_traffic(1.0) == pytest.approx(1.5e9)
    summary.write_text("- kernel_source_sha256: 0000000000000000\n- hbm_bytes_per_launch: 1.5e9\n")
    assert bench.read_traffic(1.0) is None                      # stale: another kernel source


def test_committed_traffic_summary_names_its_commands():
    text = open(os.path.join(ROOT, "profiles", "traffic_gemm_accum8192.md")).read()
    assert re.search(r"rocprofv3 --pmc FETCH_SIZE .* -- python3 \S*bench\.py", text)
    assert re.search(r"rocprofv3 --pmc WRITE_SIZE .* -- python3 \S*bench\.py", text)
    assert re.search(r"^- kernel_source_sha256: [0-9a-f]{16}$", text, flags=re.M)


def test_every_profile_names_its_command():
    """Each committed summary gives the command that produced its figures."""
    pdir = os.path.join(ROOT, "profiles")
    for name in os.listdir(pdir):
        text = open(os.path.join(pdir, name)).read()
        assert "bench.py" in text or "autotune" in text, name


def test_peak_is_the_published_fp16_dense_figure():
    assert bench.PEAK_TFLOPS == pytest.approx(2516.58, abs=0.01)   # 256 CUs x 4096 FLOP/clk x 2.4 GHz
