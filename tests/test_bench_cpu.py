"""Host-side checks of bench.py's contract (no GPU needed): one GPU only, a clean error
without a GPU, and the committed traffic summary parses into per-launch byte counts."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _run(*args, timeout=120):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=timeout, cwd=ROOT)


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_is_refused_with_a_message(n):
    p = _run("--gpus", n)
    assert p.returncode == 2
    assert "one GPU" in p.stderr and f"--gpus {n}" in p.stderr
    assert p.stdout.strip() == ""


@pytest.mark.parametrize("workload", ["single_1024", "large_4096"])
def test_traffic_summary_parses(workload):
    text = open(bench.traffic_path(workload)).read()
    assert "```traffic" in text and "rocprofv3 --pmc FETCH_SIZE" in text and "rocprofv3 --pmc WRITE_SIZE" in text
    block = text.split("```traffic", 1)[1].split("```", 1)[0].strip().splitlines()
    fams = {line.split()[0] for line in block}
    # both workloads run their matrix products on the three-piece kernel
    assert {"gemm_x3", "qr_panel", "quant", "dequant"} <= fams
    rec = bench.recorded_traffic(workload)
    # every family whose kernel source is unchanged since the counters carries a positive byte count
    for fam, b in rec.items():
        assert fam in fams and b > 0


def test_profiles_name_their_commands():
    prof = os.path.join(ROOT, "profiles")
    for name in os.listdir(prof):
        text = open(os.path.join(prof, name)).read()
        assert "rocprofv3" in text, name
        assert "bench.py" in text, name
