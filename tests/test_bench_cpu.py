"""bench.py on the CPU: its helpers are present and importable, `--gpus N` with N > 1 exits
with a message before touching a GPU, the CPU share and CPU model are read, and the
oracle baseline runs on a small workload."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


def test_helpers_present():
    for name in ("parse", "cpu_share", "stream_ceiling", "kernel_source_digest", "measured_traffic", "make_inputs",
                 "make_step", "main", "cpu_baseline", "cpu_model"):
        assert callable(getattr(bench, name)), name


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and not r.stdout


def test_cpu_share_and_model():
    avail, quota = bench.cpu_share()
    assert avail >= 1 and (quota is None or quota >= 1)
    assert "family" in bench.cpu_model()


def test_cpu_baseline_on_the_tiny_workload():
    wl = workloads.get("rms_adaln_256x2048")
    out = bench.cpu_baseline(wl, workloads.calibration_amax(wl.name), wl.m, np)
    assert out["kind"] == "oracle" and out["threads"] >= 1 and out["value"] > 0 and out["single_thread_seconds"] > 0
