"""Positive engagement: a fresh child process makes one call of every entry point under
rocprofv3 --kernel-trace, and the trace must hold exactly the library kernels each call
launches, in order -- one per static call, three per per-call (dynamic) form (four for the
FP8 LayerNorm: its scale kernel sits between the passes) -- so no call can have been served
by anything but the library's own kernels.  The RMSNorm + adaLN entries are also told apart
by their last template argument (the amax pass or the producer)."""
import csv
import glob
import json
import os
import shutil
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBRARY_KERNELS = ("quantize_kernel", "amax_x_kernel", "zero_amax_kernel", "rms_adaln_staged", "rms_adaln_general",
                   "swiglu_kernel", "residual_rms_kernel", "rms_silu_kernel", "ln_fp8_kernel",
                   "amax_to_fp8_scale_kernel")


def kernel_of(name):
    """(library kernel, 'amax' / 'producer' for the staged RMSNorm + adaLN kernel) or None."""
    if "nvfp4act" not in name:
        return None
    for base in LIBRARY_KERNELS:
        if ("::" + base + "(") in name or ("::" + base + "<") in name or name.startswith(base):
            if base == "rms_adaln_staged":
                args = name.split("rms_adaln_staged<", 1)[1].split(">", 1)[0].split(",")
                return [base, "amax" if args[-1].strip() == "true" else "producer"]
            return [base, None]
    return None


def test_every_entry_point_launches_its_own_kernels(tmp_path):
    prof = shutil.which("rocprofv3")
    if prof is None:
        pytest.skip("rocprofv3 is not installed")
    expected_path = tmp_path / "expected.json"
    cmd = [prof, "--kernel-trace", "--output-format", "csv", "-d", str(tmp_path / "trace"), "-o", "p", "--",
           sys.executable, os.path.join(ROOT, "tests", "engagement_calls.py"), str(expected_path)]
    print("engagement child:", " ".join(cmd), flush=True)
    r = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=100)
    # rocprofv3 itself may end with a segmentation fault after the program finished and the
    # results are written; the child's last line and the trace file decide
    assert "engagement calls done" in r.stdout, (r.returncode, r.stdout[-2000:], r.stderr[-2000:])
    traces = glob.glob(str(tmp_path / "trace" / "**" / "*kernel_trace.csv"), recursive=True)
    assert traces, r.stderr[-2000:]
    rows = []
    for path in traces:
        rows.extend(csv.DictReader(open(path)))
    rows.sort(key=lambda row: int(row["Start_Timestamp"]))
    got = [kv for kv in (kernel_of(row["Kernel_Name"]) for row in rows) if kv is not None]
    expected = json.load(open(expected_path))
    assert got == expected, "\n".join("%-40s %s" % (g, e) for g, e in zip(got + [None] * len(expected),
                                                                         expected + [None] * len(got)))
