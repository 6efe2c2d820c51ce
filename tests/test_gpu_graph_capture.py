"""The library's first call in a process can be captured into a HIP graph: no compute entry
point waits on the device or touches the null stream (the SiLU tables are part of the code
object).  Runs tests/graph_first_call.py in a fresh process, so that its captured
swiglu_nvfp4 call really is the first."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_first_call_captured_into_a_graph_replays_like_eager_calls():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "graph_first_call.py")], cwd=ROOT,
                       capture_output=True, text=True, timeout=100)
    assert r.returncode == 0 and "graph replays match" in r.stdout, (r.returncode, r.stdout[-3000:], r.stderr[-3000:])
