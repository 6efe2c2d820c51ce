"""The oracle pins again, against the oracle built with AddressSanitizer and
UndefinedBehaviorSanitizer (host code only), in a child process with the ASan runtime
preloaded: an out-of-bounds access, a use of freed memory or an undefined operation
anywhere in the C oracle the pins reach fails the run."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=%s" % name], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(bool(os.environ.get("LD_PRELOAD")), reason="the environment already preloads a library")
def test_oracle_pins_under_address_and_undefined_sanitizers(tmp_path):
    asan = runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = oracle.build_sanitized(str(tmp_path / "liboracle_san.so"))
    env = dict(os.environ)
    env.update(NVFP4_ORACLE_LIB=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle_pins.py"), "-x", "-q",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out, out[-2000:]


@pytest.mark.skipif(bool(os.environ.get("LD_PRELOAD")), reason="the environment already preloads a library")
def test_the_sanitized_build_reports_an_out_of_bounds_write(tmp_path):
    """Control: a call whose output buffer is two elements short is caught in the child."""
    asan = runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = oracle.build_sanitized(str(tmp_path / "liboracle_san.so"))
    env = dict(os.environ)
    env.update(NVFP4_ORACLE_LIB=lib, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0")
    code = ("import numpy as np, oracle\n"
            "x = np.zeros(64, np.float32); out = np.zeros(62, np.uint16)\n"
            "oracle._load().orc_bf16_round(x.ctypes.data, out.ctypes.data, 64)\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]
