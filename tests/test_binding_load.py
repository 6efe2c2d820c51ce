"""The binding fails loudly instead of falling back: importing it without a built library,
or with a library built from other sources than those beside it, raises ImportError."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = "nvfp4_activation_quantization_amd"
LIB = os.path.join(ROOT, PKG, "libnvfp4act.so")


def copy_package(dst, with_library):
    os.makedirs(os.path.join(dst, PKG))
    shutil.copy(os.path.join(ROOT, PKG, "__init__.py"), os.path.join(dst, PKG))
    shutil.copytree(os.path.join(ROOT, PKG, "csrc"), os.path.join(dst, PKG, "csrc"))
    shutil.copytree(os.path.join(ROOT, "include"), os.path.join(dst, "include"))
    if with_library:
        shutil.copy(LIB, os.path.join(dst, PKG))


def import_error(root):
    code = "import sys; sys.path.insert(0, %r)\ntry:\n    import %s\nexcept ImportError as e:\n    print('IMPORTERROR', e)\n" % (root, PKG)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300, cwd=root)
    assert out.returncode == 0, out.stderr[-2000:]
    return out.stdout


def test_missing_library_raises(tmp_path):
    copy_package(str(tmp_path), with_library=False)
    out = import_error(str(tmp_path))
    assert "IMPORTERROR" in out and "not built" in out


@pytest.mark.skipif(not os.path.exists(LIB), reason="the library is not built")
def test_library_of_other_sources_raises(tmp_path):
    copy_package(str(tmp_path), with_library=True)
    with open(os.path.join(str(tmp_path), PKG, "csrc", "common.hpp"), "a") as f:
        f.write("\n// edited after the build\n")
    out = import_error(str(tmp_path))
    assert "IMPORTERROR" in out and "other sources" in out


@pytest.mark.skipif(not os.path.exists(LIB), reason="the library is not built")
def test_library_of_these_sources_loads(tmp_path):
    copy_package(str(tmp_path), with_library=True)
    out = import_error(str(tmp_path))
    assert "IMPORTERROR" not in out
