"""Host check of the invariant-divisor constants the kernels use for index
arithmetic (CPU only): builds tests/native/fastdiv_check.cpp with g++ against
the library's fastdiv.h and runs it."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_fastdiv_exact(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = tmp_path / "fastdiv_check"
    subprocess.run([gxx, "-O2", "-std=c++17", "-fsanitize=address,undefined",
                    "-I", os.path.join(ROOT, "vision_transformer_dynamic_region_amd", "csrc"),
                    os.path.join(ROOT, "tests", "native", "fastdiv_check.cpp"), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.startswith("ok")
