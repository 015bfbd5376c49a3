"""Host check of the persistent attention launch arithmetic (CPU only):
builds tests/native/launch_plan_check.cpp with g++ (address and undefined
behaviour sanitizers on) against the library's launch_plan.h and runs it."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_launch_plan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = tmp_path / "launch_plan_check"
    subprocess.run([gxx, "-O1", "-std=c++17", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all",
                    "-I", os.path.join(ROOT, "vision_transformer_dynamic_region_amd", "csrc"),
                    os.path.join(ROOT, "tests", "native", "launch_plan_check.cpp"), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.startswith("ok")
