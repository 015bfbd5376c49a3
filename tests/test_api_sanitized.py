"""The C-ABI front end built for the host alone under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

The front end (bra_api.cpp) and its host helpers (host_plan.cpp) are
compiled with the sanitizers, linked with stand-ins for the kernel launchers
(tests/native/api_stubs.cpp) and with tests/native/api_check.cpp, and run:
each entry point is called with arguments it must reject, so the argument
checks, the workspace arithmetic and the error text run under the
sanitizers.  No call passes validation; a stand-in that is reached fails
the check.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "vision_transformer_dynamic_region_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_api_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")):
        pytest.skip("g++ or the HIP headers not available")
    exe = str(tmp_path / "api_check")
    # host code only: the HIP headers for the runtime types, no device code
    subprocess.run([gxx, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROCM, "include"), "-I", CSRC,
                    os.path.join(CSRC, "bra_api.cpp"), os.path.join(CSRC, "host_plan.cpp"),
                    os.path.join(ROOT, "tests", "native", "api_stubs.cpp"),
                    os.path.join(ROOT, "tests", "native", "api_check.cpp"),
                    "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                    "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    out = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.startswith("ok"), out.stdout
