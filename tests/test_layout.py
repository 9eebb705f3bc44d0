"""Host check of the persistent MFMA kernels' block ranges and split-K
contribution layout (csrc/layout.cpp), compiled with the host C++ compiler."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gather_lora_matmul_amd", "csrc")


def test_layout_ranges_and_contributions(tmp_path):
    cxx = shutil.which("g++") or shutil.which("c++")
    if not cxx:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path / "layout_check")
    subprocess.run([cxx, "-O2", "-std=c++17", "-I" + CSRC, os.path.join(ROOT, "tests", "native", "layout_check.cpp"),
                    os.path.join(CSRC, "layout.cpp"), "-o", exe], check=True)
    r = subprocess.run([exe, "1500"], capture_output=True, text=True, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr


def test_device_planner_matches_host_planner(tmp_path):
    """The device planner (csrc/devplan.h), run sequentially on the host, against
    the host planner's grouping and tiles and the host layout without set-up term."""
    cxx = shutil.which("g++") or shutil.which("c++")
    inc = "/opt/rocm/include"
    if not cxx or not os.path.isdir(inc):
        pytest.skip("no host C++ compiler or ROCm headers")
    exe = str(tmp_path / "devplan_check")
    subprocess.run([cxx, "-O2", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I" + inc, "-I" + CSRC,
                    os.path.join(ROOT, "tests", "native", "devplan_check.cpp"),
                    os.path.join(CSRC, "layout.cpp"), "-o", exe], check=True)
    r = subprocess.run([exe, "400"], capture_output=True, text=True, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
