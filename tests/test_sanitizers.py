"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Builds with the host compilers, with -fsanitize=address,undefined and no
recovery, and runs:
  * the fp64 oracle's C entry points (tests/native/oracle_check.c);
  * the block-range layout of the MFMA kernels (layout.cpp with
    tests/native/layout_check.cpp);
  * the device planner run on the host (devplan.h with
    tests/native/devplan_check.cpp);
  * the library's host paths -- pool, page table, planner, launch-shape
    preparation, argument checks (pool.cpp, plan.cpp, api.cpp, layout.cpp with
    tests/native/host_check.cpp, kernels stubbed out: host-only pools never
    launch one).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gather_lora_matmul_amd", "csrc")
NATIVE = os.path.join(ROOT, "tests", "native")
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")
ROCM_INC = "/opt/rocm/include"


def _run(cmd, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout, env=ENV)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-4000:], r.stderr[-6000:])
    return r.stdout


def test_oracle_under_sanitizers(tmp_path):
    cc = shutil.which("gcc")
    if not cc:
        pytest.skip("no gcc")
    exe = str(tmp_path / "oracle_check")
    _run([cc, "-std=c99", "-fopenmp", "-ffp-contract=off"] + SAN +
         [os.path.join(NATIVE, "oracle_check.c"), os.path.join(ROOT, "oracle", "lora_oracle.c"),
          "-lm", "-o", exe])
    print(_run([exe]))


def test_layout_under_sanitizers(tmp_path):
    cxx = shutil.which("g++")
    if not cxx:
        pytest.skip("no g++")
    exe = str(tmp_path / "layout_check")
    _run([cxx, "-std=c++17", "-I" + CSRC] + SAN +
         [os.path.join(NATIVE, "layout_check.cpp"), os.path.join(CSRC, "layout.cpp"), "-o", exe])
    print(_run([exe, "300"]))


def test_device_planner_under_sanitizers(tmp_path):
    cxx = shutil.which("g++")
    if not cxx or not os.path.isdir(ROCM_INC):
        pytest.skip("no g++ or ROCm headers")
    exe = str(tmp_path / "devplan_check")
    _run([cxx, "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I" + ROCM_INC, "-I" + CSRC] + SAN +
         [os.path.join(NATIVE, "devplan_check.cpp"), os.path.join(CSRC, "layout.cpp"), "-o", exe])
    print(_run([exe, "150"]))


def test_host_library_paths_under_sanitizers(tmp_path):
    cxx = shutil.which("g++")
    if not cxx or not os.path.isdir(ROCM_INC):
        pytest.skip("no g++ or ROCm headers")
    libdir = "/opt/rocm/lib"
    exe = str(tmp_path / "host_check")
    srcs = [os.path.join(CSRC, f) for f in ("pool.cpp", "plan.cpp", "api.cpp", "layout.cpp")]
    _run([cxx, "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I" + ROCM_INC, "-I" + CSRC] + SAN +
         [os.path.join(NATIVE, "host_check.cpp")] + srcs +
         ["-L" + libdir, "-Wl,-rpath," + libdir, "-lamdhip64", "-o", exe])
    print(_run([exe, "25"]))
