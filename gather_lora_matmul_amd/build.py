"""Build liblora_mi355x.so (hipcc, gfx950) in-tree.

    python gather_lora_matmul_amd/build.py      # (by path: importing the package loads the library)
    python gather_lora_matmul_amd/build.py --timeline
        # profiling build liblora_mi355x_timeline.so: the fused decode kernel
        # records a per-block timeline (lora_debug_block_timeline); load it
        # with LORA_MI355X_LIB=<path>
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "liblora_mi355x.so")
BUILD_DIR = os.path.join(HERE, "_build")
ARCH = os.environ.get("LORA_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
# Packed fp32 instructions are kept out of every kernel (the compiler is free to
# form them from plain float code otherwise).
COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument", "-I" + CSRC]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _compile(src: str, build_dir: str = BUILD_DIR, defines=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON + ["-D" + d for d in defines] + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    return obj


def build(verbose: bool = False, timeline: bool = False) -> str:
    build_dir = BUILD_DIR + ("_timeline" if timeline else "")
    lib = LIB.replace(".so", "_timeline.so") if timeline else LIB
    defines = ("LORA_BLOCK_TIMELINE",) if timeline else ()
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    jobs = min(len(srcs), max(1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda f: _compile(f, build_dir, defines), srcs))
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)
    return lib


if __name__ == "__main__":
    build(verbose=True, timeline="--timeline" in sys.argv[1:])
    sys.exit(0)
