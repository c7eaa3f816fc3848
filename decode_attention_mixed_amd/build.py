"""Build libmkv.so (HIP, gfx950) and the CPU-only metadata test library in-tree.

    python -m decode_attention_mixed_amd.build

Outputs (next to this file): libmkv.so, libmkv_hosttest.so.  Objects go to
_build/.  Every HIP source is compiled for gfx950 with packed-fp32 instructions
disabled; the cache-writing kernels (append, demote) are compiled with
-ffp-contract=off so their fp32 steps round exactly as written.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function",
]

# (source, extra flags)
LIB_SOURCES = [
    ("mkv_meta.cpp", []),
    ("mkv_api.cpp", []),
    ("kernels_quant.hip", ["-ffp-contract=off"]),
    ("kernels_partial.hip", ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mllvm", "-amdgpu-kernarg-preload-count=2"]),
    ("kernels_merge.hip", ["-mllvm", "-amdgpu-kernarg-preload-count=12"]),
    ("workspace.hip", []),
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r


def _compile(src, extra):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *HIP_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
    _run(cmd)
    return obj


def build_hip(verbose=False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(LIB_SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(*s), LIB_SOURCES))
    out = os.path.join(HERE, "libmkv.so")
    tmp = out + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


def build_host_test(verbose=False) -> str:
    """CPU-only metadata library for tests (host compiler, no HIP runtime)."""
    os.makedirs(BUILD, exist_ok=True)
    out = os.path.join(HERE, "libmkv_hosttest.so")
    cxx = shutil.which("g++") or "g++"
    _run([cxx, "-O1", "-g", "-std=c++17", "-shared", "-fPIC", "-D__HIP_PLATFORM_AMD__",
          "-I", INCLUDE, "-I", CSRC, "-I", os.path.join(ROCM, "include"),
          os.path.join(CSRC, "mkv_meta.cpp"), os.path.join(CSRC, "host_test_api.cpp"),
          "-o", out + ".tmp"])
    os.replace(out + ".tmp", out)
    if verbose:
        print("built", out)
    return out


def build_all(verbose=False):
    build_host_test(verbose)
    return build_hip(verbose)


if __name__ == "__main__":
    build_all(verbose=True)
    sys.exit(0)
