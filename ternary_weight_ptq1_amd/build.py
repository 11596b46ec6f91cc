"""Build the HIP library in-tree for gfx950 (hipcc cross-compiles without a GPU).

    python -m ternary_weight_ptq1_amd.build

compiles every ``csrc/*.hip`` / ``csrc/*.cpp`` into ``libptq1.so`` next to
this file.  Flags: -O3, gfx950 only, packed-FP32 VALU ops disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build", "ptq1")
LIB = os.path.join(PKG, "libptq1.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: the GEMM scales every block's partial with VALU
    # FMAs, which cannot read accumulation registers directly.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return path


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


SAN_DIR = os.path.join(ROOT, "_build", "sanitize")
SAN_LIB = os.path.join(SAN_DIR, "libptq1.so")


def build_sanitized(verbose: bool = False) -> str:
    """The same library with its host code (argument validation, workspace
    layout, launch planning: api.cpp) compiled by g++ under AddressSanitizer
    and UndefinedBehaviorSanitizer, linked with the GPU objects of build().
    Loaded by the binding when PTQ1_LIB names it; for host-only test runs
    (the sanitizers instrument no GPU code)."""
    build()
    os.makedirs(SAN_DIR, exist_ok=True)
    obj = os.path.join(SAN_DIR, "api.cpp.o")
    cmd = ["g++", "-std=c++17", "-O1", "-fPIC", "-Wall", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-I",
           os.path.join(ROOT, "include"), "-I", CSRC, "-c", os.path.join(CSRC, "api.cpp"), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    gpu_objs = [os.path.join(BUILD_DIR, os.path.basename(src) + ".o") for src in sources() if not src.endswith(".cpp")]
    cmd = ["g++", "-shared", "-fsanitize=address,undefined", "-o", SAN_LIB, obj, *gpu_objs, "-L/opt/rocm/lib",
           "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


if __name__ == "__main__":
    import sys

    if "--sanitize" in sys.argv:
        build_sanitized(verbose=True)
    else:
        build(verbose=True)
