"""Build libpagedattn.so for gfx950 with hipcc, in the package directory.

Usage: ``python -m attention_paged_kv_varlen_amd.build`` (or ``build()``).  Every
call recompiles.  The packed-FP32 target feature is switched off for the device
code (ordinary float code only); the host-only sources (planner, C ABI) are
compiled as plain C++ without it.  The same call builds ``chip_probe``, a
stand-alone measurement program (csrc/chip_probe.hip) that shares no code with
the library.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libpagedattn.so")
PROBE = os.path.join(PKG, "chip_probe")
ARCH = os.environ.get("PA_OFFLOAD_ARCH", "gfx950")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

SOURCES = ["kernels.hip", "noalloc.hip", "planner.cpp", "api.cpp"]
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    """Compile every source and link libpagedattn.so; returns its path."""
    cc = hipcc()
    tmp = tempfile.mkdtemp(prefix="pagedattn_build_")
    try:
        objs = []
        for src in SOURCES:
            path = os.path.join(CSRC, src)
            obj = os.path.join(tmp, src + ".o")
            if src.endswith(".hip"):
                lang = ["-x", "hip", f"--offload-arch={ARCH}", *DEVICE_FLAGS]
            else:  # host code only: no device pass, so no device-only flags
                lang = ["-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include")]
            cmd = [cc, *lang, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
                   "-I", os.path.join(ROOT, "include"), "-c", path, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.run(cmd, check=True)
            objs.append(obj)
        out_tmp = LIB + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out_tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(out_tmp, LIB)
        probe_tmp = PROBE + ".tmp"
        cmd = [cc, "-x", "hip", f"--offload-arch={ARCH}", *DEVICE_FLAGS, "-O3", "-std=c++17", "-Wall",
               os.path.join(CSRC, "chip_probe.hip"), "-o", probe_tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(probe_tmp, PROBE)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
