"""Build the HIP library ``libpa_kv.so`` in-tree with hipcc for gfx950.

Usage: ``python -m paged_kv_attention_13_amd.build`` (also called by the
repository's ``__graft_entry__.build()``).  Always recompiles.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libpa_kv.so"
ARCH = os.environ.get("PA_OFFLOAD_ARCH", "gfx950")

# Packed-FP32 VALU forms are disabled for the device code: the kernels are
# written for scalar/dot2 arithmetic and must not be re-vectorised into them.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


CHECKED_LIB_NAME = "libpa_kv_checked.so"


def build(verbose: bool = False, checked: bool = False) -> str:
    """Build the library; with ``checked``, the debug build whose kernels check the device
    metadata at each use (PA_DEVICE_CHECKS=1), as ``libpa_kv_checked.so``."""
    out = os.path.join(PKG, CHECKED_LIB_NAME if checked else LIB_NAME)
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC, *DEVICE_FLAGS,
           *(["-DPA_DEVICE_CHECKS=1"] if checked else []), *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(x for x in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in x)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{msgs}")
    if msgs.strip() and verbose:
        print(msgs)
    os.replace(tmp, out)
    return out


HOST_SOURCES = ("pa_host.cpp", "pa_api.cpp", "pa_runtime.cpp", os.path.join("host_only", "launch_stubs.cpp"))
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def build_host_only(out_dir: str = None, sanitize: bool = True) -> str:
    """The library's host code (argument checks, plans, metadata checkers, block manager,
    scheduler) built with g++ as a shared library of the same ABI, every kernel launch
    replaced by a "no device" error; with ``sanitize``, under AddressSanitizer and
    UndefinedBehaviorSanitizer.  Returns the path of the built library."""
    out_dir = out_dir or os.path.join(ROOT, "_build")
    os.makedirs(out_dir, exist_ok=True)
    out = os.path.join(out_dir, "libpa_host_san.so" if sanitize else "libpa_host.so")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-Wall", "-Wno-unused-function",
           *(SANITIZE if sanitize else []), "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, f) for f in HOST_SOURCES], "-o", out + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"g++ failed ({r.returncode}):\n{r.stdout}{r.stderr}")
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, checked="--checked" in sys.argv))
