"""Build the HIP library in-tree with hipcc for gfx950 (explicit commands, no JIT cache)."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmi355emb.so")
ARCH = "gfx950"

# Packed fp32 instructions are kept out of all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}):\n{' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False) -> str:
    """Compile every source and link libmi355emb.so next to this file; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    k_obj = os.path.join(BUILD, "emb_kernels.o")
    h_obj = os.path.join(BUILD, "emb_host.o")
    _run([hipcc, "-x", "hip", f"--offload-arch={ARCH}", *COMMON, *DEVICE_FLAGS, "-c",
          os.path.join(CSRC, "emb_kernels.hip"), "-o", k_obj], verbose)
    _run([hipcc, "-x", "c++", *COMMON, "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__", "-c",
          os.path.join(CSRC, "emb_host.cpp"), "-o", h_obj], verbose)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, k_obj, h_obj,
          "-lpthread"], verbose)
    os.replace(tmp, LIB)
    return LIB


SAN_LIB = os.path.join(BUILD, "san", "libmi355emb_san.so")


def build_sanitized(verbose: bool = False) -> str:
    """The host runtime built with AddressSanitizer and UndefinedBehaviorSanitizer (host code only,
    compiled by g++; the kernels object is the regular build's), linked into SAN_LIB.  The CPU
    tests load it in a process started with the ASan runtime preloaded.  Returns its path."""
    k_obj = os.path.join(BUILD, "emb_kernels.o")
    if not os.path.exists(k_obj):
        build(verbose)
    d = os.path.dirname(SAN_LIB)
    os.makedirs(d, exist_ok=True)
    h_obj = os.path.join(d, "emb_host_san.o")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer"]
    _run(["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-Wall", *san, "-I", os.path.join(ROOT, "include"),
          "-I", CSRC, "-I", os.path.join(rocm, "include"), "-D__HIP_PLATFORM_AMD__", "-c",
          os.path.join(CSRC, "emb_host.cpp"), "-o", h_obj], verbose)
    tmp = SAN_LIB + ".tmp"
    _run(["g++", "-shared", "-fPIC", *san[:1], "-o", tmp, k_obj, h_obj,
          "-L", os.path.join(rocm, "lib"), "-Wl,-rpath," + os.path.join(rocm, "lib"), "-lamdhip64",
          "-lpthread"], verbose)
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    if "--sanitized" in sys.argv:
        print(build_sanitized(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
