"""Host-only build of the C ABI layer under AddressSanitizer and UndefinedBehaviorSanitizer.

    python level_pooled_kv_amd/build_hostcheck.py

Compiles psa_api.cpp (argument validation, derived sizes, workspace layout) with g++ and
the sanitizers, with csrc/psa_host_stubs.cpp standing in for the device launchers, into
_build/libpsa_hostcheck.so. The binding loads it instead of libpsa.so when PSA_LIBRARY
names it; run the host ABI tests that way with the sanitizer runtime preloaded (see
tests/test_host_sanitizer.py). No device code is built here.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(BUILD, "libpsa_hostcheck.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SANITIZERS = "address,undefined"


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           f"-fsanitize={SANITIZERS}", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, "-Wall", "-Wno-unused-function",
           os.path.join(CSRC, "psa_api.cpp"), os.path.join(CSRC, "psa_host_stubs.cpp"),
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"host-check build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {LIB}", flush=True)
    return LIB


def asan_runtime() -> str:
    """Path of the AddressSanitizer runtime g++ links against (for LD_PRELOAD)."""
    return subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()


if __name__ == "__main__":
    build()
    sys.exit(0)
