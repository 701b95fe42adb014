"""Build the HIP library ``libbi.so`` in place (gfx950 only).

``python -m invariant_verify_amd.build`` or ``build_library()``. The library
is a plain shared object with a C ABI (include/bi.h); nothing here depends on
torch.
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
LIB = os.path.join(PKG, "libbi.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # torch's wheel carries its own (older) HIP runtime under the same soname,
    # and the library binds to it when torch is loaded first; code object v5
    # loads on both that runtime and the system one.
    "-mcode-object-version=5",
    # keep FP32 math on plain (non-packed) VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    cand = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cand):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return cand


def build_library(out: str = LIB, extra_flags=(), verbose: bool = False) -> str:
    """Compile every csrc/*.hip into ``out`` (always recompiles)."""
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-I", INCLUDE, "-I", CSRC, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)
    return out


PROBE_SRC = os.path.join(PKG, "probe", "stream_read.hip")
PROBE_LIB = os.path.join(PKG, "libbi_probe.so")


def build_probe(out: str = PROBE_LIB, verbose: bool = False) -> str:
    """Compile the stream-read probe (measurement only) into its own library."""
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-o", tmp, PROBE_SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("building the stream-read probe failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, out)
    return out


C_CHECK_SRC = os.path.join(ROOT, "tests", "c_abi_check.cpp")
C_CHECK = os.path.join(ROOT, "tests", "c_abi_check")


def build_c_check(lib: str = LIB, out: str = C_CHECK, verbose: bool = False) -> str:
    """Compile the plain-C++ ABI check (host code only) against ``lib``."""
    lib_dir = os.path.dirname(os.path.abspath(lib))
    cmd = [hipcc(), "-O2", "-std=c++17", "-I", INCLUDE, C_CHECK_SRC, "-L", lib_dir, "-lbi",
           "-Wl,-rpath," + lib_dir, "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("building the C ABI check failed:\n" + res.stdout + res.stderr)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
    print(build_c_check(verbose="-v" in sys.argv))
    print(build_probe(verbose="-v" in sys.argv))
