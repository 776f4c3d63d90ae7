"""Build libhisparse.so (the C-ABI HIP library) in-tree with hipcc for gfx950."""

from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libhisparse.so")
LIB_SANITIZED = os.path.join(PKG, "libhisparse_sanitized.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # Packed fp32 instructions stay off (no floating point here, but the rule
    # is global for this code base). The device pass honours the feature
    # (tests/test_build_flags.py checks the generated gfx950 code); the host
    # pass does not know it and warns, harmlessly.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]

# Host-side AddressSanitizer and UndefinedBehaviorSanitizer for the library's
# host code (argument checks, plans, launches); device code is not
# instrumented. Each -fsanitize option goes to the host pass only.
SANITIZE_FLAGS = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined".split() + [
    "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, sanitize: bool = False, out: str = "") -> str:
    """Compile every HIP source into one shared library and return its path.
    With ``sanitize`` the host code is instrumented (SANITIZE_FLAGS) and the
    library goes to ``out`` or LIB_SANITIZED; a process loading it needs
    clang's ASan runtime preloaded (``tests/test_sanitizers.py`` does this)."""
    lib = out or (LIB_SANITIZED if sanitize else LIB)
    tmp = lib + ".tmp"
    cmd = [HIPCC, *FLAGS, *(SANITIZE_FLAGS if sanitize else []), "-I", INCLUDE, "-I", CSRC,
           *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
