"""Build the HIP library ``libspecverify.so`` in-tree for gfx950."""

from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "specverify.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libspecverify.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# host code only: AddressSanitizer and UndefinedBehaviorSanitizer on the host
# layer (argument checks, workspace layout, launch set-up); the device code is
# built as usual
SANITIZE_FLAGS = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-omit-frame-pointer -g".split()


def build_library(verbose: bool = False, out: str = LIB, sanitize: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, *(SANITIZE_FLAGS if sanitize else []), "-I" + INCLUDE, SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    import sys

    if "--sanitize" in sys.argv:
        print(build_library(verbose=True, out=sys.argv[sys.argv.index("--sanitize") + 1], sanitize=True))
    else:
        print(build_library(verbose=True))
