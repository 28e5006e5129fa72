"""Build libspecverify.so (HIP, gfx950) in place with hipcc.

Usage: python -m device_draft_verification_specverify_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCE = os.path.join(HERE, "csrc", "specverify.hip")
HOST_SOURCES = [os.path.join(HERE, "csrc", "bandit.cpp")]
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(HERE, "libspecverify.so")
# The same sources with device-side index checks (-DSV_DEVICE_CHECKS): a debug
# build for running the GPU tests with every work unit's indices checked.
CHECKED_LIBRARY = os.path.join(HERE, "libspecverify_checked.so")
ARCH = "gfx950"

# Packed FP32 instructions stay off: the compiler must not form them.
# Machine-level loop-invariant code motion stays off too: it hoists per-thread
# addresses and constants out of the streaming loops into registers that stay
# live across them (about 20 extra VGPRs in the streaming kernel). Private
# arrays are not moved to LDS: that costs occupancy instead of registers.
HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-disable-machine-licm",
    "-mllvm", "-disable-promote-alloca-to-lds",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def build(verbose: bool = False, extra_flags: list[str] | None = None,
          checked: bool = False) -> str:
    """Compile the HIP source into LIBRARY, or CHECKED_LIBRARY with the device-side
    index checks (always recompiles). Returns the path."""
    out = CHECKED_LIBRARY if checked else LIBRARY
    tmp = out + ".tmp"
    flags = [*HIP_FLAGS, *(extra_flags or []), *(["-DSV_DEVICE_CHECKS"] if checked else [])]
    cmd = [hipcc(), *flags, "-I", INCLUDE, SOURCE, *HOST_SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    if verbose and res.stderr.strip():
        print(res.stderr, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True, checked="--checked" in sys.argv[1:]))
