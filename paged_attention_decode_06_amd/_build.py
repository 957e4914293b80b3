"""Compile the HIP library for gfx950 (hipcc cross-compiles; no GPU needed)."""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "pa_decode.hip")
SOURCES = [SRC, os.path.join(HERE, "csrc", "pa_prefill.hip"), os.path.join(HERE, "csrc", "pa_moe.hip"),
           os.path.join(HERE, "csrc", "pa_probe.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpa_decode.so")
ARCH = "gfx950"

# Packed fp32 VALU forms are switched off for all device code.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def build(verbose: bool = False, extra_flags: list[str] | None = None, out: str = LIB) -> str:
    """Build libpa_decode.so next to this file and return its path."""
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, *(extra_flags or []), "-I", INCLUDE, *SOURCES, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (res.stdout + res.stderr).splitlines()
            if "packed-fp32-ops" not in l and "is not a recognized feature" not in l]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
