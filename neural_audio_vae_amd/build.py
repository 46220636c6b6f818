"""Build the mh3a HIP library in-tree for gfx950.

    python -m neural_audio_vae_amd.build

compiles csrc/*.hip and csrc/*.cpp with hipcc into
neural_audio_vae_amd/libmh3a.so (always recompiles).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libmh3a.so")
SOURCES = [os.path.join(PKG, "csrc", f) for f in ("mh3a_host.cpp", "mh3a_plan.cpp", "mh3a_kernels.hip")]
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the mh3a library needs the ROCm toolchain")


def build(verbose=False):
    tmp = LIB + ".tmp"
    cmd = [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # keep the compiler from emitting packed fp32 VALU ops
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
        "-o", tmp,
    ] + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libmh3a.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
