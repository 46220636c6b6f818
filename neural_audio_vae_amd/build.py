"""Build the mh3a HIP library in-tree for gfx950.

    python -m neural_audio_vae_amd.build

compiles csrc/*.hip and csrc/*.cpp with hipcc, one process per source (the
conv kernel's tile shapes sit in translation units of their own so that
they compile in parallel), and links neural_audio_vae_amd/libmh3a.so.
Always recompiles.
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmh3a.so")
OBJ = os.path.join(PKG, "_build")
ARCH = "gfx950"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the mh3a library needs the ROCm toolchain")


def compile_flags(defines=()):
    return [f"-D{d}" for d in defines] + [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # keep the compiler from emitting packed fp32 VALU ops (the host
        # pass warns that it does not know the feature; only the device
        # pass acts on it)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    ]


def _compile(src, verbose, defines=(), obj_dir=OBJ):
    obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
    cmd = [hipcc()] + compile_flags(defines) + ["-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    return src, obj, res


def build(verbose=False, jobs=None, defines=(), out=LIB, only=None):
    """Compile every source (or only those named in `only`, taking the other
    objects from the last full build) with optional -D defines (the
    documented build-time options) and link `out`."""
    obj_dir = OBJ if not defines else os.path.join(OBJ, "_".join(d.replace("=", "") for d in defines))
    os.makedirs(obj_dir, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(16, os.cpu_count() or 1)
    failed = []
    # the largest translation units first
    order = sorted(srcs, key=lambda s: -os.path.getsize(s))
    todo = [s for s in order if only is None or os.path.basename(s) in only]
    objs = [os.path.join(OBJ, os.path.basename(s) + ".o") for s in order if s not in todo]
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for src, obj, res in ex.map(lambda s: _compile(s, verbose, defines, obj_dir), todo):
            if res.returncode != 0:
                failed.append((src, res))
            objs.append(obj)
    if failed:
        for src, res in failed:
            sys.stderr.write(f"--- {os.path.basename(src)}\n" + res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libmh3a.so")
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + sorted(objs)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("linking libmh3a.so failed")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
