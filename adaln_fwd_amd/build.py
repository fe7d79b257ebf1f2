"""Compile the HIP sources into ``adaln_fwd_amd/libadaln.so`` for gfx950.

Cross-compiles on a machine without a GPU.  Always recompiles: each source
to an object file (in parallel, in a private temporary directory), then one
link.  Every kernel is launched from the source that defines it, so no
relocatable device code is needed."""

from __future__ import annotations

import glob
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libadaln.so")
SOURCES = sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    f"--offload-arch={ARCH}",
    # packed-fp32 instructions stay off (hipcc's host pass warns it does not
    # know the feature; that warning is harmless)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                         text=True)
    out = "\n".join(l for l in res.stdout.splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out, file=sys.stderr)


def _jobs() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(8, n, len(SOURCES)))


def build(verbose: bool = False) -> str:
    with tempfile.TemporaryDirectory(prefix="adaln_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(s) + ".o")
                for s in SOURCES]
        with ThreadPoolExecutor(_jobs()) as ex:
            list(ex.map(lambda so: _run([hipcc(), *FLAGS, "-c", so[0], "-o",
                                         so[1]], verbose),
                        zip(SOURCES, objs)))
        tmp = LIB + ".tmp"
        _run([hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs,
              "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
