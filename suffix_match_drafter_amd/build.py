"""Build libsfx.so (gfx950) in-tree with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SO = os.path.join(HERE, "libsfx.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 instructions stay off for every HIP code object of this library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip"))) + \
        [os.path.join(HERE, "csrc", "sfx_api.cpp"), os.path.join(HERE, "csrc", "corpus_file.cpp")]


def build(force: bool = True, verbose: bool = False) -> str:
    if not force and os.path.exists(SO):
        return SO
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-o", SO + ".tmp",
           *sources(), "-lpthread"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(SO + ".tmp", SO)
    return SO


if __name__ == "__main__":
    build(force=True, verbose="-v" in sys.argv)
    print(SO)
