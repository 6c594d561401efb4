"""Build libpa_decode.so (gfx950) in-tree with hipcc.

    python -m decode_attention_paged_amd.build [--verbose]

Every HIP source under csrc/ is compiled for gfx950 only and linked into
decode_attention_paged_amd/libpa_decode.so next to this file.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libpa_decode.so")
BUILD_DIR = os.path.join(HERE, "_build")
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
    # packed fp32 VALU forms stay off (they are generated from scalar code otherwise)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]

SOURCES = ["pa_api.hip", "pa_mha.hip", "pa_gqa.hip", "pa_mla.hip", "pa_reduce.hip", "pa_append.hip"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out:
        print(out, flush=True)


def build(verbose: bool = False, save_temps: bool = False) -> str:
    """Compile every source and link the shared library; return its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    objs = []

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if save_temps:
            cmd += ["-save-temps=obj"]
        _run(cmd, verbose)
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv, save_temps="--save-temps" in sys.argv))
