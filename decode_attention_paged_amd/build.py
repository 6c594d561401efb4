"""Build libpa_decode.so (gfx950) in-tree with hipcc.

    python -m decode_attention_paged_amd.build [--verbose]

Every HIP source under csrc/ is compiled for gfx950 only and linked into
decode_attention_paged_amd/libpa_decode.so next to this file.
"""

from __future__ import annotations

import os
import re
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

SOURCES = ["pa_api.hip", "pa_mha.hip", "pa_gqa.hip", "pa_sched.hip", "pa_mla.hip", "pa_reduce.hip",
           "pa_append.hip", "pa_probe.hip"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    lines = [l for l in (r.stdout + r.stderr).splitlines()
             if "packed-fp32-ops" not in l and l.strip()]
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n" + "\n".join(lines))
    remarks = [l for l in lines if "kernel-resource-usage" in l]
    other = [l for l in lines if "kernel-resource-usage" not in l]
    if verbose and other:
        print("\n".join(other), flush=True)
    return remarks


def resource_usage(remarks):
    """Per-kernel figures from the compiler's kernel-resource-usage remarks:
    {kernel: {"VGPRs": n, "AGPRs": n, "ScratchSize": n, "VGPRs Spill": n, ...}}."""
    usage, name = {}, None
    for line in remarks:
        m = re.search(r"remark:\s+Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            usage[name] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\d+)", line)
        if m and name is not None:
            usage[name][m.group(1).strip()] = int(m.group(2))
    return usage


def check_usage(usage):
    """Refuse kernels that spill vector registers or use scratch memory.

    The kernels count their own vector-memory waits around asm loads (the
    latent kernels) and size their register tiles to the register file; a
    spill adds memory operations the hand-counted waits do not know about,
    and scratch traffic the bandwidth figures do not account for.
    """
    bad = {k: v for k, v in usage.items()
           if v.get("ScratchSize", 0) > 0 or v.get("VGPRs Spill", 0) > 0}
    if bad:
        raise RuntimeError("kernels spill or use scratch: " +
                           "; ".join(f"{k}: {v}" for k, v in sorted(bad.items())))


def build(verbose: bool = False, save_temps: bool = False) -> str:
    """Compile every source and link the shared library; return its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    objs = []

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *COMMON_FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c",
               os.path.join(CSRC, src), "-o", obj]
        if save_temps:
            cmd += ["-save-temps=obj"]
        return obj, _run(cmd, verbose)

    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(compile_one, SOURCES))
    objs = [o for o, _ in results]
    usage = {}
    for _, remarks in results:
        usage.update(resource_usage(remarks))
    if not usage:
        raise RuntimeError("the compiler reported no kernel resource usage")
    check_usage(usage)
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv, save_temps="--save-temps" in sys.argv))
