"""Build librse.so (the HIP library) in-tree with hipcc for gfx950.

Usage: python recommender_sparse_embedding_amd/build.py   (or __graft_entry__.build())
This file must stay importable without the package (it builds what the
package loads).
"""

from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "librse.so")
BUILD_DIR = os.path.join(ROOT, "_build")

ARCH = os.environ.get("RSE_OFFLOAD_ARCH", "gfx950")

# -ffp-contract=off: no fused multiply-adds, so the fp64 update arithmetic
# rounds exactly like the written expressions.  The packed-fp32 feature is
# disabled for all device code.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build librse.so)")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every csrc/*.hip for gfx950 and link librse.so (always rebuilds)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    srcs = sources()
    objs = [os.path.join(BUILD_DIR, os.path.basename(s) + ".o") for s in srcs]

    def compile_one(src_obj):
        src, obj = src_obj
        cmd = [cc, *HIPCC_FLAGS, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        return r.stderr

    jobs = jobs or min(8, os.cpu_count() or 1)
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        for err in ex.map(compile_one, zip(srcs, objs)):
            warn = [ln for ln in err.splitlines() if "warning" in ln and "packed-fp32" not in ln]
            if warn and verbose:
                print("\n".join(warn))
    tmp = OUT + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
