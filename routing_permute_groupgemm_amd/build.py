"""Build libmoe.so (HIP, gfx950) in-tree with hipcc: every source compiled to an
object in parallel, then one link."""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libmoe.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # keep the compiler from emitting packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)


def build_library(verbose: bool = False) -> str:
    """MOE_HIPCC_FLAGS (environment) adds compiler flags, e.g. -DMOE_GEMM_MFMA16=0 to build the down dgrad
    on 32x32x16 MFMAs for an A/B comparison of the same sources."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    inc = ["-I", os.path.join(ROOT, "include")] + os.environ.get("MOE_HIPCC_FLAGS", "").split()
    with tempfile.TemporaryDirectory(prefix="moe_build_") as tmpdir:
        objs, cmds = [], []
        for src in sources():
            obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
            objs.append(obj)
            cmds.append([hipcc, *HIPCC_FLAGS, *inc, "-c", src, "-o", obj])
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        with cf.ThreadPoolExecutor(max(1, min(len(cmds), os.cpu_count() or 1))) as ex:
            list(ex.map(_run, cmds))
        tmp = LIB + f".tmp{os.getpid()}"
        link = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        _run(link)
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
