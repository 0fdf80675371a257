"""Builds libmuon_ns.so in-tree with hipcc for gfx950.

    python -m muon_newton_schulz_06_amd.build

Every HIP source is compiled with packed-fp32 instruction selection turned
off and the result is linked as one shared library next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmuon_ns.so")
SOURCES = ["gemm_axpy.hip", "gemm_sq.hip", "gemm_final.hip", "gemm_syrk.hip", "elementwise.hip",
           "select.hip", "noalloc.hip", "plan.cpp", "api.cpp"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm under /opt/rocm)")


def flags():
    return [
        "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-mcode-object-version=5",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-pass-failed", "-I", os.path.join(os.path.dirname(HERE), "include"),
    ]


def build(verbose: bool = False) -> str:
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="muon_build_") as tmp:
        def compile_one(src):
            obj = os.path.join(tmp, src + ".o")
            cmd = [cc, *flags(), "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
            return obj
        # one compiler process per source, at most six at once
        with ThreadPoolExecutor(max_workers=min(6, len(SOURCES))) as ex:
            objs = list(ex.map(compile_one, SOURCES))
        out_tmp = LIB + ".tmp"
        cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", out_tmp, *objs]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stderr}")
        os.replace(out_tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
