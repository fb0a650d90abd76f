"""Compile the HIP sources into the package's ``libkvq.so`` for gfx950.

Run as ``python -m quantized_decode_attention_keys_amd.build`` or through
``build()``; it always recompiles (sources in parallel, then one link).
hipcc cross-compiles without a GPU.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libkvq.so")
SOURCES = ["kvq_host.cpp", "kvq_kernels.hip", "kvq_attend_d64.hip", "kvq_attend_d128.hip",
           "kvq_geometry.hip", "kvq_fp8.hip", "kvq_scratch.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions stay off everywhere in this library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
]


def build(verbose: bool = False) -> str:
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    with tempfile.TemporaryDirectory() as tmp:
        procs, objs = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            cmd = [HIPCC, *FLAGS, *inc, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd)))
            objs.append(obj)
        failed = [src for src, p in procs if p.wait() != 0]
        if failed:
            raise RuntimeError(f"hipcc failed on {failed}")
        out = LIB + ".tmp"
        subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs,
                               "-o", out])
    os.replace(out, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
