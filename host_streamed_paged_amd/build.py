"""Compile libkvs.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m host_streamed_paged_amd.build  (or __graft_entry__.build()).
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvs.so")

SOURCES = ["kvs_runtime.cpp", "kvs_kernels.hip", "kvs_decode.hip", "kvs_mfma.hip", "kvs_verify.hip", "kvs_prefill.hip", "kvs_append.hip"]

# Packed FP32 math is disabled for every HIP source: hipcc -O3 would otherwise
# form v_pk_* fp32 instructions on its own.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP toolchain is required to build libkvs.so")


def build(verbose: bool = False) -> str:
    cc = hipcc()
    objs = []
    build_dir = os.path.join(HERE, "_build")
    os.makedirs(build_dir, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *HIP_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c",
               os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".hip"):
            cmd.insert(1, "-x")
            cmd.insert(2, "hip")
        _run(cmd, verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = ("unknown target feature", "packed-fp32-ops")
    err = "\n".join(l for l in r.stderr.splitlines() if not any(n in l for n in noise))
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


if __name__ == "__main__":
    print(build(verbose=True))
