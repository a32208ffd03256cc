"""Build libiqd.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Flags that the numerics depend on:
  -ffp-contract=off                      no fused multiply-add contraction
  -fno-fast-math                         IEEE semantics, correctly rounded '/'
  -fno-gpu-flush-denormals-to-zero       keep fp32 subnormals
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                         no packed fp32 VALU instructions
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libiqd.so")
ARCH = "gfx950"

SOURCES = ["abi.cpp", "quantize.hip", "w8a8_matvec.hip", "w8a8_mfvec.hip", "w8a8_mfma.hip", "blockq8_matvec.hip", "blockq8_mfvec.hip",
           "lm_head.hip", "requant.hip", "attention.hip", "fp8.hip", "ceiling.hip", "static_scratch.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result", "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source to an object in parallel, then link libiqd.so."""
    bdir = os.path.join(HERE, "_build")
    os.makedirs(bdir, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [HIPCC, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        if len([p for _, p in procs if p.poll() is None]) >= jobs:
            procs[0][1].wait()
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        if out.strip():
            print(out, file=sys.stderr)
        if p.returncode != 0:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
