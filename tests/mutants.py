"""Build and call the test-only faulty candidate kernel (csrc/mutant_linear.hip).

`build()` compiles it for gfx950 into csrc/libmutant.so; `linear()` runs it on
device tensors.  It is a second kernel behind the same interface as the
library's W8A8 linear, with one epilogue fault of the conformance catalogue
switched in (0 = none, 1..5 = F1..F5).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc", "mutant_linear.hip")
LIB = os.path.join(HERE, "csrc", "libmutant.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FAULT_CODES = {"null": 0, "F1": 1, "F2": 2, "F3": 3, "F4": 4, "F5": 5}

_lib = None


def build() -> str:
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17", "-fPIC", "-shared",
           "-ffp-contract=off", "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-x", "hip", SRC, "-o", tmp]
    subprocess.run(cmd, check=True, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is not built (run __graft_entry__.build())")
        lib = ctypes.CDLL(LIB)
        lib.mutant_linear.restype = ctypes.c_int
        lib.mutant_linear.argtypes = [ctypes.c_int] + [ctypes.c_void_p] * 4 + [ctypes.c_int64] * 3 + \
            [ctypes.c_void_p] * 3
        _lib = lib
    return _lib


def linear(fault: str, q, s_a, w, s_w, with_acc: bool = True):
    """Candidate arm on the GPU: q int8 [b, K], s_a fp32 [b], w int8 [N, K],
    s_w fp32 [N] (contiguous cuda tensors).  Returns (y bf16 [b, N], acc int32
    [b, N] or None)."""
    import torch

    lib = _load()
    for t in (q, s_a, w, s_w):
        assert t.is_cuda and t.is_contiguous()
    b, K = q.shape
    N = w.shape[0]
    assert w.shape[1] == K and s_a.shape == (b,) and s_w.shape == (N,)
    assert q.dtype == torch.int8 and w.dtype == torch.int8
    assert s_a.dtype == torch.float32 and s_w.dtype == torch.float32
    y = torch.empty((b, N), dtype=torch.bfloat16, device=q.device)
    acc = torch.empty((b, N), dtype=torch.int32, device=q.device) if with_acc else None
    st = torch.cuda.current_stream().cuda_stream
    rc = lib.mutant_linear(FAULT_CODES[fault], q.data_ptr(), s_a.data_ptr(), w.data_ptr(), s_w.data_ptr(),
                           b, N, K, y.data_ptr(), acc.data_ptr() if acc is not None else None, st)
    if rc != 0:
        raise RuntimeError(f"mutant_linear({fault}) returned {rc}")
    return y, acc
