"""ctypes binding of libiqd.so (the gfx950 kernels behind the C ABI in include/iqd.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels.  torch supplies device memory and the current stream.  If the
library is missing or cannot be loaded, every call raises: there is no CPU or
PyTorch fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libiqd.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "iqd.h")

IQD_OK = 0
IQD_ERR_INVALID = -1
IQD_ERR_ALIGN = -2
IQD_ERR_RANGE = -3
IQD_ERR_UNSUPPORTED = -4
IQD_ERR_WORKSPACE = -5
IQD_ERR_HIP = -6

IQD_OP_W8A8 = 1
IQD_OP_BLOCKQ8 = 2
IQD_OP_LM_HEAD = 3
IQD_OP_W8A8_BF16 = 4
IQD_OP_FP8 = 5
IQD_OP_KQ6 = 6
IQD_OP_KQ4 = 7

IQD_K_MAX = 131071
IQD_SPLIT_K_MAX = 64


class IqdError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        msg = status_str(status) if _lib is not None else str(status)
        if status == IQD_ERR_HIP and _lib is not None:
            msg += f" ({_lib.iqd_last_hip_error().decode()})"
        super().__init__(f"{what}: {msg}")


_lib = None

P = ctypes.c_void_p
I64 = ctypes.c_int64
I32 = ctypes.c_int32
SZ = ctypes.c_size_t

SIGNATURES = {
    "quantize_activations": (ctypes.c_int, [P, I64, I64, I32, P, P, P]),
    "w8a8_linear": (ctypes.c_int, [P, P, P, P, I64, I64, I64, P, I32, P, SZ, P]),
    "w8a8_linear_bf16": (ctypes.c_int, [P, P, P, I64, I64, I64, P, P, P, P, SZ, P]),
    "blockq8_linear": (ctypes.c_int, [P, P, P, P, I64, I64, I64, P, I32, P, SZ, P]),
    "kq6_linear": (ctypes.c_int, [P, P, P, P, P, P, I64, I64, I64, P, I32, P, SZ, P]),
    "kq4_linear": (ctypes.c_int, [P, P, P, P, P, I64, I64, I64, P, I32, P, SZ, P]),
    "lm_head_argmax": (ctypes.c_int, [P, P, P, P, I64, I64, I64, P, P, P, SZ, P]),
    "lm_head_argmax_static": (ctypes.c_int, [P, P, P, P, I64, I64, I64, P, P, P]),
    "pow2_requantize": (ctypes.c_int, [P, P, I64, I64, P, P, P]),
    "quantize_fp8": (ctypes.c_int, [P, I64, I64, P, P, P]),
    "fp8_linear": (ctypes.c_int, [P, P, P, P, I64, I64, I64, P, I32, P, SZ, P]),
    "attn_decode": (ctypes.c_int, [P, P, P, I64, I64, I64, I64, I64, I64, I64, I64, I64, ctypes.c_float, P, P, SZ,
                                   P]),
    "attn_workspace_bytes": (SZ, [I64, I64, I64, I64, I64]),
    "iqd_read_ceiling": (ctypes.c_int, [P, I64, P, P]),
    "iqd_workspace_bytes": (SZ, [ctypes.c_int, I64, I64, I64, I32]),
    "iqd_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "iqd_last_hip_error": (ctypes.c_char_p, []),
}


def header_functions() -> list[str]:
    """Names of the functions include/iqd.h declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                      text, flags=re.M)


def load():
    """Load libiqd.so (raises OSError when it is missing: no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise OSError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                      "(hipcc --offload-arch=gfx950); there is no fallback path")
    # torch supplies the device memory and streams, so libiqd must bind to the
    # same HIP runtime instance as torch.  torch bundles its own copy of
    # libamdhip64 (same SONAME as the system one it was built against); loading
    # torch first makes the dynamic loader resolve libiqd's dependency to that
    # already-loaded copy instead of starting a second, separate runtime.
    import torch  # noqa: F401

    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().iqd_status_str(int(status)).decode()


def workspace_bytes(op: int, b: int, N: int, K: int, split_k: int = 1) -> int:
    return int(load().iqd_workspace_bytes(op, b, N, K, split_k))


# --- torch glue ---------------------------------------------------------------

def _torch():
    import torch

    return torch


def _stream_ptr():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check_tensor(t, name: str, dtypes, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (strides are never guessed)")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _raise(status: int, what: str):
    if status != IQD_OK:
        raise IqdError(status, what)


def _workspace(nbytes: int, device):
    torch = _torch()
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def quantize_activations(x, group: int = 0, q=None, scale=None):
    """x bf16 [b, K] -> (q int8 [b, K], scale fp32 [b] or [b, K/32])."""
    torch = _torch()
    _check_tensor(x, "x", (torch.bfloat16,))
    b, K = x.shape
    if q is None:
        q = torch.empty((b, K), dtype=torch.int8, device=x.device)
    if scale is None:
        scale = torch.empty((b,) if group == 0 else (b, K // 32), dtype=torch.float32, device=x.device)
    _check_tensor(q, "q", (torch.int8,), (b, K))
    _check_tensor(scale, "scale", (torch.float32,))
    st = load().quantize_activations(_ptr(x), b, K, group, _ptr(q), _ptr(scale), _stream_ptr())
    _raise(st, "quantize_activations")
    return q, scale


def w8a8_linear(q, s_a, w, s_w, split_k: int = 1, y=None, workspace=None):
    """q int8 [b, K], s_a fp32 [b], w int8 [N, K], s_w fp32 [N] -> y bf16 [b, N]."""
    torch = _torch()
    _check_tensor(q, "q", (torch.int8,))
    b, K = q.shape
    N = w.shape[0]
    _check_tensor(s_a, "s_a", (torch.float32,), (b,))
    _check_tensor(w, "w", (torch.int8,), (N, K))
    _check_tensor(s_w, "s_w", (torch.float32,), (N,))
    if y is None:
        y = torch.empty((b, N), dtype=torch.bfloat16, device=q.device)
    _check_tensor(y, "y", (torch.bfloat16,), (b, N))
    need = workspace_bytes(IQD_OP_W8A8, b, N, K, split_k)
    if workspace is None:
        workspace = _workspace(need, q.device)
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load().w8a8_linear(_ptr(q), _ptr(s_a), _ptr(w), _ptr(s_w), b, N, K, _ptr(y), split_k, _ptr(workspace),
                            wsb, _stream_ptr())
    _raise(st, "w8a8_linear")
    return y


def blockq8_linear(q, d_a, w, d_w, split_k: int = 1, y=None, workspace=None):
    """q int8 [b, K], d_a fp32 [b, K/32], w int8 [N, K], d_w fp16 [N, K/32] -> y bf16 [b, N]."""
    torch = _torch()
    _check_tensor(q, "q", (torch.int8,))
    b, K = q.shape
    N = w.shape[0]
    _check_tensor(d_a, "d_a", (torch.float32,), (b, K // 32))
    _check_tensor(w, "w", (torch.int8,), (N, K))
    _check_tensor(d_w, "d_w", (torch.float16, torch.int16), (N, K // 32))
    if y is None:
        y = torch.empty((b, N), dtype=torch.bfloat16, device=q.device)
    _check_tensor(y, "y", (torch.bfloat16,), (b, N))
    need = workspace_bytes(IQD_OP_BLOCKQ8, b, N, K, split_k)
    if workspace is None:
        workspace = _workspace(need, q.device)
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load().blockq8_linear(_ptr(q), _ptr(d_a), _ptr(w), _ptr(d_w), b, N, K, _ptr(y), split_k, _ptr(workspace),
                               wsb, _stream_ptr())
    _raise(st, "blockq8_linear")
    return y


def kq6_linear(q, d_a, ql, qh, sc, d, split_k: int = 1, y=None, workspace=None):
    """q int8 [b, K], d_a fp32 [b, K/32], kq6 weights ql uint8 [N, K/2], qh uint8 [N, K/4],
    sc int8 [N, K/16], d fp16 [N, K/256] -> y bf16 [b, N]."""
    torch = _torch()
    _check_tensor(q, "q", (torch.int8,))
    b, K = q.shape
    N = ql.shape[0]
    _check_tensor(d_a, "d_a", (torch.float32,), (b, K // 32))
    _check_tensor(ql, "ql", (torch.uint8,), (N, K // 2))
    _check_tensor(qh, "qh", (torch.uint8,), (N, K // 4))
    _check_tensor(sc, "sc", (torch.int8,), (N, K // 16))
    _check_tensor(d, "d", (torch.float16, torch.int16), (N, K // 256))
    if y is None:
        y = torch.empty((b, N), dtype=torch.bfloat16, device=q.device)
    _check_tensor(y, "y", (torch.bfloat16,), (b, N))
    need = workspace_bytes(IQD_OP_KQ6, b, N, K, split_k)
    if workspace is None:
        workspace = _workspace(need, q.device)
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load().kq6_linear(_ptr(q), _ptr(d_a), _ptr(ql), _ptr(qh), _ptr(sc), _ptr(d), b, N, K, _ptr(y), split_k,
                           _ptr(workspace), wsb, _stream_ptr())
    _raise(st, "kq6_linear")
    return y


def kq4_linear(q, d_a, ql, scm, dm, split_k: int = 1, y=None, workspace=None):
    """q int8 [b, K], d_a fp32 [b, K/32], kq4 weights ql uint8 [N, K/2], scm uint8 [N, K/32, 2]
    (sub-scale, minimum), dm fp16 [N, K/256, 2] (d, dmin) -> y bf16 [b, N]."""
    torch = _torch()
    _check_tensor(q, "q", (torch.int8,))
    b, K = q.shape
    N = ql.shape[0]
    _check_tensor(d_a, "d_a", (torch.float32,), (b, K // 32))
    _check_tensor(ql, "ql", (torch.uint8,), (N, K // 2))
    _check_tensor(scm, "scm", (torch.uint8,), (N, K // 32, 2))
    _check_tensor(dm, "dm", (torch.float16, torch.int16), (N, K // 256, 2))
    if y is None:
        y = torch.empty((b, N), dtype=torch.bfloat16, device=q.device)
    _check_tensor(y, "y", (torch.bfloat16,), (b, N))
    need = workspace_bytes(IQD_OP_KQ4, b, N, K, split_k)
    if workspace is None:
        workspace = _workspace(need, q.device)
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load().kq4_linear(_ptr(q), _ptr(d_a), _ptr(ql), _ptr(scm), _ptr(dm), b, N, K, _ptr(y), split_k,
                           _ptr(workspace), wsb, _stream_ptr())
    _raise(st, "kq4_linear")
    return y


def w8a8_linear_bf16(x, w, s_w, y=None, q_out=None, s_a_out=None, workspace=None):
    """x bf16 [b, K], w int8 [N, K], s_w fp32 [N] -> y bf16 [b, N]; quantize_activations
    and w8a8_linear in one call (q_out int8 [b, K] / s_a_out fp32 [b] optionally receive the
    quantized activations)."""
    torch = _torch()
    _check_tensor(x, "x", (torch.bfloat16,))
    b, K = x.shape
    N = w.shape[0]
    _check_tensor(w, "w", (torch.int8,), (N, K))
    _check_tensor(s_w, "s_w", (torch.float32,), (N,))
    if y is None:
        y = torch.empty((b, N), dtype=torch.bfloat16, device=x.device)
    _check_tensor(y, "y", (torch.bfloat16,), (b, N))
    if q_out is not None:
        _check_tensor(q_out, "q_out", (torch.int8,), (b, K))
    if s_a_out is not None:
        _check_tensor(s_a_out, "s_a_out", (torch.float32,), (b,))
    need = 0 if (q_out is not None and s_a_out is not None) else workspace_bytes(IQD_OP_W8A8_BF16, b, N, K, 1)
    if workspace is None:
        workspace = _workspace(need, x.device)
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load().w8a8_linear_bf16(_ptr(x), _ptr(w), _ptr(s_w), b, N, K, _ptr(y), _ptr(q_out), _ptr(s_a_out),
                                 _ptr(workspace), wsb, _stream_ptr())
    _raise(st, "w8a8_linear_bf16")
    return y


def lm_head_argmax(q, s_a, w, s_w, logits=True, argmax=None, workspace=None):
    """-> (logits bf16 [b, N] or None, argmax int32 [b]).  logits=False skips writing logits."""
    torch = _torch()
    _check_tensor(q, "q", (torch.int8,))
    b, K = q.shape
    N = w.shape[0]
    _check_tensor(s_a, "s_a", (torch.float32,), (b,))
    _check_tensor(w, "w", (torch.int8,), (N, K))
    _check_tensor(s_w, "s_w", (torch.float32,), (N,))
    lg = None
    if logits is True:
        lg = torch.empty((b, N), dtype=torch.bfloat16, device=q.device)
    elif isinstance(logits, torch.Tensor):
        lg = logits
        _check_tensor(lg, "logits", (torch.bfloat16,), (b, N))
    if argmax is None:
        argmax = torch.empty((b,), dtype=torch.int32, device=q.device)
    _check_tensor(argmax, "argmax", (torch.int32,), (b,))
    need = workspace_bytes(IQD_OP_LM_HEAD, b, N, K, 1)  # covers the no-logits case too
    if workspace is None:
        workspace = _workspace(need, q.device)
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load().lm_head_argmax(_ptr(q), _ptr(s_a), _ptr(w), _ptr(s_w), b, N, K, _ptr(lg), _ptr(argmax),
                               _ptr(workspace), wsb, _stream_ptr())
    _raise(st, "lm_head_argmax")
    return lg, argmax


IQD_STATIC_SCRATCH_BYTES = 8 << 20


def lm_head_argmax_static(q, s_a, w, s_w, logits=True, argmax=None):
    """lm_head_argmax with the library's own device scratch in place of a
    workspace (allocates nothing when logits and argmax are given) ->
    (logits bf16 [b, N] or None, argmax int32 [b])."""
    torch = _torch()
    _check_tensor(q, "q", (torch.int8,))
    b, K = q.shape
    N = w.shape[0]
    _check_tensor(s_a, "s_a", (torch.float32,), (b,))
    _check_tensor(w, "w", (torch.int8,), (N, K))
    _check_tensor(s_w, "s_w", (torch.float32,), (N,))
    lg = None
    if logits is True:
        lg = torch.empty((b, N), dtype=torch.bfloat16, device=q.device)
    elif isinstance(logits, torch.Tensor):
        lg = logits
        _check_tensor(lg, "logits", (torch.bfloat16,), (b, N))
    if argmax is None:
        argmax = torch.empty((b,), dtype=torch.int32, device=q.device)
    _check_tensor(argmax, "argmax", (torch.int32,), (b,))
    st = load().lm_head_argmax_static(_ptr(q), _ptr(s_a), _ptr(w), _ptr(s_w), b, N, K, _ptr(lg), _ptr(argmax),
                                      _stream_ptr())
    _raise(st, "lm_head_argmax_static")
    return lg, argmax


def pow2_requantize(w, s_w, w_out=None, s_out=None):
    """w int8 [N, K], s_w fp32 [N] -> (w' int8 [N, K], s' fp32 [N])."""
    torch = _torch()
    _check_tensor(w, "w", (torch.int8,))
    N, K = w.shape
    _check_tensor(s_w, "s_w", (torch.float32,), (N,))
    if w_out is None:
        w_out = torch.empty_like(w)
    if s_out is None:
        s_out = torch.empty_like(s_w)
    _check_tensor(w_out, "w_out", (torch.int8,), (N, K))
    _check_tensor(s_out, "s_out", (torch.float32,), (N,))
    st = load().pow2_requantize(_ptr(w), _ptr(s_w), N, K, _ptr(w_out), _ptr(s_out), _stream_ptr())
    _raise(st, "pow2_requantize")
    return w_out, s_out


def attn_workspace_bytes(b: int, Hq: int, Hkv: int, D: int, pos0: int) -> int:
    return int(load().attn_workspace_bytes(b, Hq, Hkv, D, pos0))


def _check_cache(t, name: str, Hkv: int, D: int):
    """A bf16 cache [cells, Hkv, D] with unit stride along D; its cell and
    head strides are passed as they are (a view into a larger buffer is fine)."""
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be a bf16 cuda tensor")
    if t.dim() != 3 or t.shape[1] != Hkv or t.shape[2] != D or t.stride(2) != 1:
        raise ValueError(f"{name} must be [cells, {Hkv}, {D}] with unit stride along the last dimension")


def attn_decode(q, k_cache, v_cache, pos0: int, scale: float, out=None, workspace=None):
    """q bf16 [b, Hq, D]; k_cache, v_cache bf16 [cells, Hkv, D] (strided views
    allowed); query t at position pos0 + t -> out bf16 [b, Hq, D]."""
    torch = _torch()
    _check_tensor(q, "q", (torch.bfloat16,))
    b, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    _check_cache(k_cache, "k_cache", Hkv, D)
    _check_cache(v_cache, "v_cache", Hkv, D)
    if pos0 + b > min(k_cache.shape[0], v_cache.shape[0]):
        raise ValueError("the caches must hold cells 0 .. pos0 + b - 1")
    if out is None:
        out = torch.empty_like(q)
    _check_tensor(out, "out", (torch.bfloat16,), (b, Hq, D))
    need = attn_workspace_bytes(b, Hq, Hkv, D, pos0)
    if workspace is None:
        workspace = _workspace(need, q.device)
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load().attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), k_cache.stride(0), k_cache.stride(1),
                            v_cache.stride(0), v_cache.stride(1), b, Hq, Hkv, D, pos0, float(scale), _ptr(out),
                            _ptr(workspace), wsb, _stream_ptr())
    _raise(st, "attn_decode")
    return out


def quantize_fp8(x, q=None, scale=None):
    """bf16 [b, K] -> (E4M3 codes uint8 [b, K], s_a fp32 [b])."""
    torch = _torch()
    _check_tensor(x, "x", (torch.bfloat16,))
    b, K = x.shape
    if q is None:
        q = torch.empty((b, K), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty((b,), dtype=torch.float32, device=x.device)
    _check_tensor(q, "q", (torch.uint8,), (b, K))
    _check_tensor(scale, "scale", (torch.float32,), (b,))
    st = load().quantize_fp8(_ptr(x), b, K, _ptr(q), _ptr(scale), _stream_ptr())
    _raise(st, "quantize_fp8")
    return q, scale


def fp8_linear(q, s_a, w, s_w, split_k: int = 1, y=None, workspace=None):
    """E4M3 q [b, K], s_a [b], E4M3 w [N, K], s_w [N] -> y bf16 [b, N]."""
    torch = _torch()
    _check_tensor(q, "q", (torch.uint8,))
    b, K = q.shape
    N = w.shape[0]
    _check_tensor(s_a, "s_a", (torch.float32,), (b,))
    _check_tensor(w, "w", (torch.uint8,), (N, K))
    _check_tensor(s_w, "s_w", (torch.float32,), (N,))
    if y is None:
        y = torch.empty((b, N), dtype=torch.bfloat16, device=q.device)
    _check_tensor(y, "y", (torch.bfloat16,), (b, N))
    need = workspace_bytes(IQD_OP_FP8, b, N, K, split_k)
    if workspace is None:
        workspace = _workspace(need, q.device)
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load().fp8_linear(_ptr(q), _ptr(s_a), _ptr(w), _ptr(s_w), b, N, K, _ptr(y), split_k, _ptr(workspace), wsb,
                           _stream_ptr())
    _raise(st, "fp8_linear")
    return y


def read_ceiling(t, sink):
    """Measurement helper: stream the bytes of device tensor t (contiguous, a
    multiple of 16 bytes) with the mat-vec kernels' loads; sink is an int32
    [1] device tensor."""
    torch = _torch()
    if not (t.is_cuda and t.is_contiguous()):
        raise ValueError("t must be a contiguous cuda tensor")
    _check_tensor(sink, "sink", (torch.int32,), (1,))
    st = load().iqd_read_ceiling(_ptr(t), t.numel() * t.element_size(), _ptr(sink), _stream_ptr())
    _raise(st, "iqd_read_ceiling")
