"""CPU oracle for the batch-invariant int8 linear layer (test infrastructure).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import this package.  The product path
(the HIP library and its Python binding) never imports, loads or calls it,
and it imports nothing from the product package.

The arithmetic lives in ``oracle.c`` (plain scalar C, one binary32 operation
per expression, no fused multiply-add); this module only marshals numpy
arrays through ctypes.  bf16 and fp16 tensors travel as their uint16 bit
patterns.  Every function cites, in ``oracle.c``, the passage of the pages it
follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

# gcc flags: one rounding per float operation, no contraction, no fast-math,
# no host-specific instruction selection.
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=c11",
          "-Wall", "-Wextra", "-pthread"]

OK = 0
ERR_ARGS = -1
ERR_OVERFLOW = -2


class OracleError(RuntimeError):
    pass


def default_threads() -> int:
    """Worker threads when a call passes nthreads=0: OMP_NUM_THREADS when
    it is set (the host's CPU share on a shared machine), else every core.
    Threads split output rows only, so the count never changes a result."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    return os.cpu_count() or 1


def _nt(n: int) -> int:
    return n if n > 0 else default_threads()


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc and return its path."""
    if not force and os.path.exists(_LIB_PATH) and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    f32 = ctypes.c_float
    sig = {
        "oracle_f32_add": (f32, [f32, f32]),
        "oracle_f32_sub": (f32, [f32, f32]),
        "oracle_f32_mul": (f32, [f32, f32]),
        "oracle_f32_div": (f32, [f32, f32]),
        "oracle_i32_to_f32": (f32, [ctypes.c_int32]),
        "oracle_bf16_rne": (ctypes.c_uint16, [ctypes.c_uint32]),
        "oracle_bf16_to_f32": (f32, [ctypes.c_uint16]),
        "oracle_fp16_to_f32": (f32, [ctypes.c_uint16]),
        "oracle_epilogue": (ctypes.c_uint16, [ctypes.c_int32, f32, f32]),
        "oracle_block_partial": (f32, [ctypes.c_int32, f32, ctypes.c_uint16]),
        "oracle_tree_sum": (f32, [P, I64]),
        "oracle_dot_i8": (ctypes.c_int, [P, P, I64, P]),
        "oracle_quantize_token": (ctypes.c_int, [P, I64, I64, P, P]),
        "oracle_quantize_block32": (ctypes.c_int, [P, I64, I64, P, P]),
        "oracle_w8a8": (ctypes.c_int, [P, P, P, P, I64, I64, I64, P, ctypes.c_int]),
        "oracle_blockq8": (ctypes.c_int, [P, P, P, P, I64, I64, I64, P, ctypes.c_int]),
        "oracle_argmax_row": (ctypes.c_int32, [P, I64]),
        "oracle_lm_head_argmax": (ctypes.c_int, [P, P, P, P, I64, I64, I64, P, P, ctypes.c_int]),
        "oracle_pow2_nearest": (f32, [f32]),
        "oracle_pow2_requant": (ctypes.c_int, [P, P, I64, I64, P, P]),
        "oracle_attn_exp": (f32, [f32]),
        "oracle_e4m3_to_f32": (f32, [ctypes.c_uint8]),
        "oracle_f32_to_e4m3": (ctypes.c_uint8, [f32]),
        "oracle_quantize_fp8": (ctypes.c_int, [P, I64, I64, P, P]),
        "oracle_fp8_linear": (ctypes.c_int, [P, P, P, P, I64, I64, I64, P, ctypes.c_int]),
        "oracle_kq6_decode": (ctypes.c_int, [P, P, I64, I64, P]),
        "oracle_kq6_linear": (ctypes.c_int, [P, P, P, P, P, P, I64, I64, I64, P, ctypes.c_int]),
        "oracle_kq4_linear": (ctypes.c_int, [P, P, P, P, P, I64, I64, I64, P, ctypes.c_int]),
        "oracle_attn_decode": (ctypes.c_int, [P, P, P, I64, I64, I64, I64, I64, I64, I64, I64, I64, f32, I64, I64,
                                              P, ctypes.c_int]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _arr(a, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.dtype(dtype):
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def _check(status: int, what: str):
    if status == ERR_OVERFLOW:
        raise OracleError(f"{what}: int32 accumulator overflow (int64 shadow differs)")
    if status != OK:
        raise OracleError(f"{what}: status {status}")


# --- scalar primitives (one binary32 operation each) ------------------------

def f32_add(a, b) -> np.float32:
    return np.float32(_load().oracle_f32_add(float(np.float32(a)), float(np.float32(b))))


def f32_sub(a, b) -> np.float32:
    return np.float32(_load().oracle_f32_sub(float(np.float32(a)), float(np.float32(b))))


def f32_mul(a, b) -> np.float32:
    return np.float32(_load().oracle_f32_mul(float(np.float32(a)), float(np.float32(b))))


def f32_div(a, b) -> np.float32:
    return np.float32(_load().oracle_f32_div(float(np.float32(a)), float(np.float32(b))))


def i32_to_f32(v: int) -> np.float32:
    return np.float32(_load().oracle_i32_to_f32(int(v)))


def bf16_rne(bits: int) -> int:
    """fp32 bit pattern -> bf16 bit pattern, round to nearest even."""
    return int(_load().oracle_bf16_rne(int(bits) & 0xFFFFFFFF))


def bf16_to_f32(h: int) -> np.float32:
    return np.float32(_load().oracle_bf16_to_f32(int(h)))


def fp16_to_f32(h: int) -> np.float32:
    return np.float32(_load().oracle_fp16_to_f32(int(h)))


def epilogue(acc: int, s_a, s_w) -> int:
    """bf16 bits of (fl32(acc) * s_a) * s_w."""
    return int(_load().oracle_epilogue(int(acc), float(np.float32(s_a)), float(np.float32(s_w))))


def block_partial(isum: int, d_a, d_w_bits: int) -> np.float32:
    return np.float32(_load().oracle_block_partial(int(isum), float(np.float32(d_a)), int(d_w_bits)))


def tree_sum(leaves) -> np.float32:
    a = _arr(np.asarray(leaves, dtype=np.float32), np.float32)
    return np.float32(_load().oracle_tree_sum(_ptr(a), a.size))


def dot_i8(a, w) -> int:
    a = _arr(a, np.int8)
    w = _arr(w, np.int8)
    assert a.size == w.size
    out = np.zeros(1, np.int32)
    _check(_load().oracle_dot_i8(_ptr(a), _ptr(w), a.size, _ptr(out)), "dot_i8")
    return int(out[0])


# --- tensor operations -------------------------------------------------------

def quantize_token(x_bits: np.ndarray):
    """x bf16 bits uint16 [b, K] -> (q int8 [b, K], s fp32 [b])."""
    x = _arr(x_bits, np.uint16)
    b, K = x.shape
    q = np.empty((b, K), np.int8)
    s = np.empty((b,), np.float32)
    _check(_load().oracle_quantize_token(_ptr(x), b, K, _ptr(q), _ptr(s)), "quantize_token")
    return q, s


def quantize_block32(x_bits: np.ndarray):
    """x bf16 bits uint16 [b, K] -> (q int8 [b, K], d fp32 [b, K/32])."""
    x = _arr(x_bits, np.uint16)
    b, K = x.shape
    q = np.empty((b, K), np.int8)
    d = np.empty((b, K // 32), np.float32)
    _check(_load().oracle_quantize_block32(_ptr(x), b, K, _ptr(q), _ptr(d)), "quantize_block32")
    return q, d


def w8a8(q, s_a, w, s_w, nthreads: int = 0) -> np.ndarray:
    """-> y bf16 bits uint16 [b, N]."""
    q = _arr(q, np.int8)
    s_a = _arr(s_a, np.float32)
    w = _arr(w, np.int8)
    s_w = _arr(s_w, np.float32)
    b, K = q.shape
    N, K2 = w.shape
    assert K == K2 and s_a.shape == (b,) and s_w.shape == (N,)
    y = np.empty((b, N), np.uint16)
    _check(_load().oracle_w8a8(_ptr(q), _ptr(s_a), _ptr(w), _ptr(s_w), b, N, K, _ptr(y), _nt(nthreads)), "w8a8")
    return y


def blockq8(q, d_a, w, d_w_bits, nthreads: int = 0) -> np.ndarray:
    """q int8 [b,K], d_a fp32 [b,K/32], w int8 [N,K], d_w fp16 bits [N,K/32] -> y bf16 bits [b,N]."""
    q = _arr(q, np.int8)
    d_a = _arr(d_a, np.float32)
    w = _arr(w, np.int8)
    d_w = _arr(d_w_bits, np.uint16)
    b, K = q.shape
    N = w.shape[0]
    assert w.shape == (N, K) and d_a.shape == (b, K // 32) and d_w.shape == (N, K // 32)
    y = np.empty((b, N), np.uint16)
    _check(_load().oracle_blockq8(_ptr(q), _ptr(d_a), _ptr(w), _ptr(d_w), b, N, K, _ptr(y), _nt(nthreads)),
           "blockq8")
    return y


def argmax_row(y_bits) -> int:
    y = _arr(y_bits, np.uint16)
    return int(_load().oracle_argmax_row(_ptr(y), y.size))


def lm_head_argmax(q, s_a, w, s_w, nthreads: int = 0):
    """-> (logits bf16 bits uint16 [b, N], argmax int32 [b])."""
    q = _arr(q, np.int8)
    s_a = _arr(s_a, np.float32)
    w = _arr(w, np.int8)
    s_w = _arr(s_w, np.float32)
    b, K = q.shape
    N = w.shape[0]
    logits = np.empty((b, N), np.uint16)
    am = np.empty((b,), np.int32)
    _check(_load().oracle_lm_head_argmax(_ptr(q), _ptr(s_a), _ptr(w), _ptr(s_w), b, N, K, _ptr(logits),
                                         _ptr(am), _nt(nthreads)), "lm_head_argmax")
    return logits, am


def pow2_nearest(s) -> np.float32:
    return np.float32(_load().oracle_pow2_nearest(float(np.float32(s))))


def pow2_requant(w, s_w):
    """-> (w' int8 [N, K], s' fp32 [N])."""
    w = _arr(w, np.int8)
    s_w = _arr(s_w, np.float32)
    N, K = w.shape
    wo = np.empty((N, K), np.int8)
    so = np.empty((N,), np.float32)
    _check(_load().oracle_pow2_requant(_ptr(w), _ptr(s_w), N, K, _ptr(wo), _ptr(so)), "pow2_requant")
    return wo, so


# --- decode attention over a KV cache in fixed 256-cell chunks -------------------

ATTN_CHUNK = 256


def attn_exp(x) -> np.float32:
    """The attention recipe's e^x (x <= 0), binary32 operations only."""
    return np.float32(_load().oracle_attn_exp(float(np.float32(x))))


def _cache_view(c: np.ndarray, name: str):
    """A bf16 cache [cells, heads, D] (uint16 bits, any cell and head strides,
    unit stride along D) -> (array, cell stride, head stride) in elements."""
    if c.dtype != np.uint16 or c.ndim != 3 or c.strides[2] != 2 or c.strides[0] % 2 or c.strides[1] % 2:
        raise TypeError(f"{name}: expected uint16 [cells, heads, D] with unit stride along D")
    return c, c.strides[0] // 2, c.strides[1] // 2


def attn_decode(q, k_cache, v_cache, pos0: int, scale, heads=None, nthreads: int = 0) -> np.ndarray:
    """q bf16 bits [b, Hq, D]; k_cache, v_cache bf16 bits [cells, Hkv, D]
    (views with their own strides are fine); query t at position pos0 + t.
    -> out bf16 bits [b, Hq, D] (zeros outside `heads`, a (lo, hi) range)."""
    q = _arr(q, np.uint16)
    b, Hq, D = q.shape
    k, kc, kh = _cache_view(k_cache, "k_cache")
    v, vc, vh = _cache_view(v_cache, "v_cache")
    Hkv = k.shape[1]
    if v.shape[1] != Hkv or k.shape[2] != D or v.shape[2] != D:
        raise ValueError("cache shapes do not match q")
    if pos0 + b > min(k.shape[0], v.shape[0]):
        raise ValueError("positions past the cache")
    h0, h1 = heads if heads is not None else (0, Hq)
    out = np.zeros((b, Hq, D), np.uint16)
    kp = ctypes.c_void_p(k.__array_interface__["data"][0])
    vp = ctypes.c_void_p(v.__array_interface__["data"][0])
    _check(_load().oracle_attn_decode(_ptr(q), kp, vp, kc, kh, vc, vh, b, Hq, Hkv, D, pos0, float(np.float32(scale)),
                                      h0, h1, _ptr(out), _nt(nthreads)), "attn_decode")
    return out


# --- FP8 (E4M3) W8A8 linear with the fixed tree ----------------------------------

def e4m3_to_f32(code: int) -> np.float32:
    return np.float32(_load().oracle_e4m3_to_f32(int(code) & 0xFF))


def f32_to_e4m3(x) -> int:
    return int(_load().oracle_f32_to_e4m3(float(np.float32(x))))


def quantize_fp8(x_bits: np.ndarray):
    """bf16 bits [b, K] -> (e4m3 codes uint8 [b, K], s_a fp32 [b])."""
    x = _arr(x_bits, np.uint16)
    b, K = x.shape
    q = np.empty((b, K), np.uint8)
    s = np.empty((b,), np.float32)
    _check(_load().oracle_quantize_fp8(_ptr(x), b, K, _ptr(q), _ptr(s)), "quantize_fp8")
    return q, s


def fp8_linear(q, s_a, w, s_w, nthreads: int = 0) -> np.ndarray:
    """e4m3 q [b, K], s_a [b], e4m3 w [N, K], s_w [N] -> y bf16 bits [b, N]."""
    q = _arr(q, np.uint8)
    w = _arr(w, np.uint8)
    s_a = _arr(s_a, np.float32)
    s_w = _arr(s_w, np.float32)
    b, K = q.shape
    N = w.shape[0]
    y = np.empty((b, N), np.uint16)
    _check(_load().oracle_fp8_linear(_ptr(q), _ptr(s_a), _ptr(w), _ptr(s_w), b, N, K, _ptr(y), _nt(nthreads)),
           "fp8_linear")
    return y


# --- k-quant-style 6-bit superblocks (kq6) ------------------------------------

def kq6_decode(ql, qh) -> np.ndarray:
    """Low plane uint8 [N, K/2] and high plane uint8 [N, K/4] -> codes int8 [N, K] in [-32, 31]."""
    ql = _arr(ql, np.uint8)
    qh = _arr(qh, np.uint8)
    N, K2 = ql.shape
    K = 2 * K2
    assert qh.shape == (N, K // 4)
    codes = np.empty((N, K), np.int8)
    _check(_load().oracle_kq6_decode(_ptr(ql), _ptr(qh), N, K, _ptr(codes)), "kq6_decode")
    return codes


def kq6_linear(q, d_a, ql, qh, sc, d_bits, nthreads: int = 0) -> np.ndarray:
    """q int8 [b,K], d_a fp32 [b,K/32], ql uint8 [N,K/2], qh uint8 [N,K/4], sc int8 [N,K/16],
    d fp16 bits [N,K/256] -> y bf16 bits [b,N]."""
    q = _arr(q, np.int8)
    d_a = _arr(d_a, np.float32)
    ql = _arr(ql, np.uint8)
    qh = _arr(qh, np.uint8)
    sc = _arr(sc, np.int8)
    d = _arr(d_bits, np.uint16)
    b, K = q.shape
    N = ql.shape[0]
    assert ql.shape == (N, K // 2) and qh.shape == (N, K // 4) and sc.shape == (N, K // 16)
    assert d.shape == (N, K // 256) and d_a.shape == (b, K // 32)
    y = np.empty((b, N), np.uint16)
    _check(_load().oracle_kq6_linear(_ptr(q), _ptr(d_a), _ptr(ql), _ptr(qh), _ptr(sc), _ptr(d), b, N, K, _ptr(y),
                                     _nt(nthreads)), "kq6_linear")
    return y


def kq4_linear(q, d_a, ql, scm, dm_bits, nthreads: int = 0) -> np.ndarray:
    """q int8 [b,K], d_a fp32 [b,K/32], ql uint8 [N,K/2], scm uint8 [N,K/32,2] (sub-scale, minimum),
    dm fp16 bits [N,K/256,2] (d, dmin) -> y bf16 bits [b,N]."""
    q = _arr(q, np.int8)
    d_a = _arr(d_a, np.float32)
    ql = _arr(ql, np.uint8)
    scm = _arr(scm, np.uint8)
    dm = _arr(dm_bits, np.uint16)
    b, K = q.shape
    N = ql.shape[0]
    assert ql.shape == (N, K // 2) and scm.shape == (N, K // 32, 2) and dm.shape == (N, K // 256, 2)
    assert d_a.shape == (b, K // 32)
    y = np.empty((b, N), np.uint16)
    _check(_load().oracle_kq4_linear(_ptr(q), _ptr(d_a), _ptr(ql), _ptr(scm), _ptr(dm), b, N, K, _ptr(y), _nt(nthreads)),
           "kq4_linear")
    return y
