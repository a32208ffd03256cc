"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/iqd.h declares, and rejects bad arguments before any
launch.  Fake, never-dereferenced pointers are used: every call below must
return from validation."""
import ctypes

import pytest

import invariant_quantized_decode_token_amd as iqd
from invariant_quantized_decode_token_amd import _lib as L


@pytest.fixture(scope="module")
def lib():
    return iqd.load()


def test_exports_every_declared_function(lib):
    names = iqd.header_functions()
    assert set(names) == {"quantize_activations", "w8a8_linear", "w8a8_linear_bf16", "blockq8_linear", "lm_head_argmax",
                          "pow2_requantize", "iqd_workspace_bytes", "iqd_status_str", "iqd_last_hip_error",
                          "attn_decode", "attn_workspace_bytes", "quantize_fp8", "fp8_linear", "kq6_linear",
                          "kq4_linear", "iqd_read_ceiling", "lm_head_argmax_static"}
    for n in names:
        assert hasattr(lib, n), n


def test_lm_head_static_validation(lib):
    def call(b=4, N=1000, K=512, q=A, lg=0, am=5 * A):
        return lib.lm_head_argmax_static(ptr(q), ptr(2 * A), ptr(3 * A), ptr(4 * A), b, N, K, ptr(lg), ptr(am), None)
    assert call(b=16, N=300000, K=64, am=64 * A) == L.IQD_ERR_WORKSPACE  # 9.6 MB of logits > the static scratch
    assert call(q=A + 8) == L.IQD_ERR_ALIGN
    assert call(K=40) == L.IQD_ERR_INVALID
    assert call(am=0) == L.IQD_ERR_INVALID
    assert call(am=3 * A + 16) == L.IQD_ERR_INVALID             # argmax inside the weights


def test_read_ceiling_validation(lib):
    rc = lib.iqd_read_ceiling
    assert rc(None, 1024, ptr(A), None) == L.IQD_ERR_INVALID
    assert rc(ptr(A), 1000, ptr(2 * A), None) == L.IQD_ERR_INVALID     # not a multiple of 16
    assert rc(ptr(A), 0, ptr(2 * A), None) == L.IQD_ERR_INVALID
    assert rc(ptr(A + 8), 1024, ptr(2 * A), None) == L.IQD_ERR_ALIGN
    assert rc(ptr(A), 1024, ptr(A + 64), None) == L.IQD_ERR_INVALID    # sink inside the buffer


def test_status_strings(lib):
    for code in range(-6, 1):
        s = iqd.status_str(code)
        assert s.startswith("IQD_")
    assert "unknown" in iqd.status_str(42)


def test_workspace_bytes():
    assert iqd.workspace_bytes(L.IQD_OP_W8A8, 8, 4096, 4096, 1) == 0
    assert iqd.workspace_bytes(L.IQD_OP_W8A8, 8, 4096, 4096, 4) == 4 * 8 * 4096 * 4
    assert iqd.workspace_bytes(L.IQD_OP_W8A8, 8, 4096, 4096, 3) == 0       # rejected split
    assert iqd.workspace_bytes(L.IQD_OP_W8A8, 8, 4096, 131072, 1) == 0     # rejected K
    assert iqd.workspace_bytes(L.IQD_OP_BLOCKQ8, 16, 4096, 12288, 16) == 16 * 16 * 4096 * 4
    assert iqd.workspace_bytes(L.IQD_OP_BLOCKQ8, 16, 4096, 4096, 8) == 8 * 16 * 4096 * 4  # 16-leaf subtrees
    assert iqd.workspace_bytes(L.IQD_OP_BLOCKQ8, 16, 4096, 256, 16) == 0   # 16 > L = 8
    # logits, then argmax keys: 8 bytes per (token, mat-vec workgroup), 32768 keys for a pass of up to 16 tokens
    assert iqd.workspace_bytes(L.IQD_OP_LM_HEAD, 5, 151936, 4096, 1) == (5 * 151936 * 2 + 15) // 16 * 16 + 32768 * 8
    assert iqd.workspace_bytes(L.IQD_OP_LM_HEAD, 40, 1000, 512, 1) == 40 * 1000 * 2 + 32768 * 8


A = 1 << 20  # fake, 16-byte aligned, never dereferenced


def ptr(v):
    return ctypes.c_void_p(v)


def w8a8(lib, b=4, N=64, K=256, split=1, q=A, sa=2 * A, w=3 * A, sw=4 * A, y=5 * A, ws=0, wsb=0):
    return lib.w8a8_linear(ptr(q), ptr(sa), ptr(w), ptr(sw), b, N, K, ptr(y), split, ptr(ws), wsb, None)


def test_w8a8_validation(lib):
    assert w8a8(lib, q=0) == L.IQD_ERR_INVALID
    assert w8a8(lib, b=0) == L.IQD_ERR_INVALID
    assert w8a8(lib, N=0) == L.IQD_ERR_INVALID
    assert w8a8(lib, K=0) == L.IQD_ERR_INVALID
    assert w8a8(lib, K=40) == L.IQD_ERR_INVALID              # K % 16
    assert w8a8(lib, K=131072) == L.IQD_ERR_RANGE
    assert w8a8(lib, split=3) == L.IQD_ERR_UNSUPPORTED
    assert w8a8(lib, split=128) == L.IQD_ERR_UNSUPPORTED
    assert w8a8(lib, K=32, split=4) == L.IQD_ERR_UNSUPPORTED  # more splits than 16-byte vectors
    assert w8a8(lib, b=17, split=2) == L.IQD_ERR_WORKSPACE  # the tiled path splits K too
    assert w8a8(lib, q=A + 8) == L.IQD_ERR_ALIGN
    assert w8a8(lib, w=3 * A + 4) == L.IQD_ERR_ALIGN
    assert w8a8(lib, sa=2 * A + 2) == L.IQD_ERR_ALIGN
    assert w8a8(lib, y=5 * A + 1) == L.IQD_ERR_ALIGN
    assert w8a8(lib, split=2) == L.IQD_ERR_WORKSPACE
    assert w8a8(lib, split=2, ws=6 * A, wsb=100) == L.IQD_ERR_WORKSPACE
    assert w8a8(lib, split=2, ws=6 * A + 4, wsb=1 << 20) == L.IQD_ERR_ALIGN
    assert w8a8(lib, y=A + 64) == L.IQD_ERR_INVALID          # output overlaps q
    assert w8a8(lib, y=3 * A + 100) == L.IQD_ERR_INVALID     # output overlaps w
    assert w8a8(lib, split=2, ws=5 * A, wsb=1 << 20) == L.IQD_ERR_INVALID  # workspace overlaps y


def test_blockq8_validation(lib):
    def call(b=4, N=64, K=1024, split=1, dw=4 * A, ws=0, wsb=0):
        return lib.blockq8_linear(ptr(A), ptr(2 * A), ptr(3 * A), ptr(dw), b, N, K, ptr(5 * A), split, ptr(ws), wsb,
                                  None)
    assert call(K=48) == L.IQD_ERR_INVALID                   # K % 32
    assert call(K=131072 + 32) == L.IQD_ERR_RANGE
    assert call(K=256, split=16) == L.IQD_ERR_UNSUPPORTED    # L = 8 leaves: at most 8 splits
    assert call(K=256, split=8) == L.IQD_ERR_WORKSPACE       # one leaf per split
    assert call(split=3) == L.IQD_ERR_UNSUPPORTED
    assert call(K=4096, split=128) == L.IQD_ERR_UNSUPPORTED  # above IQD_SPLIT_K_MAX
    assert call(K=4096, split=8) == L.IQD_ERR_WORKSPACE      # 16-leaf subtrees
    assert call(K=4096, split=4) == L.IQD_ERR_WORKSPACE
    assert call(dw=4 * A + 1) == L.IQD_ERR_ALIGN


def test_kq6_validation(lib):
    def call(b=4, N=64, K=1024, split=1, q=A, ql=3 * A, qh=4 * A, sc=6 * A, d=7 * A, y=5 * A, ws=0, wsb=0):
        return lib.kq6_linear(ptr(q), ptr(2 * A), ptr(ql), ptr(qh), ptr(sc), ptr(d), b, N, K, ptr(y), split, ptr(ws),
                              wsb, None)
    assert call(K=512 + 32) == L.IQD_ERR_INVALID             # K % 256
    assert call(K=131072 + 256) == L.IQD_ERR_RANGE
    assert call(K=256, split=16) == L.IQD_ERR_UNSUPPORTED    # L = 8 leaves: at most 8 splits
    assert call(K=256, split=8) == L.IQD_ERR_WORKSPACE       # one leaf per split
    assert call(split=3) == L.IQD_ERR_UNSUPPORTED
    assert call(K=4096, split=128) == L.IQD_ERR_UNSUPPORTED  # above IQD_SPLIT_K_MAX
    assert call(K=4096, split=8) == L.IQD_ERR_WORKSPACE      # 16-leaf subtrees
    assert call(K=4096, split=4) == L.IQD_ERR_WORKSPACE
    assert call(ql=3 * A + 8) == L.IQD_ERR_ALIGN
    assert call(qh=4 * A + 4) == L.IQD_ERR_ALIGN
    assert call(d=7 * A + 1) == L.IQD_ERR_ALIGN
    assert call(y=3 * A + 2048) == L.IQD_ERR_INVALID        # output overlaps the low plane
    assert call(ql=0) == L.IQD_ERR_INVALID
    assert iqd.workspace_bytes(L.IQD_OP_KQ6, 8, 4096, 12288, 16) == 16 * 8 * 4096 * 4
    assert iqd.workspace_bytes(L.IQD_OP_KQ6, 8, 4096, 1000, 1) == 0  # K % 256


def test_kq4_validation(lib):
    def call(b=4, N=64, K=1024, split=1, q=A, ql=3 * A, scm=4 * A, dm=6 * A, y=5 * A, ws=0, wsb=0):
        return lib.kq4_linear(ptr(q), ptr(2 * A), ptr(ql), ptr(scm), ptr(dm), b, N, K, ptr(y), split, ptr(ws), wsb,
                              None)
    assert call(K=512 + 32) == L.IQD_ERR_INVALID             # K % 256
    assert call(K=256, split=16) == L.IQD_ERR_UNSUPPORTED    # L = 8 leaves: at most 8 splits
    assert call(K=4096, split=4) == L.IQD_ERR_WORKSPACE
    assert call(scm=4 * A + 1) == L.IQD_ERR_ALIGN
    assert call(dm=6 * A + 2) == L.IQD_ERR_ALIGN
    assert call(y=4 * A + 64) == L.IQD_ERR_INVALID           # output overlaps the (sub-scale, minimum) pairs
    assert call(scm=0) == L.IQD_ERR_INVALID
    assert iqd.workspace_bytes(L.IQD_OP_KQ4, 8, 4096, 12288, 16) == 16 * 8 * 4096 * 4


def test_quantize_validation(lib):
    def call(b=2, K=64, group=0, x=A, q=2 * A, s=3 * A):
        return lib.quantize_activations(ptr(x), b, K, group, ptr(q), ptr(s), None)
    assert call(group=16) == L.IQD_ERR_INVALID
    assert call(K=48, group=32) == L.IQD_ERR_INVALID
    assert call(K=40) == L.IQD_ERR_INVALID
    assert call(b=0) == L.IQD_ERR_INVALID
    assert call(x=A + 2) == L.IQD_ERR_ALIGN
    assert call(s=3 * A + 2) == L.IQD_ERR_ALIGN
    assert call(q=A + 16) == L.IQD_ERR_INVALID               # q overlaps x


def test_lm_head_and_requant_validation(lib):
    def call(logits=6 * A, argmax=7 * A, ws=0, wsb=0, N=1000):
        return lib.lm_head_argmax(ptr(A), ptr(2 * A), ptr(3 * A), ptr(4 * A), 4, N, 256, ptr(logits), ptr(argmax),
                                  ptr(ws), wsb, None)
    assert call(argmax=0) == L.IQD_ERR_INVALID
    assert call(logits=0) == L.IQD_ERR_WORKSPACE             # no logits buffer -> workspace needed
    assert call(argmax=7 * A + 2) == L.IQD_ERR_ALIGN
    assert lib.pow2_requantize(ptr(A), ptr(2 * A), 0, 16, ptr(3 * A), ptr(4 * A), None) == L.IQD_ERR_INVALID
    assert lib.pow2_requantize(ptr(A), ptr(2 * A), 4, 16, ptr(A + 8), ptr(4 * A), None) == L.IQD_ERR_INVALID


def test_python_binding_refuses_cpu_tensors():
    import torch

    q = torch.zeros((2, 64), dtype=torch.int8)
    with pytest.raises(ValueError, match="GPU"):
        iqd.w8a8_linear(q, torch.zeros(2), torch.zeros((8, 64), dtype=torch.int8), torch.zeros(8))


def test_w8a8_bf16_validation(lib):
    def call(x=A, w=2 * A, sw=3 * A, b=4, N=64, K=1024, y=4 * A, q=5 * A, s=6 * A, ws=0, wsb=0):
        return lib.w8a8_linear_bf16(ptr(x), ptr(w), ptr(sw), b, N, K, ptr(y), ptr(q), ptr(s), ptr(ws), wsb, None)
    assert call(x=0) == L.IQD_ERR_INVALID
    assert call(K=1000) == L.IQD_ERR_INVALID                  # K % 16
    assert call(K=131072) == L.IQD_ERR_RANGE
    assert call(x=A + 8) == L.IQD_ERR_ALIGN                   # x needs 16 bytes
    assert call(q=5 * A + 4) == L.IQD_ERR_ALIGN
    assert call(y=A + 64) == L.IQD_ERR_INVALID                # y overlaps x
    assert call(b=40, q=0) == L.IQD_ERR_WORKSPACE             # b > 16: separate quantization needs q space
    ws = iqd.workspace_bytes(L.IQD_OP_W8A8_BF16, 40, 64, 1024, 1)
    assert ws == 40 * 1024 + (40 * 4 + 15) // 16 * 16


def attn(lib, q=A, k=2 * A, v=3 * A, out=4 * A, ws=0, wsb=0, kc=1024, kh=128, vc=1024, vh=128, b=2, Hq=32, Hkv=8,
         D=128, pos0=10, scale=0.088):
    return lib.attn_decode(ptr(q), ptr(k), ptr(v), kc, kh, vc, vh, b, Hq, Hkv, D, pos0, scale, ptr(out), ptr(ws), wsb,
                           None)


def test_attn_validation(lib):
    assert attn(lib, q=0) == L.IQD_ERR_INVALID
    assert attn(lib, b=0) == L.IQD_ERR_INVALID
    assert attn(lib, Hq=30) == L.IQD_ERR_INVALID              # not a multiple of Hkv
    assert attn(lib, pos0=-1) == L.IQD_ERR_INVALID
    assert attn(lib, scale=float("nan")) == L.IQD_ERR_INVALID
    assert attn(lib, scale=float("inf")) == L.IQD_ERR_INVALID
    assert attn(lib, D=64) == L.IQD_ERR_UNSUPPORTED
    assert attn(lib, Hq=64, Hkv=2) == L.IQD_ERR_UNSUPPORTED   # 32 query heads per kv head
    assert attn(lib, q=A + 8) == L.IQD_ERR_ALIGN
    assert attn(lib, kc=1020) == L.IQD_ERR_ALIGN               # rows not 16-byte aligned
    assert attn(lib, vh=4) == L.IQD_ERR_ALIGN
    assert attn(lib, vc=1 << 22) == L.IQD_ERR_UNSUPPORTED      # a chunk would span 2 GB
    assert attn(lib, kc=64) == L.IQD_ERR_INVALID                # cells would overlap
    assert attn(lib, pos0=300) == L.IQD_ERR_WORKSPACE          # two chunks need partials
    need = iqd.attn_workspace_bytes(2, 32, 8, 128, 300)
    assert need == (2 * 32 * 2 * 2 * 4 + 255) // 256 * 256 + 2 * 32 * 2 * 128 * 4
    assert attn(lib, pos0=300, ws=5 * A, wsb=need - 16) == L.IQD_ERR_WORKSPACE
    assert attn(lib, out=A + 64) == L.IQD_ERR_INVALID          # output overlaps q
    assert iqd.attn_workspace_bytes(2, 32, 8, 128, 10) == 0    # one chunk: the fast path
    assert iqd.attn_workspace_bytes(2, 32, 8, 64, 300) == 0    # rejected shape


def fp8(lib, b=4, N=64, K=256, split=1, q=A, sa=2 * A, w=3 * A, sw=4 * A, y=5 * A, ws=0, wsb=0):
    return lib.fp8_linear(ptr(q), ptr(sa), ptr(w), ptr(sw), b, N, K, ptr(y), split, ptr(ws), wsb, None)


def test_fp8_validation(lib):
    assert fp8(lib, q=0) == L.IQD_ERR_INVALID
    assert fp8(lib, K=40) == L.IQD_ERR_INVALID                # K % 16
    assert fp8(lib, K=131072) == L.IQD_ERR_RANGE
    assert fp8(lib, split=3) == L.IQD_ERR_UNSUPPORTED
    assert fp8(lib, K=1024, split=2) == L.IQD_ERR_UNSUPPORTED  # 64 leaves: one chunk, no split
    assert fp8(lib, K=2048, split=2) == L.IQD_ERR_WORKSPACE
    assert fp8(lib, b=17, K=2048, split=2) == L.IQD_ERR_UNSUPPORTED
    assert fp8(lib, q=A + 8) == L.IQD_ERR_ALIGN
    assert iqd.workspace_bytes(L.IQD_OP_FP8, 4, 64, 2048, 2) == 2 * 4 * 64 * 4
    assert iqd.workspace_bytes(L.IQD_OP_FP8, 4, 64, 2048, 1) == 0
    assert lib.quantize_fp8(ptr(A), 2, 40, ptr(2 * A), ptr(3 * A), None) == L.IQD_ERR_INVALID
    assert lib.quantize_fp8(ptr(A), 2, 64, ptr(A + 32), ptr(3 * A), None) == L.IQD_ERR_INVALID  # q overlaps x
