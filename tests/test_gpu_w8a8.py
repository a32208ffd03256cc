"""GPU parity of activation quantization and the W8A8 linear (tolerance 0 ulp).

Every GPU result is compared bit for bit with the CPU oracle on the same
seeded inputs, and every token row at b > 1 with the same token at b = 1
(batch invariance, the property speculative verification needs)."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import assert_bits_equal, dev, host, host_bits, sample_rows, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def iqd():
    import invariant_quantized_decode_token_amd as m

    m.load()
    return m


def gpu_quant(iqd, x_bits):
    q, s = iqd.quantize_activations(dev(x_bits))
    return q, s


# ----------------------------------------------------------------------------
# quantization
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(5, 512), (3, 16), (2, 48), (4, 4112), (7, 12288), (1, 131056)])
def test_quantize_token_parity(iqd, shape):
    b, K = shape
    x = W.normal_bf16(W.rng(K + b), b, K)
    x[0, :] = 0  # an all-zero token: s = 0, q = 0
    if b > 2:
        x[1, :7] = W.f32_to_bf16_bits(np.array([1e30, -1e30, 1e-30, 3.0, -3.0, 0.0, 65504.0], np.float32))
    oq, os_ = oracle.quantize_token(x)
    q, s = gpu_quant(iqd, x)
    torch().cuda.synchronize()
    assert_bits_equal(host(q), oq, "q")
    assert_bits_equal(host(s).view(np.uint32), os_.view(np.uint32), "s_a")


@pytest.mark.parametrize("K", [512, 4096, 8192, 12288, 32768, 65536, 65552])
def test_quantize_token_edge_rows(iqd, K):
    """The standalone quantizer's kernels (one per row length class, the
    last one the two-pass kernel) on rows aimed at its quotient's fast path
    and its correctly rounded fallback: exact ties of x / s, a subnormal s
    whose reciprocal overflows, a zero row, values near the bf16 top."""
    x = _edge_rows(K)
    oq, os_ = oracle.quantize_token(x)
    q, s = gpu_quant(iqd, x)
    assert_bits_equal(host(q), oq, f"K={K} q")
    assert_bits_equal(host(s).view(np.uint32), os_.view(np.uint32), f"K={K} s_a")


def test_quantize_token_qwen3_activations(iqd):
    for i in range(4):
        L = W.qwen3_8b_layer(i, tokens=512)
        oq, os_ = oracle.quantize_token(L.x)
        q, s = gpu_quant(iqd, L.x)
        assert_bits_equal(host(q), oq, f"q {L.name}")
        assert_bits_equal(host(s).view(np.uint32), os_.view(np.uint32), f"s_a {L.name}")


@pytest.mark.parametrize("shape", [(1, 32), (3, 96), (16, 4096), (16, 12288), (5, 4128)])
def test_quantize_block32_parity(iqd, shape):
    b, K = shape
    x = W.normal_bf16(W.rng(7 * K + b), b, K)
    x[0, :32] = 0  # a zero block
    oq, od = oracle.quantize_block32(x)
    q, d = iqd.quantize_activations(dev(x), group=32)
    assert_bits_equal(host(q), oq, "q")
    assert_bits_equal(host(d).view(np.uint32), od.view(np.uint32), "d_a")


# ----------------------------------------------------------------------------
# tiny config: K=512 -> N=256, 5 tokens, b = 1..5
# ----------------------------------------------------------------------------

def test_tiny_config_all_b(iqd):
    L = W.tiny_layer()
    oq, osa = oracle.quantize_token(L.x)
    oy = oracle.w8a8(oq, osa, L.w, L.s_w)
    q, sa = gpu_quant(iqd, L.x)
    w, sw = dev(L.w), dev(L.s_w)
    for b in range(1, 6):
        for t0 in range(0, 5, b):
            t1 = min(5, t0 + b)
            y = iqd.w8a8_linear(q[t0:t1], sa[t0:t1], w, sw)
            assert_bits_equal(host_bits(y), oy[t0:t1], f"tiny b={b} t0={t0}")
        # the first b tokens as one pass
        y = iqd.w8a8_linear(q[:b], sa[:b], w, sw)
        assert_bits_equal(host_bits(y), oy[:b], f"tiny X[0:{b}]")


# ----------------------------------------------------------------------------
# ragged shapes, every b up to 16 and the b > 16 path, full oracle comparison
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("N,K", [(1, 16), (7, 48), (33, 1040), (130, 4112), (300, 12304), (67, 2064)])
def test_ragged_shapes_full_oracle(iqd, N, K):
    g = W.rng(N * 7919 + K)
    w = W.int8_weights(g, N, K)
    w[0, :16] = -128  # the ABI accepts -128
    s_w = W.log_uniform_scales(g, N)
    x = W.normal_bf16(g, 40, K)
    oq, osa = oracle.quantize_token(x)
    q, sa = gpu_quant(iqd, x)
    wd, swd = dev(w), dev(s_w)
    for b in list(range(1, 17)) + [17, 40]:
        oy = oracle.w8a8(oq[:b], osa[:b], w, s_w)
        y = iqd.w8a8_linear(q[:b], sa[:b], wd, swd)
        assert_bits_equal(host_bits(y), oy, f"N={N} K={K} b={b}")


@pytest.mark.parametrize("N,K", [(4100, 1040), (8200, 2064), (4097, 272), (24592, 4096), (4100, 12304)])
def test_matrix_core_shape_classes(iqd, N, K):
    """Shapes on both sides of the matrix-core mat-vec's launch classes (256
    and 512 tiles of 16 rows, a persistent grid past 256 workgroups), with N
    not a multiple of 16 and K not a multiple of 256, at every b <= 16;
    rows sampled against the oracle, all rows against b = 1.  The long rows
    (K = 12304, 50 MB of weights) take the dot4 kernel from b = 9, where the
    activations no longer fit the matrix-core kernel's LDS, with its
    activations read through L1 rather than staged."""
    t = torch()
    g = W.rng(N * 31 + K)
    w = W.int8_weights(g, N, K)
    s_w = W.log_uniform_scales(g, N)
    x = W.normal_bf16(g, 16, K)
    oq, osa = oracle.quantize_token(x)
    q, sa = gpu_quant(iqd, x)
    wd, swd = dev(w), dev(s_w)
    rows = np.unique(np.concatenate([sample_rows(N, 40, N), np.arange(N - 17, N)]))
    oy = oracle.w8a8(oq, osa, w[rows], s_w[rows])
    y1 = t.empty((16, N), dtype=t.bfloat16, device="cuda")
    for i in range(16):
        iqd.w8a8_linear(q[i:i + 1], sa[i:i + 1], wd, swd, y=y1[i:i + 1])
    ref = host_bits(y1)
    assert_bits_equal(ref[:, rows], oy, f"N={N} K={K} b=1 vs oracle")
    for b in range(2, 17):
        y = iqd.w8a8_linear(q[:b], sa[:b], wd, swd)
        assert_bits_equal(host_bits(y), ref[:b], f"N={N} K={K} b={b} vs b=1")


# The three tile classes of the matrix-core GEMM for b > 16, with token and
# row counts that are no multiple of any tile: 64 x 128 tiles (at most one
# round of them, K <= 8192: three M tiles, 8 stages plus a ragged one),
# 128 x 64 tiles with a 5-stage ring (the same for longer rows: 64 stages
# plus a ragged one) and 128 x 128 tiles (more than a round of narrow tiles;
# split 8 of the second shape moves there too).  Sampled rows against the
# oracle, every row against the mat-vec over 16-token chunks.  Every split of
# K gives the same bits, including splits left with no stage (K = 272 has
# three 128-byte stages; splits 4 and 8 leave some workgroups only zero
# partials).
@pytest.mark.parametrize("b,N,K", [(100, 20000, 272), (130, 2000, 1040), (70, 1000, 8208), (300, 33000, 272)])
def test_prefill_tile_classes_ragged(iqd, b, N, K):
    t = torch()
    g = W.rng(b * 7 + N + K)
    w = W.int8_weights(g, N, K)
    s_w = W.log_uniform_scales(g, N)
    x = W.normal_bf16(g, b, K)
    oq, osa = oracle.quantize_token(x)
    q, sa = gpu_quant(iqd, x)
    wd, swd = dev(w), dev(s_w)
    y = iqd.w8a8_linear(q, sa, wd, swd)
    rows = np.unique(np.concatenate([sample_rows(N, 24, N + b), np.arange(N - 9, N)]))
    assert_bits_equal(host_bits(y)[:, rows], oracle.w8a8(oq, osa, w[rows], s_w[rows]), f"b={b} N={N} K={K} vs oracle")
    ref = t.empty((b, N), dtype=t.bfloat16, device="cuda")
    for t0 in range(0, b, 16):
        t1 = min(b, t0 + 16)
        iqd.w8a8_linear(q[t0:t1], sa[t0:t1], wd, swd, y=ref[t0:t1])
    assert_bits_equal(host_bits(y), host_bits(ref), f"b={b} N={N} K={K} vs mat-vec")
    for split in (2, 4, 8):
        ys = iqd.w8a8_linear(q, sa, wd, swd, split_k=split)
        assert_bits_equal(host_bits(ys), host_bits(ref), f"b={b} N={N} K={K} split={split}")


@pytest.mark.parametrize("b", [3, 20])
def test_max_k_and_extreme_codes(iqd, b):
    """K = 131056 (the largest multiple of 16 under the bound) with every
    product at (-128)*(-128): acc = 2147287040, close to 2^31.  b = 3 takes
    the mat-vec, b = 20 the tiled matrix-core path (and its K splits)."""
    K, N = 131056, 4
    q = np.full((b, K), -128, np.int8)
    q[1::3] = 127
    q[2::3, ::2] = 0
    w = np.full((N, K), -128, np.int8)
    w[1] = 127
    s_a = np.resize(np.array([1e-9, 2.5e-3, 1.0], np.float32), b)
    s_w = np.array([1e-3, 3e-2, 0.5, 1e-5], np.float32)
    oy = oracle.w8a8(q, s_a, w, s_w)
    y = iqd.w8a8_linear(dev(q), dev(s_a), dev(w), dev(s_w))
    assert_bits_equal(host_bits(y), oy, "max K")
    for split in (2, 4, 64):
        y = iqd.w8a8_linear(dev(q), dev(s_a), dev(w), dev(s_w), split_k=split)
        assert_bits_equal(host_bits(y), oy, f"max K split {split}")


def test_split_k_matches_oracle(iqd):
    g = W.rng(99)
    N, K = 200, 4096
    w = W.int8_weights(g, N, K)
    s_w = W.log_uniform_scales(g, N)
    x = W.normal_bf16(g, 16, K)
    oq, osa = oracle.quantize_token(x)
    q, sa = gpu_quant(iqd, x)
    for b in (1, 3, 8, 16):
        oy = oracle.w8a8(oq[:b], osa[:b], w, s_w)
        for split in (1, 2, 4, 8, 16, 64):
            y = iqd.w8a8_linear(q[:b], sa[:b], dev(w), dev(s_w), split_k=split)
            assert_bits_equal(host_bits(y), oy, f"b={b} split={split}")


def test_errors_write_nothing(iqd):
    t = torch()
    g = W.rng(5)
    N, K = 64, 256
    q = dev(W.int8_weights(g, 4, K))
    sa = dev(W.log_uniform_scales(g, 4))
    w = dev(W.int8_weights(g, N, K))
    sw = dev(W.log_uniform_scales(g, N))
    y = t.full((4, N), 7.0, dtype=t.bfloat16, device="cuda")
    before = host_bits(y).copy()
    with pytest.raises(iqd.IqdError):
        iqd.w8a8_linear(q, sa, w, sw, split_k=3, y=y)
    with pytest.raises(iqd.IqdError):
        iqd.w8a8_linear(q, sa, w, sw, split_k=2, y=y, workspace=t.empty(16, dtype=t.uint8, device="cuda"))
    t.cuda.synchronize()
    assert_bits_equal(host_bits(y), before, "canary")


# ----------------------------------------------------------------------------
# Qwen3-8B-shaped decode layers: b = 1..8 (all rows vs the oracle), b = 512, split-K
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("li", range(4))
def test_qwen3_8b_layer_invariance_and_parity(iqd, li):
    t = torch()
    L = W.qwen3_8b_layer(li, tokens=512)
    T, N = L.x.shape[0], L.N
    oq, osa = oracle.quantize_token(L.x)
    q, sa = gpu_quant(iqd, L.x)
    w, sw = dev(L.w), dev(L.s_w)
    # b = 1 for every token: the reference rows
    y1 = t.empty((T, N), dtype=t.bfloat16, device="cuda")
    for i in range(T):
        iqd.w8a8_linear(q[i:i + 1], sa[i:i + 1], w, sw, y=y1[i:i + 1])
    ref = host_bits(y1)
    # every output of the 64-token verify window against the oracle; the
    # rest of the 512 prefill tokens on sampled rows
    assert_bits_equal(ref[:64], oracle.w8a8(oq[:64], osa[:64], L.w, L.s_w), f"{L.name} b=1 vs oracle, all rows")
    rows = sample_rows(N, 48, 2001 + li)
    oy = oracle.w8a8(oq[64:], osa[64:], L.w[rows], L.s_w[rows])
    assert_bits_equal(ref[64:, rows], oy, f"{L.name} b=1 vs oracle, tokens 64-511 sampled rows")
    # speculative-verify widths over the first 64 positions
    for b in range(2, 9):
        out = t.empty((64, N), dtype=t.bfloat16, device="cuda")
        for t0 in range(0, 64, b):
            t1 = min(64, t0 + b)
            iqd.w8a8_linear(q[t0:t1], sa[t0:t1], w, sw, y=out[t0:t1])
        assert_bits_equal(host_bits(out), ref[:64], f"{L.name} b={b} vs b=1")
    # split-K at b = 8
    for split in (2, 4, 8):
        y = iqd.w8a8_linear(q[:8], sa[:8], w, sw, split_k=split)
        assert_bits_equal(host_bits(y), ref[:8], f"{L.name} split={split}")
    # prefill: all 512 tokens in one pass, twice (run-to-run bitwise), and
    # with K split over 2 and 4 workgroups per tile
    y512 = iqd.w8a8_linear(q, sa, w, sw)
    assert_bits_equal(host_bits(y512), ref, f"{L.name} b=512 vs b=1")
    y512b = iqd.w8a8_linear(q, sa, w, sw)
    assert_bits_equal(host_bits(y512b), ref, f"{L.name} b=512 second run")
    for split in (2, 4):
        ys = iqd.w8a8_linear(q, sa, w, sw, split_k=split)
        assert_bits_equal(host_bits(ys), ref, f"{L.name} b=512 split={split}")


# ----------------------------------------------------------------------------
# w8a8_linear_bf16: quantization fused into the mat-vec (one kernel for b <= 16)
# ----------------------------------------------------------------------------

def _f32_bits_to_bf16(values):
    """Exact bf16 bit patterns of values that bf16 represents exactly."""
    a = np.asarray(values, np.float32)
    bits = W.f32_to_bf16_bits(a)
    assert np.array_equal(W.bf16_bits_to_f32(bits), a), "not exactly representable in bf16"
    return bits


def _edge_rows(K):
    """Token rows aimed at the fused quantizer's two paths: exact ties of
    x / s (the correctly rounded division decides), scales whose reciprocal
    overflows (subnormal s), a zero row (s = 0), values near the bf16 top."""
    rows = np.zeros((8, K), np.uint16)
    # 1: s = 1 exactly (amax 127); ties k + 1/2 both signs
    r = np.zeros(K, np.float32)
    r[0] = 127.0
    ties = np.array([0.5, 1.5, 2.5, 3.5, 62.5, 63.5, 125.5, 126.5], np.float32)
    r[1:1 + 16] = np.concatenate([ties, -ties])
    rows[1] = _f32_bits_to_bf16(r)
    # 2: s = 2^-3 exactly (amax 15.875); ties on that grid
    r = np.zeros(K, np.float32)
    r[5] = -15.875
    r[9:9 + 8] = (np.array([0.5, 1.5, 2.5, 7.5, 100.5, 101.5, -3.5, -4.5], np.float32) * 0.125)
    rows[2] = _f32_bits_to_bf16(r)
    # 3: amax = 2^-126: s is subnormal and 1 / s overflows
    r = np.zeros(K, np.float32)
    r[0] = 2.0 ** -126
    r[1:6] = [2.0 ** -127, -2.0 ** -126, 2.0 ** -130, 3 * 2.0 ** -129, -2.0 ** -133]
    rows[3] = _f32_bits_to_bf16(r)
    # 4: amax the smallest subnormal bf16
    rows[4, 7] = 0x0001
    rows[4, 8] = 0x8001
    # 5: near the top of bf16
    r = np.zeros(K, np.float32)
    r[0] = 3.0e38
    r[1:4] = [-1.0e38, 2.5e37, 1.0]
    rows[5, :] = W.f32_to_bf16_bits(r)
    # 6, 7: N(0, 1) with 1 % outliers x 20
    g = W.rng(K + 17)
    rows[6:8] = W.normal_bf16(g, 2, K)
    return rows  # row 0 stays all zero


def _every_quotient_rows(nrows, K, seed):
    """Token rows that each hold every bf16 value of magnitude in
    [amax / 512, amax], both signs, in a seeded order, zeros after them; each
    row has its own amax (bf16, exponent uniform in [-6, 10], mantissa
    uniform). So for the row's scale s = amax / 127 every quotient x / s of
    magnitude at least 1/4 occurs, with whatever lies near a half-integer:
    the quantizers' fast path and their fallback to the correctly rounded
    division both meet every value that scale can produce."""
    g = W.rng(seed)
    rows = np.zeros((nrows, K), np.uint16)
    for i in range(nrows):
        e = int(g.integers(-6, 11))
        top = ((e + 127) << 7) | int(g.integers(0, 128))
        pos = np.arange(top - (9 << 7), top + 1, dtype=np.uint16)  # bf16 patterns order as values
        vals = np.concatenate([pos, pos | np.uint16(0x8000)])
        assert vals.size <= K
        rows[i, :vals.size] = vals[g.permutation(vals.size)]
    return rows


def test_quantize_token_every_quotient(iqd):
    """The standalone quantizer on 64 rows of every quotient of their scale
    (147,584 values), bit for bit against the oracle's division."""
    x = _every_quotient_rows(64, 2320, 4242)
    oq, os_ = oracle.quantize_token(x)
    q, s = gpu_quant(iqd, x)
    assert_bits_equal(host(q), oq, "q")
    assert_bits_equal(host(s).view(np.uint32), os_.view(np.uint32), "s_a")


@pytest.mark.parametrize("K", [2320, 4624])
def test_fused_quantizer_every_quotient(iqd, K):
    """The quantization inside the fused linear kernels on the same rows:
    K = 2320 takes the matrix-core kernel with the quantization fused in
    (b = 1..4), K = 4624 at b = 1 the dot4 kernel with it fused in (rows longer
    than 4096, no more outputs than K).  The quantized activations and scales
    it writes out, and its outputs, against the oracle."""
    t = torch()
    g = W.rng(K + 99)
    N = 64
    w = W.int8_weights(g, N, K)
    s_w = W.log_uniform_scales(g, N)
    x = _every_quotient_rows(16, K, 77 + K)
    oq, osa = oracle.quantize_token(x)
    oy = oracle.w8a8(oq, osa, w, s_w)
    xd, wd, swd = dev(x), dev(w), dev(s_w)
    for b in ((1, 2, 3, 4) if K < 4096 else (1,)):
        for t0 in range(0, 16, b):
            bb = min(b, 16 - t0)
            q_out = t.empty((bb, K), dtype=t.int8, device="cuda")
            s_out = t.empty((bb,), dtype=t.float32, device="cuda")
            y = iqd.w8a8_linear_bf16(xd[t0:t0 + bb], wd, swd, q_out=q_out, s_a_out=s_out)
            what = f"K={K} b={bb} t0={t0}"
            assert_bits_equal(host(q_out), oq[t0:t0 + bb], what + " q")
            assert_bits_equal(host(s_out).view(np.uint32), osa[t0:t0 + bb].view(np.uint32), what + " s_a")
            assert_bits_equal(host_bits(y), oy[t0:t0 + bb], what + " y")


@pytest.mark.parametrize("N,K", [(256, 512), (130, 4112), (4100, 1040), (8200, 2064), (300, 12304), (6144, 4096)])
def test_fused_bf16_matches_quantize_then_linear(iqd, N, K):
    t = torch()
    g = W.rng(N * 13 + K)
    w = W.int8_weights(g, N, K)
    s_w = W.log_uniform_scales(g, N)
    x = np.concatenate([_edge_rows(K), W.normal_bf16(g, 32, K)])  # 40 token rows
    oq, osa = oracle.quantize_token(x)
    rows = np.arange(N)  # every output row
    oy = oracle.w8a8(oq, osa, w, s_w)
    xd, wd, swd = dev(x), dev(w), dev(s_w)
    for b in list(range(1, 17)) + [17, 40]:
        # b = 1 takes every edge row alone (ties, subnormal scale, zero row, ...)
        for t0 in (range(0, 8) if b == 1 else (0, 40 - b)) if b < 40 else (0,):
            q_out = t.empty((b, K), dtype=t.int8, device="cuda")
            s_out = t.empty((b,), dtype=t.float32, device="cuda")
            y = iqd.w8a8_linear_bf16(xd[t0:t0 + b], wd, swd, q_out=q_out, s_a_out=s_out)
            assert_bits_equal(host_bits(y)[:, rows], oy[t0:t0 + b], f"N={N} K={K} b={b} t0={t0} y")
            assert_bits_equal(host(q_out), oq[t0:t0 + b], f"N={N} K={K} b={b} t0={t0} q")
            assert_bits_equal(host(s_out).view(np.uint32), osa[t0:t0 + b].view(np.uint32), f"N={N} K={K} b={b} s")
        # without the optional outputs (the fallback path then uses the workspace)
        y2 = iqd.w8a8_linear_bf16(xd[:b], wd, swd)
        assert_bits_equal(host_bits(y2)[:, rows], oy[:b], f"N={N} K={K} b={b} no outputs")


@pytest.mark.parametrize("model", ["8B", "14B"])
def test_fused_bf16_qwen3_layers_equal_unfused(iqd, model):
    """Every Qwen3-8B and Qwen3-14B decode layer at b = 1..8 (the 14B shapes
    change launch configuration between b = 2 and b = 4): the fused call
    equals quantize_activations + w8a8_linear on all outputs."""
    layer = W.qwen3_8b_layer if model == "8B" else W.qwen3_14b_layer
    for li in range(4):
        L = layer(li, tokens=8)
        oq, osa = oracle.quantize_token(L.x)
        oy = oracle.w8a8(oq, osa, L.w, L.s_w)
        xd, wd, swd = dev(L.x), dev(L.w), dev(L.s_w)
        q, sa = iqd.quantize_activations(xd)
        for b in range(1, 9):
            ref = iqd.w8a8_linear(q[:b], sa[:b], wd, swd)
            y = iqd.w8a8_linear_bf16(xd[:b], wd, swd)
            assert_bits_equal(host_bits(y), host_bits(ref), f"{L.name} b={b}")
            assert_bits_equal(host_bits(y), oy[:b], f"{L.name} b={b} vs oracle, all rows")
