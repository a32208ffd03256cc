"""GPU parity of the FP8 (E4M3) W8A8 path (tolerance 0 ulp): the per-token
quantizer bit for bit (including ties at E4M3 midpoints and saturation),
the linear layer against the oracle over ragged K and N, every b from 1 to
33 and every allowed split, the tree and group-order witnesses, and
Qwen3-8B shapes with every b equal to b = 1."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import assert_bits_equal, dev, host, host_bits, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def iqd():
    import invariant_quantized_decode_token_amd as m

    m.load()
    return m


def splits_for(K):
    G = K // 16
    L = 1
    while L < G:
        L *= 2
    return [s for s in (1, 2, 4, 8, 16, 32, 64) if s == 1 or 64 * s <= L]


def test_quantizer_bitwise(iqd):
    g = W.rng(41)
    x = W.normal_bf16(g, 6, 4096)
    x, _ = W.add_outlier_channels(g, x)
    ties = np.zeros((3, 64), np.float32)
    # token 3: amax 448 (s = 1); every gap between consecutive E4M3 magnitudes
    # from 2^-9 to 448 at its midpoint (ties go to the even code), both signs
    vals = sorted({float(oracle.e4m3_to_f32(c)) for c in range(0x7F)})
    mids = [(a + b) / 2 for a, b in zip(vals, vals[1:])]
    ties_t = np.zeros((1, 256), np.float32)
    ties_t[0, 0] = 448.0
    assert len(mids) == 126
    ties_t[0, 1:1 + len(mids)] = mids
    ties_t[0, 128:128 + len(mids)] = [-m for m in mids]
    tb = W.f32_to_bf16_bits(ties_t)
    assert np.array_equal(W.bf16_bits_to_f32(tb), ties_t)  # midpoints are bf16 values
    for xb in (x, tb, W.f32_to_bf16_bits(ties)):
        oq, osa = oracle.quantize_fp8(xb)
        q, sa = iqd.quantize_fp8(dev(xb))
        assert_bits_equal(host(q), oq, "codes")
        assert_bits_equal(host(sa).view(np.uint32), osa.view(np.uint32), "scales")


def case(K, N=37, b=16, seed=0):
    g = W.rng(1000 * K + seed)
    w = W.e4m3_weight_codes(g, N, K)
    s_w = W.log_uniform_scales(g, N, 1e-5, 1e-3)
    x = W.normal_bf16(g, b, K)
    q, s_a = oracle.quantize_fp8(x)
    return q, s_a, w, s_w


@pytest.mark.parametrize("K", [16, 32, 48, 112, 592, 1040, 2048, 4096, 12288])
def test_oracle_parity_ragged(iqd, K):
    q, s_a, w, s_w = case(K)
    oy = oracle.fp8_linear(q, s_a, w, s_w)
    qd, sad, wd, swd = dev(q), dev(s_a), dev(w), dev(s_w)
    for b in (1, 2, 3, 5, 8, 11, 16):
        y = iqd.fp8_linear(qd[:b], sad[:b], wd, swd)
        assert_bits_equal(host_bits(y), oy[:b], f"K={K} b={b}")
    for split in splits_for(K):
        y = iqd.fp8_linear(qd[:5], sad[:5], wd, swd, split_k=split)
        assert_bits_equal(host_bits(y), oy[:5], f"K={K} split={split}")


def test_more_than_sixteen_tokens(iqd):
    q, s_a, w, s_w = case(1040, b=33, seed=3)
    oy = oracle.fp8_linear(q, s_a, w, s_w)
    y = iqd.fp8_linear(dev(q), dev(s_a), dev(w), dev(s_w))
    assert_bits_equal(host_bits(y), oy, "b=33")


def code(v):
    c = oracle.f32_to_e4m3(v)
    assert float(oracle.e4m3_to_f32(c)) == v
    return c


def test_witnesses(iqd):
    """The oracle's witnesses on the GPU: group sums [A, 2^-4, -A, 2^-4]
    (A = 1.5 * 2^20) give 0 only under the adjacent-pair tree; products
    [2^16, 2^-8, -2^16, 2^-8] give 2^-8 only when a group adds in order.
    Repeated across the row at offsets that put them inside one chunk, across
    chunks and at the padding edge."""
    K = 16 * 600  # 600 groups: 1024 leaves, the last 424 padding
    rows = []
    for start in (0, 60, 64, 124, 512, 596):
        q = np.zeros(K, np.uint8)
        w = np.zeros(K, np.uint8)
        g0 = start
        q[16 * g0:16 * g0 + 16], w[16 * g0:16 * g0 + 16] = code(384.0), code(256.0)
        q[16 * (g0 + 1)], w[16 * (g0 + 1)] = code(0.25), code(0.25)
        q[16 * (g0 + 2):16 * (g0 + 3)], w[16 * (g0 + 2):16 * (g0 + 3)] = code(384.0), code(-256.0)
        q[16 * (g0 + 3)], w[16 * (g0 + 3)] = code(0.25), code(0.25)
        rows.append((q, w))
    q2 = np.zeros(K, np.uint8)
    w2 = np.zeros(K, np.uint8)
    for i, (a, b_) in enumerate([(256.0, 256.0), (0.0625, 0.0625), (256.0, -256.0), (0.0625, 0.0625)]):
        q2[16 * 7 + i], w2[16 * 7 + i] = code(a), code(b_)
    rows.append((q2, w2))
    # one token row per case against its own weight row: use a diagonal layout
    n = len(rows)
    Q = np.stack([r[0] for r in rows])
    Wm = np.stack([r[1] for r in rows])
    one_a = np.ones(n, np.float32)
    one_w = np.ones(n, np.float32)
    oy = oracle.fp8_linear(Q, one_a, Wm, one_w)
    for i in range(n - 1):
        assert oy[i, i] == 0x0000, i
    assert W.bf16_bits_to_f32(oy[n - 1:, n - 1])[0] == 2.0 ** -8
    for split in splits_for(K):
        y = iqd.fp8_linear(dev(Q), dev(one_a), dev(Wm), dev(one_w), split_k=split)
        assert_bits_equal(host_bits(y), oy, f"witnesses split={split}")


@pytest.mark.parametrize("li", range(4))
def test_qwen3_8b_invariance_and_parity(iqd, li):
    t = torch()
    L = W.fp8_layer(li, tokens=16)
    q, s_a = iqd.quantize_fp8(dev(L.x))
    oq, osa = oracle.quantize_fp8(L.x)
    assert_bits_equal(host(q), oq, f"{L.name} codes")
    wd, swd = dev(L.w), dev(L.s_w)
    one = t.empty((16, L.N), dtype=t.bfloat16, device="cuda")
    for i in range(16):
        iqd.fp8_linear(q[i:i + 1], s_a[i:i + 1], wd, swd, y=one[i:i + 1])
    ref = host_bits(one)
    assert_bits_equal(ref, oracle.fp8_linear(oq, osa, L.w, L.s_w), f"{L.name} b=1 vs oracle, all rows")
    for b in range(2, 17):
        out = t.empty((16, L.N), dtype=t.bfloat16, device="cuda")
        for t0 in range(0, 16, b):
            t1 = min(16, t0 + b)
            iqd.fp8_linear(q[t0:t1], s_a[t0:t1], wd, swd, y=out[t0:t1])
        assert_bits_equal(host_bits(out), ref, f"{L.name} b={b}")
    for split in splits_for(L.K):
        y = iqd.fp8_linear(q[:8], s_a[:8], wd, swd, split_k=split)
        assert_bits_equal(host_bits(y), ref[:8], f"{L.name} split={split}")
