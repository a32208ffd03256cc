"""GPU parity of the block-quantized (q8_0-style) linear (tolerance 0 ulp):
oracle parity, invariance across b and split-K, tree witnesses, padding."""
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
    m = K // 32
    L = 1
    while L < m:
        L *= 2
    return [s for s in (1, 2, 4, 8, 16, 32, 64) if s <= L]


@pytest.mark.parametrize("K", [32, 64, 96, 160, 544, 1056, 2080, 4128, 8224])
def test_ragged_k_full_oracle(iqd, K):
    g = W.rng(31 * K)
    N = 37
    w, d_w = W.q8_0_weights(g, N, K)
    x = W.normal_bf16(g, 16, K)
    oq, od = oracle.quantize_block32(x)
    od[3, ::3] *= -1.0  # negative activation scales exercise -0 leaves
    q, d = dev(oq), dev(od)
    wd, dwd = dev(w), dev(d_w, "fp16")
    for b in (1, 2, 3, 7, 16, 20):
        oy = oracle.blockq8(oq[:min(b, 16)], od[:min(b, 16)], w, d_w)
        if b > 16:
            xb = np.concatenate([oq, oq[:b - 16]])
            db = np.concatenate([od, od[:b - 16]])
            oy = oracle.blockq8(xb, db, w, d_w)
            y = iqd.blockq8_linear(dev(xb), dev(db), wd, dwd)
        else:
            y = iqd.blockq8_linear(q[:b], d[:b], wd, dwd)
        assert_bits_equal(host_bits(y), oy, f"K={K} b={b}")
    for split in splits_for(K):
        y = iqd.blockq8_linear(q[:5], d[:5], wd, dwd, split_k=split)
        assert_bits_equal(host_bits(y), oracle.blockq8(oq[:5], od[:5], w, d_w), f"K={K} split={split}")


@pytest.mark.parametrize("K", [4096, 12288])
def test_tree_witnesses(iqd, K):
    m = K // 32
    rows = [[(0, 1)], [(28, 1)], [(32, 8)], [(0, 32)], [(128, 32)], [(256, 32)], [(0, 64)],
            [(0, 1), (4, 1), (64, 16)], [(96, 8), (32, 1)]]
    rows = [r for r in rows if all(p + 3 * h < m for p, h in r)]
    q, d_a, w, d_w = W.tree_witness_operands(K, rows, b=3)
    oy = oracle.blockq8(q, d_a, w, d_w)
    assert np.all(oy == 0)
    for split in splits_for(K):
        for b in (1, 3):
            y = iqd.blockq8_linear(dev(q[:b]), dev(d_a[:b]), dev(w), dev(d_w, "fp16"), split_k=split)
            assert_bits_equal(host_bits(y), oy[:b], f"witness K={K} split={split} b={b}")


@pytest.mark.parametrize("K", [96, 4096, 12288])
def test_negative_zero_padding(iqd, K):
    q, d_a, w, d_w = W.negative_zero_operands(K, N=5, b=2)
    oy = oracle.blockq8(q, d_a, w, d_w)
    for split in splits_for(K):
        y = iqd.blockq8_linear(dev(q), dev(d_a), dev(w), dev(d_w, "fp16"), split_k=split)
        assert_bits_equal(host_bits(y), oy, f"-0 K={K} split={split}")


@pytest.mark.parametrize("li", range(2))
def test_blockq8_config_invariance_and_parity(iqd, li):
    t = torch()
    L = W.blockq8_layer(li, tokens=16)
    N = L.N
    oq, od = oracle.quantize_block32(L.x)
    q, d = iqd.quantize_activations(dev(L.x), group=32)
    assert_bits_equal(host(q), oq, f"{L.name} q")
    assert_bits_equal(host(d).view(np.uint32), od.view(np.uint32), f"{L.name} d_a")
    w, dw = dev(L.w), dev(L.d_w, "fp16")
    y1 = t.empty((16, N), dtype=t.bfloat16, device="cuda")
    for i in range(16):
        iqd.blockq8_linear(q[i:i + 1], d[i:i + 1], w, dw, y=y1[i:i + 1])
    ref = host_bits(y1)
    assert_bits_equal(ref, oracle.blockq8(oq, od, L.w, L.d_w), f"{L.name} b=1 vs oracle, all rows")
    for b in range(2, 17):
        for split in splits_for(L.K):
            out = t.empty((16, N), dtype=t.bfloat16, device="cuda")
            for t0 in range(0, 16, b):
                t1 = min(16, t0 + b)
                iqd.blockq8_linear(q[t0:t1], d[t0:t1], w, dw, split_k=split, y=out[t0:t1])
            assert_bits_equal(host_bits(out), ref, f"{L.name} b={b} split={split}")


# ----------------------------------------------------------------------------
# the matrix-core kernel (taken from b = 9 on where its LDS fits): ragged K and N,
# padding-only waves, -0 padding and tree witnesses on that path
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("K", [2336, 3104, 4128, 8224])
def test_matrix_core_path_ragged(iqd, K):
    g = W.rng(77 * K)
    N = 37
    w, d_w = W.q8_0_weights(g, N, K)
    x = W.normal_bf16(g, 16, K)
    oq, od = oracle.quantize_block32(x)
    od[5, 1::4] *= -1.0
    oy = oracle.blockq8(oq, od, w, d_w)
    q, d, wd, dwd = dev(oq), dev(od), dev(w), dev(d_w, "fp16")
    for split in splits_for(K):
        y = iqd.blockq8_linear(q, d, wd, dwd, split_k=split)
        assert_bits_equal(host_bits(y), oy, f"K={K} b=16 split={split}")


# (4096, 9) and (6176, 9) take the matrix-core kernel (b >= 9, activations in
# LDS; 6176 pads 193 blocks to a 256-leaf tree), (12288, 4) the lane-pair one.
@pytest.mark.parametrize("K,b", [(4096, 9), (6176, 9), (12288, 4)])
def test_matrix_core_path_padding_and_witnesses(iqd, K, b):
    q, d_a, w, d_w = W.negative_zero_operands(K, N=5, b=b)
    oy = oracle.blockq8(q, d_a, w, d_w)
    for split in splits_for(K):
        y = iqd.blockq8_linear(dev(q), dev(d_a), dev(w), dev(d_w, "fp16"), split_k=split)
        assert_bits_equal(host_bits(y), oy, f"-0 K={K} b={b} split={split}")
    m = K // 32
    rows = [[(0, 1)], [(16, 4)], [(32, 8)], [(0, 32)], [(128, 32)], [(256, 32)], [(0, 64)], [(96, 8), (32, 1)]]
    rows = [r for r in rows if all(p + 3 * h < m for p, h in r)]
    q, d_a, w, d_w = W.tree_witness_operands(K, rows, b=b)
    oy = oracle.blockq8(q, d_a, w, d_w)
    assert np.all(oy == 0)
    for split in splits_for(K):
        y = iqd.blockq8_linear(dev(q), dev(d_a), dev(w), dev(d_w, "fp16"), split_k=split)
        assert_bits_equal(host_bits(y), oy, f"witness K={K} b={b} split={split}")
