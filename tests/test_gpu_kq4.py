"""GPU parity of the kq4 superblock linear layer (tolerance 0 ulp): the
oracle over ragged K and N, every b from 1 to 20 and every allowed split; a
tree witness whose leaves come from both the scale term and the minimum
term; the largest fields and activations at the largest K; and Qwen3-8B o
and down shapes with every b equal to b = 1."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import assert_bits_equal, dev, host_bits, torch

pytestmark = pytest.mark.gpu

FP16_ONE = 0x3C00


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


def run(iqd, q, d_a, ql, scm, dm, split_k=1):
    return host_bits(iqd.kq4_linear(dev(q), dev(d_a), dev(ql), dev(scm), dev(dm, "fp16"), split_k=split_k))


def case(K, N=37, b=20, seed=0):
    g = W.rng(5000 * K + seed)
    codes, scm, dm = W.kq4_weights(g, N, K)
    x = W.normal_bf16(g, b, K)
    q, d_a = oracle.quantize_block32(x)
    return q, d_a, W.kq4_pack(codes), scm, dm


@pytest.mark.parametrize("K", [256, 512, 1280, 4096, 12288])
def test_oracle_parity_ragged(iqd, K):
    q, d_a, ql, scm, dm = case(K)
    oy = oracle.kq4_linear(q, d_a, ql, scm, dm)
    for b in (1, 2, 3, 5, 8, 11, 16, 20):
        assert_bits_equal(run(iqd, q[:b], d_a[:b], ql, scm, dm), oy[:b], f"K={K} b={b}")
    for split in splits_for(K):
        assert_bits_equal(run(iqd, q[:5], d_a[:5], ql, scm, dm, split), oy[:5], f"K={K} split={split}")


def test_tree_witnesses(iqd):
    """Leaves [2^27, 1, -2^27, 1] at blocks p .. p + 3 of a K = 12288 row, d =
    dmin = 1: 2^27 from the minimum term alone (sc = 0, m = 32, four
    activations -128: msum = -2^14, d_a = 2^13, leaf = 0 - (-2^27)); -2^27 from
    the scale term alone (sc = 32, four codes 8 against -128: isum = -2^17,
    d_a = 2^10, m = 0); 1 from sc = code = q = 1.  The adjacent-pair tree
    gives 0."""
    K = 12288
    m = K // 32
    starts = [0, 28, 32, 124, 256, 380]
    R = len(starts)
    codes = np.zeros((R, K), np.uint8)
    scm = np.zeros((R, m, 2), np.uint8)
    dm = np.full((R, K // 256, 2), FP16_ONE, np.uint16)
    q = np.zeros((R, K), np.int8)
    d_a = np.ones((R, m), np.float32)
    for r, p in enumerate(starts):
        for blk, kind in zip(range(p, p + 4), ("min", "one", "scale", "one")):
            k = 32 * blk
            if kind == "one":
                codes[r, k], q[r, k], scm[r, blk, 0] = 1, 1, 1
            elif kind == "min":
                scm[r, blk, 1] = 32
                q[r, k:k + 4] = -128
                d_a[r, blk] = 2.0 ** 13
            else:
                scm[r, blk, 0] = 32
                codes[r, k:k + 4] = 8
                q[r, k:k + 4] = -128
                d_a[r, blk] = 2.0 ** 10
    ql = W.kq4_pack(codes)
    oy = oracle.kq4_linear(q, d_a, ql, scm, dm)
    for r in range(R):
        assert oy[r, r] == 0x0000, r
    for split in splits_for(K):
        assert_bits_equal(run(iqd, q, d_a, ql, scm, dm, split), oy, f"witness split={split}")


def test_largest_fields_at_the_largest_k(iqd):
    """K = 130816: codes 15, sub-scales and minimums 63, activations -128 and
    127 in a pattern, the real quantizer's scales; the largest integer sums
    the format allows, every split."""
    K, N, b = 130816, 3, 2
    g = W.rng(77)
    codes = np.full((N, K), 15, np.uint8)
    codes[1] = g.integers(0, 16, K)
    scm = np.full((N, K // 32, 2), 63, np.uint8)
    scm[2, :, 1] = 0
    q = np.full((b, K), -128, np.int8)
    q[1, ::3] = 127
    d_a = np.exp(g.uniform(-12, -4, (b, K // 32))).astype(np.float32)
    dm = np.exp(g.uniform(-10, -3, (N, K // 256, 2))).astype(np.float16).view(np.uint16)
    ql = W.kq4_pack(codes)
    oy = oracle.kq4_linear(q, d_a, ql, scm, dm)
    for split in (1, 2, 32):
        assert_bits_equal(run(iqd, q, d_a, ql, scm, dm, split), oy, f"largest split={split}")


@pytest.mark.parametrize("li", range(len(W.KQ6_SHAPES)))
def test_qwen3_8b_invariance_and_parity(iqd, li):
    t = torch()
    L = W.kq4_layer(li, tokens=16)
    oq, oda = oracle.quantize_block32(L.x)
    q, d_a = iqd.quantize_activations(dev(L.x), group=32)
    qld, scmd, dmd = dev(L.ql), dev(L.scm), dev(L.dm, "fp16")
    one = t.empty((16, L.N), dtype=t.bfloat16, device="cuda")
    for i in range(16):
        iqd.kq4_linear(q[i:i + 1], d_a[i:i + 1], qld, scmd, dmd, y=one[i:i + 1])
    ref = host_bits(one)
    want = oracle.kq4_linear(oq, oda, L.ql, L.scm, L.dm)
    assert_bits_equal(ref, want, f"{L.name} b=1 vs oracle, all rows")
    for b in range(2, 17):
        out = t.empty((16, L.N), dtype=t.bfloat16, device="cuda")
        for t0 in range(0, 16, b):
            t1 = min(16, t0 + b)
            iqd.kq4_linear(q[t0:t1], d_a[t0:t1], qld, scmd, dmd, y=out[t0:t1])
        assert_bits_equal(host_bits(out), ref, f"{L.name} b={b}")
    for split in splits_for(L.K):
        y = iqd.kq4_linear(q[:8], d_a[:8], qld, scmd, dmd, split_k=split)
        assert_bits_equal(host_bits(y), ref[:8], f"{L.name} split={split}")
