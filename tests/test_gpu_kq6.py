"""GPU parity of the kq6 superblock linear layer (tolerance 0 ulp): the
oracle over ragged K and N, every b from 1 to 20 (past 16 in token chunks)
and every allowed split; the tree witness at several places in the tree;
the 2^24 block extreme at the largest K; and Qwen3-8B o and down shapes with
every b equal to b = 1."""
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


def run(iqd, q, d_a, ql, qh, sc, d, split_k=1):
    return host_bits(iqd.kq6_linear(dev(q), dev(d_a), dev(ql), dev(qh), dev(sc), dev(d, "fp16"), split_k=split_k))


def case(K, N=37, b=20, seed=0):
    g = W.rng(3000 * K + seed)
    codes, sc, d = W.kq6_weights(g, N, K)
    ql, qh = W.kq6_pack(codes)
    x = W.normal_bf16(g, b, K)
    q, d_a = oracle.quantize_block32(x)
    return q, d_a, ql, qh, sc, d


@pytest.mark.parametrize("K", [256, 512, 768, 1280, 4096, 12288])
def test_oracle_parity_ragged(iqd, K):
    q, d_a, ql, qh, sc, d = case(K)
    oy = oracle.kq6_linear(q, d_a, ql, qh, sc, d)
    for b in (1, 2, 3, 5, 8, 11, 16, 20):
        assert_bits_equal(run(iqd, q[:b], d_a[:b], ql, qh, sc, d), oy[:b], f"K={K} b={b}")
    for split in splits_for(K):
        assert_bits_equal(run(iqd, q[:5], d_a[:5], ql, qh, sc, d, split), oy[:5], f"K={K} split={split}")


def test_tree_witnesses(iqd):
    """Leaves [2^27, 1, -2^27, 1] (2^27: sc * c = 64 * -16 against q = -128
    with d_a = 2^10; 1: sc = c = q = 1) at blocks p .. p + 3 of a K = 12288
    row (384 leaves, tree of 512): inside the first chunk of 32 blocks, at
    its end, across chunk slots and next to the padding.  Every other block
    is 0.  The adjacent-pair tree gives 0 for each row."""
    K = 12288
    m = K // 32
    starts = [0, 28, 32, 124, 256, 380]
    R = len(starts)
    codes = np.zeros((R, K), np.int8)
    sc = np.ones((R, K // 16), np.int8)
    d = np.full((R, K // 256), FP16_ONE, np.uint16)
    # one activation row per witness row: token r against weight row r
    q = np.zeros((R, K), np.int8)
    d_a = np.ones((R, m), np.float32)
    for r, p in enumerate(starts):
        for blk, kind in zip(range(p, p + 4), ("big+", "one", "big-", "one")):
            k = 32 * blk
            if kind == "one":
                codes[r, k], q[r, k] = 1, 1
            else:
                codes[r, k] = -16 if kind == "big+" else 16
                sc[r, k // 16] = 64
                q[r, k] = -128
                d_a[r, blk] = 2.0 ** 10
    ql, qh = W.kq6_pack(codes)
    oy = oracle.kq6_linear(q, d_a, ql, qh, sc, d)
    for r in range(R):
        assert oy[r, r] == 0x0000, r
    for split in splits_for(K):
        assert_bits_equal(run(iqd, q, d_a, ql, qh, sc, d, split), oy, f"witness split={split}")


def test_extreme_block_sums_at_the_largest_k(iqd):
    """K = 130816 (the largest multiple of 256 under the bound): every code
    -32, every sub-scale -128, every activation -128, so every block's
    integer sum is -2^24; d_a = 2^-20 makes each leaf -16 and the root
    -16 * 4088 = -65408, exact in fp32.  In bf16 that is a tie between
    -65280 and -65536, which goes to the even one, -65536.  A second row
    mixes signs."""
    K, N, b = 130816, 2, 2
    codes = np.full((N, K), -32, np.int8)
    codes[1, 1::2] = 31
    sc = np.full((N, K // 16), -128, np.int8)
    sc[1, ::3] = 127
    q = np.full((b, K), -128, np.int8)
    q[1, ::5] = 127
    d_a = np.full((b, K // 32), 2.0 ** -20, np.float32)
    d = np.full((N, K // 256), FP16_ONE, np.uint16)
    ql, qh = W.kq6_pack(codes)
    oy = oracle.kq6_linear(q, d_a, ql, qh, sc, d)
    assert W.bf16_bits_to_f32(oy)[0, 0] == -65536.0
    for split in (1, 2, 32):
        assert_bits_equal(run(iqd, q, d_a, ql, qh, sc, d, split), oy, f"extreme split={split}")


@pytest.mark.parametrize("li", range(len(W.KQ6_SHAPES)))
def test_qwen3_8b_invariance_and_parity(iqd, li):
    t = torch()
    L = W.kq6_layer(li, tokens=16)
    oq, oda = oracle.quantize_block32(L.x)
    q, d_a = iqd.quantize_activations(dev(L.x), group=32)
    qld, qhd, scd, dd = dev(L.ql), dev(L.qh), dev(L.sc), dev(L.d, "fp16")
    one = t.empty((16, L.N), dtype=t.bfloat16, device="cuda")
    for i in range(16):
        iqd.kq6_linear(q[i:i + 1], d_a[i:i + 1], qld, qhd, scd, dd, y=one[i:i + 1])
    ref = host_bits(one)
    want = oracle.kq6_linear(oq, oda, L.ql, L.qh, L.sc, L.d)
    assert_bits_equal(ref, want, f"{L.name} b=1 vs oracle, all rows")
    for b in range(2, 17):
        out = t.empty((16, L.N), dtype=t.bfloat16, device="cuda")
        for t0 in range(0, 16, b):
            t1 = min(16, t0 + b)
            iqd.kq6_linear(q[t0:t1], d_a[t0:t1], qld, qhd, scd, dd, y=out[t0:t1])
        assert_bits_equal(host_bits(out), ref, f"{L.name} b={b}")
    for split in splits_for(L.K):
        y = iqd.kq6_linear(q[:8], d_a[:8], qld, qhd, scd, dd, split_k=split)
        assert_bits_equal(host_bits(y), ref[:8], f"{L.name} split={split}")
