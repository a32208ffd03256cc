"""Pins of the oracle's kq4 superblock linear layer (4-bit codes, a sub-scale
and a minimum per 32 weights, fp16 d and dmin per 256): two reductions to the
pinned block-quantized oracle (zero minimums, where each block is the q8_0
leaf on weights sc * q; zero sub-scales, where each block is the q8_0 leaf on
weights -m with dmin as the scale), an exact closed form with power-of-two
scales, and the range check of the 6-bit fields.

Sources: "why speculative decoding changed my output", opening (Qwen3-8B at
q4_k_m) and section "the mat-vec kernel" (int8 activation blocks of 32, exact
integer products, each block's integer result scaled into fp32).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as W
from exact import bf16, bf16_bits_of


def operands(seed, b, N, K, sc_hi=63, m_hi=63):
    g = W.rng(seed)
    codes, scm, dm = W.kq4_weights(g, N, K)
    scm[..., 0] = g.integers(0, sc_hi + 1, scm.shape[:2])
    scm[..., 1] = g.integers(0, m_hi + 1, scm.shape[:2])
    x = W.normal_bf16(g, b, K)
    q, d_a = oracle.quantize_block32(x)
    return codes, scm, dm, q, d_a


@pytest.mark.parametrize("K", [256, 1280, 4096])
def test_zero_minimums_reduce_to_blockq8(K):
    """m = 0: the minimum term is fl(fl(0 * d_a) * dmin) = +0 and p - (+0) = p,
    so each leaf is the q8_0 leaf of weights sc_j * q_k (sub-scales up to 8
    keep them within int8) with d as the block scale."""
    codes, scm, dm, q, d_a = operands(K, 3, 29, K, sc_hi=8, m_hi=0)
    got = oracle.kq4_linear(q, d_a, W.kq4_pack(codes), scm, dm)
    w = (np.repeat(scm[..., 0], 32, axis=1).astype(np.int16) * codes).astype(np.int8)
    want = oracle.blockq8(q, d_a, w, np.repeat(dm[..., 0], 8, axis=1))
    assert np.array_equal(got, want)


@pytest.mark.parametrize("K", [256, 1280])
def test_zero_subscales_reduce_to_blockq8_of_the_minimums(K):
    """sc = 0: each leaf is +0 - fl(fl(fl32(m_j * sum a) * d_a) * dmin), the
    exact negation of the q8_0 leaf of weights -m_j over the block with dmin
    as the block scale."""
    codes, scm, dm, q, d_a = operands(K + 7, 4, 23, K, sc_hi=0, m_hi=63)
    got = oracle.kq4_linear(q, d_a, W.kq4_pack(codes), scm, dm)
    w = -np.repeat(scm[..., 1], 32, axis=1).astype(np.int8)
    want = oracle.blockq8(q, d_a, w, np.repeat(dm[..., 1], 8, axis=1))
    assert np.array_equal(got, want)


def test_power_of_two_scales_give_the_exact_sum():
    """d = 2^-3, dmin = 2^-4, d_a = 2^-5, small codes and activations: both
    terms of every leaf, the leaves and every partial sum are multiples of
    2^-9 far below 2^24 units, so y = bf16 of the exact value
    sum_j (sc_j * sum q a * 2^-8 - m_j * sum a * 2^-9)."""
    g = W.rng(9)
    b, N, K = 2, 5, 512
    codes = g.integers(0, 16, (N, K), dtype=np.uint8)
    scm = g.integers(0, 64, (N, K // 32, 2), dtype=np.uint8)
    q = g.integers(-3, 4, (b, K), dtype=np.int8)
    dm = np.zeros((N, K // 256, 2), np.uint16)
    dm[..., 0] = 0x3000   # fp16 2^-3
    dm[..., 1] = 0x2C00   # fp16 2^-4
    d_a = np.full((b, K // 32), 2.0 ** -5, np.float32)
    got = oracle.kq4_linear(q, d_a, W.kq4_pack(codes), scm, dm)
    for t in range(b):
        for n in range(N):
            tot = Fraction(0)
            for j in range(K // 32):
                blk = slice(32 * j, 32 * j + 32)
                qa = int((codes[n, blk].astype(np.int64) * q[t, blk]).sum())
                asum = int(q[t, blk].astype(np.int64).sum())
                tot += Fraction(int(scm[n, j, 0]) * qa, 2 ** 8) - Fraction(int(scm[n, j, 1]) * asum, 2 ** 9)
            assert got[t, n] == bf16_bits_of(float(bf16(tot))), (t, n)  # an exact 0 is +0 under RNE


def test_six_bit_fields_are_range_checked():
    codes, scm, dm, q, d_a = operands(1, 1, 2, 256)
    scm[1, 3, 1] = 64
    with pytest.raises(oracle.OracleError):
        oracle.kq4_linear(q, d_a, W.kq4_pack(codes), scm, dm)
