"""Pins of the oracle's kq6 superblock linear layer against what fixes it
from outside: the two bit planes against bytes worked out by hand from the
layout, the packer against the oracle's decoder, two reductions to the
block-quantized oracle (unit sub-scales; small sub-scales folded into int8
weights), an exact closed form with power-of-two scales, the 2^24 extreme of
a block's integer sum, and the canonical tree's witness built from kq6
operands.

Sources: "why speculative decoding changed my output", section "the mat-vec
kernel" (q6_k rows as weight blocks of 256 against int8 activation blocks of
32, exact integer products, each block's integer result scaled into fp32).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as W
from exact import bf16, bf16_bits_of

FP16_ONE = 0x3C00


def planes(codes):
    return W.kq6_pack(np.asarray(codes, np.int8))


def test_planes_match_bytes_worked_by_hand():
    """All codes 0 (u = 32 = 0b10_0000): every low byte 0x00, every high byte
    0b10101010.  Weight 131 = 16 * 8 + 3 set to 31 (u = 63 = 0b11_1111): low
    byte 8 * 8 + 3 = 67 gets 0xF in its lower nibble (3 < 8); high byte
    4 * 8 + 3 = 35 gets 0b11 in bits 0-1 (3 / 4 = 0).  Weight 261 = 16 * 16 +
    5 set to -32 (u = 0): low byte 128 + 5 keeps 0x00, high byte 64 + 1 = 65
    gets 0b00 in bits 2-3 (5 / 4 = 1)."""
    c = np.zeros((1, 512), np.int8)
    ql, qh = planes(c)
    assert (ql == 0x00).all() and (qh == 0xAA).all()
    c[0, 131] = 31
    c[0, 261] = -32
    ql, qh = planes(c)
    want_ql = np.zeros(256, np.uint8)
    want_ql[67] = 0x0F
    want_qh = np.full(128, 0xAA, np.uint8)
    want_qh[35] = 0xAB                     # 0b10_10_10_11
    want_qh[65] = 0xA2                     # 0b10_10_00_10
    assert np.array_equal(ql[0], want_ql)
    assert np.array_equal(qh[0], want_qh)
    assert np.array_equal(oracle.kq6_decode(ql, qh), c)


def test_decoder_inverts_the_packer_for_every_code():
    g = W.rng(11)
    c = g.integers(-32, 32, (7, 1024), dtype=np.int8)
    c[0, :64] = np.arange(-32, 32)         # every code once
    ql, qh = planes(c)
    assert np.array_equal(oracle.kq6_decode(ql, qh), c)


def operands(seed, b, N, K, sc_lo=-127, sc_hi=127):
    g = W.rng(seed)
    codes = g.integers(-32, 32, (N, K), dtype=np.int8)
    sc = g.integers(sc_lo, sc_hi + 1, (N, K // 16), dtype=np.int8)
    d = np.exp(g.uniform(np.log(1e-6), np.log(1e-4), (N, K // 256))).astype(np.float16).view(np.uint16)
    x = W.normal_bf16(g, b, K)
    q, d_a = oracle.quantize_block32(x)
    return codes, sc, d, q, d_a


@pytest.mark.parametrize("K", [256, 768, 4096])
def test_unit_subscales_reduce_to_blockq8(K):
    """sc = 1 everywhere: each block's integer sum is the q8_0 one with the
    codes as weights, and its weight scale is its superblock's d."""
    codes, _, d, q, d_a = operands(K, 3, 37, K)
    sc = np.ones((37, K // 16), np.int8)
    ql, qh = planes(codes)
    got = oracle.kq6_linear(q, d_a, ql, qh, sc, d)
    want = oracle.blockq8(q, d_a, codes, np.repeat(d, 8, axis=1))
    assert np.array_equal(got, want)


@pytest.mark.parametrize("K", [256, 1280])
def test_subscales_apply_per_16_weights(K):
    """Small sub-scales (|sc| <= 3, so |sc * c| <= 96 fits int8): the layer
    equals the q8_0 layer on weights sc[k / 16] * c[k]."""
    codes, sc, d, q, d_a = operands(K + 1, 4, 29, K, -3, 3)
    ql, qh = planes(codes)
    got = oracle.kq6_linear(q, d_a, ql, qh, sc, d)
    w = (np.repeat(sc, 16, axis=1).astype(np.int16) * codes).astype(np.int8)
    want = oracle.blockq8(q, d_a, w, np.repeat(d, 8, axis=1))
    assert np.array_equal(got, want)
    # and a misplaced sub-scale (one per 32 weights) would not
    w_bad = (np.repeat(sc[:, ::2], 32, axis=1).astype(np.int16) * codes).astype(np.int8)
    assert not np.array_equal(got, oracle.blockq8(q, d_a, w_bad, np.repeat(d, 8, axis=1)))


def test_power_of_two_scales_give_the_exact_sum():
    """d = 2^-3 and d_a = 2^-5 everywhere, codes and activations small: every
    leaf and every partial sum is an integer multiple of 2^-8 below 2^16, so
    the float program is exact and y = bf16(exact sum), whatever the tree."""
    g = W.rng(5)
    b, N, K = 2, 6, 768
    codes = g.integers(-32, 32, (N, K), dtype=np.int8)
    sc = g.integers(-4, 5, (N, K // 16), dtype=np.int8)
    q = g.integers(-3, 4, (b, K), dtype=np.int8)
    d = np.full((N, K // 256), 0x3000, np.uint16)   # fp16 2^-3
    d_a = np.full((b, K // 32), 2.0 ** -5, np.float32)
    ql, qh = planes(codes)
    got = oracle.kq6_linear(q, d_a, ql, qh, sc, d)
    for t in range(b):
        for n in range(N):
            w = np.repeat(sc[n], 16).astype(np.int64) * codes[n]
            exact = Fraction(int((w * q[t]).sum()), 2 ** 8)
            assert got[t, n] == bf16_bits_of(float(bf16(exact))), (t, n)


def test_extreme_block_sum_is_exact():
    """codes -32, sub-scale -128, activations -128 over one 32-block:
    isum = 32 * 4096 * -128 = -2^24, exact in int32 and in fp32; with
    d_a = 2^-10 and d = 1 the output is -2^14 exactly."""
    K = 256
    codes = np.zeros((1, K), np.int8)
    codes[0, :32] = -32
    sc = np.zeros((1, K // 16), np.int8)
    sc[0, :2] = -128
    q = np.zeros((1, K), np.int8)
    q[0, :32] = -128
    d_a = np.full((1, K // 32), 2.0 ** -10, np.float32)
    d = np.full((1, 1), FP16_ONE, np.uint16)
    ql, qh = planes(codes)
    got = oracle.kq6_linear(q, d_a, ql, qh, sc, d)
    assert W.bf16_bits_to_f32(got)[0, 0] == -(2.0 ** 14)


def test_tree_witness_from_kq6_operands():
    """Leaves [2^27, 1, -2^27, 1, 0, 0, 0, 0] over K = 256: 2^27 from one
    weight sc * c = 64 * -16 against q = -128 (isum = 2^17) with d_a = 2^10,
    d = 1; 1 from sc = c = q = 1.  The adjacent-pair tree gives 0; adding
    left to right would give 1, pairing (x0 + x2) + (x1 + x3) would give 2."""
    K = 256
    codes = np.zeros((1, K), np.int8)
    sc = np.ones((1, K // 16), np.int8)
    q = np.zeros((1, K), np.int8)
    d_a = np.ones((1, K // 32), np.float32)
    for blk, sign in ((0, 1), (2, -1)):
        codes[0, 32 * blk] = -16 * sign
        sc[0, 2 * blk] = 64
        q[0, 32 * blk] = -128
        d_a[0, blk] = 2.0 ** 10
    for blk in (1, 3):
        codes[0, 32 * blk] = 1
        q[0, 32 * blk] = 1
    d = np.full((1, 1), FP16_ONE, np.uint16)
    ql, qh = planes(codes)
    got = oracle.kq6_linear(q, d_a, ql, qh, sc, d)
    assert got[0, 0] == 0x0000
    leaves = np.array([2.0 ** 27, 1, -(2.0 ** 27), 1, 0, 0, 0, 0], np.float32)
    assert oracle.tree_sum(leaves) == 0.0
