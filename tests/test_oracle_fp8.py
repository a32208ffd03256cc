"""Pins of the oracle's FP8 (E4M3) path: the format decoded and encoded
against its definition (every code; every midpoint; brute force on random
values), the per-token quantizer's closed forms, and the linear layer's
fixed order: exact rational emulation on tiny shapes, witnesses that tell
the adjacent-pair tree and the in-group order apart from other orders, and
an exact-integer case.

Sources: "My speculative decoder got slower" ("The FP8 kernel that was
secretly FP16", "Two matmul schedules that survived"); "Deterministic LLM
Inference Across GPU Kernels ...", Abstract (FP8 differences grow with the
reduction depth).
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as W
from exact import bf16, bf16_bits_of, f32


def e4m3_def(c):
    """The OCP E4M3 value of code c as a Fraction (None for NaN)."""
    s = -1 if c & 0x80 else 1
    e, m = (c >> 3) & 15, c & 7
    if e == 15 and m == 7:
        return None
    return s * (Fraction(m, 512) if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7))


TABLE = {c: e4m3_def(c) for c in range(256)}
POS = sorted((v, c) for c, v in TABLE.items() if v is not None and c < 0x80)  # 0x00 .. 0x7E


def test_decode_every_code():
    for c in range(256):
        v = float(oracle.e4m3_to_f32(c))
        want = TABLE[c]
        if want is None:
            assert math.isnan(v)
        else:
            assert Fraction(v) == want, c
            assert math.copysign(1.0, v) == (-1.0 if c & 0x80 else 1.0)
    assert float(oracle.e4m3_to_f32(0x7E)) == 448.0 and float(oracle.e4m3_to_f32(0x01)) == 2.0 ** -9


def nearest(x: float):
    """Brute force: nearest finite E4M3 code to x (ties to the even code),
    saturating at 448; sign kept."""
    sign = 0x80 if math.copysign(1.0, x) < 0 else 0
    a = Fraction(abs(x))
    best = None
    for v, c in POS:
        d = abs(a - v)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0 and best[1] % 2 == 1):
            best = (d, c)
    return sign | best[1]


def test_encode_round_trips_midpoints_and_random_values():
    for c in range(256):
        if TABLE[c] is not None:
            assert oracle.f32_to_e4m3(float(oracle.e4m3_to_f32(c))) == c, c
    for (v0, c0), (v1, c1) in zip(POS, POS[1:]):
        mid = (v0 + v1) / 2
        assert Fraction(float(np.float32(float(mid)))) == mid  # exact in binary32
        want = c0 if c0 % 2 == 0 else c1
        assert oracle.f32_to_e4m3(float(mid)) == want, (c0, c1)
        assert oracle.f32_to_e4m3(-float(mid)) == 0x80 | want
    g = np.random.default_rng(8)
    xs = (np.exp2(g.uniform(-13, 10, 20000)) * g.choice([-1.0, 1.0], 20000)).astype(np.float32)
    for x in xs:
        assert oracle.f32_to_e4m3(float(x)) == nearest(float(x)), x
    assert oracle.f32_to_e4m3(1e9) == 0x7E and oracle.f32_to_e4m3(-463.9) == 0xFE
    assert oracle.f32_to_e4m3(0.0) == 0x00 and oracle.f32_to_e4m3(-0.0) == 0x80
    assert oracle.f32_to_e4m3(float("nan")) & 0x7F == 0x7F


def test_quantizer_closed_forms():
    x = np.zeros((3, 64), np.float32)
    x[0, 5], x[0, 9], x[0, 11] = 3.0, -3.0, 1.5
    x[2] = np.linspace(-2, 2, 64)
    bits = W.f32_to_bf16_bits(x)
    q, s = oracle.quantize_fp8(bits)
    assert s[0] == np.float32(3.0) / np.float32(448.0)
    assert q[0, 5] == 0x7E and q[0, 9] == 0xFE  # +-amax -> +-448
    assert q[0, 11] == oracle.f32_to_e4m3(float(np.float32(1.5) / s[0]))
    assert s[1] == 0.0 and np.all(q[1] == 0)
    # every code within half a spacing of x / s (the relative spacing of E4M3 normals is 2^-3)
    vals = W.bf16_bits_to_f32(bits[2]) / s[2]
    dec = np.array([float(oracle.e4m3_to_f32(c)) for c in q[2]])
    assert np.all(np.abs(dec - vals) <= np.maximum(np.abs(vals) * 2.0 ** -4, 2.0 ** -10) + 1e-12)


def linear_exact(q, s_a, w, s_w):
    """The fixed order with every binary32 operation rounded exactly."""
    b, K = q.shape
    N = w.shape[0]
    G = K // 16
    L = 1
    while L < G:
        L *= 2
    y = np.empty((b, N), np.uint16)
    for t in range(b):
        for n in range(N):
            leaves = []
            for gi in range(G):
                acc = Fraction(0)
                for k in range(16 * gi, 16 * gi + 16):
                    acc = f32(acc + TABLE[int(q[t, k])] * TABLE[int(w[n, k])])
                leaves.append(acc)
            leaves += [Fraction(0)] * (L - G)
            while len(leaves) > 1:
                leaves = [f32(leaves[2 * i] + leaves[2 * i + 1]) for i in range(len(leaves) // 2)]
            u = f32(leaves[0] * Fraction(float(s_a[t])))
            y[t, n] = bf16_bits_of(float(bf16(f32(u * Fraction(float(s_w[n]))))))
    return y


@pytest.mark.parametrize("K", [16, 32, 48, 96])
def test_linear_against_exact_emulation(K):
    g = W.rng(90 + K)
    w = W.e4m3_weight_codes(g, 3, K)
    x = W.normal_bf16(g, 2, K)
    q, s_a = oracle.quantize_fp8(x)
    s_w = W.log_uniform_scales(g, 3, 1e-5, 1e-3)
    got = oracle.fp8_linear(q, s_a, w, s_w)
    assert np.array_equal(got, linear_exact(q, s_a, w, s_w))


def code(v):
    c = oracle.f32_to_e4m3(v)
    assert float(oracle.e4m3_to_f32(c)) == v
    return c


def test_tree_witness_group_sums():
    """Group sums [A, 2^-4, -A, 2^-4] with A = 1.5 * 2^20 (16 products
    384 * 256; 2^-4 = 0.25 * 0.25).  The binary32 spacing is 2^-3 on both
    sides of A (of even significand), so A + 2^-4 and -A + 2^-4 are ties that
    round back to A and -A: the adjacent-pair tree gives 0, while adding left
    to right would give 2^-4 and pairing at stride two 2^-3."""
    K = 64
    q = np.zeros((1, K), np.uint8)
    w = np.zeros((1, K), np.uint8)
    q[0, 0:16] = code(384.0)
    w[0, 0:16] = code(256.0)
    q[0, 16], w[0, 16] = code(0.25), code(0.25)
    q[0, 32:48] = code(384.0)
    w[0, 32:48] = code(-256.0)
    q[0, 48], w[0, 48] = code(0.25), code(0.25)
    one = np.ones(1, np.float32)
    assert oracle.fp8_linear(q, one, w, one)[0, 0] == 0x0000
    assert np.array_equal(oracle.fp8_linear(q, one, w, one), linear_exact(q, one, w, one))


def test_group_order_witness():
    """Products [2^16, 2^-8, -2^16, 2^-8] inside one group, added in order:
    2^16 + 2^-8 is a tie at spacing 2^-7 and stays 2^16, so the group sum is
    2^-8 (pairwise it would be 0)."""
    q = np.zeros((1, 16), np.uint8)
    w = np.zeros((1, 16), np.uint8)
    q[0, 0], w[0, 0] = code(256.0), code(256.0)
    q[0, 1], w[0, 1] = code(0.0625), code(0.0625)
    q[0, 2], w[0, 2] = code(256.0), code(-256.0)
    q[0, 3], w[0, 3] = code(0.0625), code(0.0625)
    one = np.ones(1, np.float32)
    assert oracle.fp8_linear(q, one, w, one)[0, 0] == bf16_bits_of(2.0 ** -8)


def test_exact_integer_case():
    """Small integer values (|v| <= 8) and K = 4096: every partial sum is an
    integer below 2^24, so the root is the exact sum whatever the order, and
    with power-of-two scales y = bf16(sum * 2^(e_a + e_w))."""
    g = W.rng(7)
    K, N = 4096, 6
    vals = np.array([0, 1, 2, 3, 4, 5, 6, 7, 8], np.float32)
    codes = np.array([code(float(v)) for v in vals], np.uint8)
    iq = g.integers(-8, 9, (2, K))
    iw = g.integers(-8, 9, (N, K))
    q = np.where(iq < 0, codes[-iq] | 0x80, codes[np.abs(iq)]).astype(np.uint8)
    w = np.where(iw < 0, codes[-iw] | 0x80, codes[np.abs(iw)]).astype(np.uint8)
    s_a = np.array([2.0 ** -7, 2.0 ** 3], np.float32)
    s_w = np.ldexp(np.ones(N, np.float32), g.integers(-12, -2, N)).astype(np.float32)
    y = oracle.fp8_linear(q, s_a, w, s_w)
    exact = iq.astype(np.int64) @ iw.astype(np.int64).T
    for t in range(2):
        for n in range(N):
            want = bf16_bits_of(float(bf16(Fraction(int(exact[t, n])) * Fraction(float(s_a[t])) * Fraction(float(s_w[n])))))
            assert y[t, n] == want


def test_rows_depend_only_on_their_token():
    L = W.fp8_layer(1, tokens=8)
    w, s_w = L.w[:64], L.s_w[:64]
    q, s_a = oracle.quantize_fp8(L.x)
    full = oracle.fp8_linear(q, s_a, w, s_w)
    for t in range(8):
        assert np.array_equal(oracle.fp8_linear(q[t:t + 1], s_a[t:t + 1], w, s_w)[0], full[t])


# Chain-length witnesses.  The pages leave the K order open ("My speculative
# decoder got slower", "Two matmul schedules that survived": each schedule is
# one fixed rounding); the recipe takes chains of 16 consecutive products
# (one 16-byte load of codes), then the canonical tree over the chains.
# Products B = 2^16 (256 * 256) and s = 2^-10 (2^-5 * 2^-5): B + s rounds to B
# (spacing 2^-7 above 2^16) and -B + s rounds to -B (spacing 2^-8 below).

def _chain_case(ks, K):
    q = np.zeros((1, K), np.uint8)
    w = np.zeros((1, K), np.uint8)
    for k, (a, b) in zip(ks, ((256.0, 256.0), (2.0 ** -5, 2.0 ** -5), (256.0, -256.0), (2.0 ** -5, 2.0 ** -5))):
        q[0, k], w[0, k] = code(a), code(b)
    one = np.ones(1, np.float32)
    return oracle.fp8_linear(q, one, w, one)[0, 0]


def test_witness_chains_are_16_not_8():
    """Products at k = 7, 8, 9, 10 share one 16-chain: ((B + s) - B) + s = s,
    y = bf16(2^-10).  Chains of 8 would give B and (s - B) + s = -B, root 0."""
    assert _chain_case((7, 8, 9, 10), 16) == bf16_bits_of(2.0 ** -10)


def test_witness_chains_are_16_not_32():
    """Products at k = 15, 16, 17, 18: chain 0 ends at k = 15 (B), chain 1
    gives (s - B) + s = -B, root 0.  One 32-chain would give s."""
    assert _chain_case((15, 16, 17, 18), 32) == 0x0000
