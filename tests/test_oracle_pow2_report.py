"""Power-of-two weight scales on the Qwen3-14B-shaped layers, at layer level,
in the oracle: how far the outputs under the requantized weights and scales
move from those under the layer's own scales, and whether the two epilogue
orders (acc * s_a) * s_w (canonical) and acc * (s_a * s_w) (the F3 order)
agree.  Expected: they disagree on some outputs under the layer's own scales
and on none under power-of-two scales, where both scale multiplies are exact
("Deterministic LLM Inference Across GPU Kernels: Power-of-Two INT8
Quantization Scales and the Limits of Tolerance-Based Conformance", Abstract
and Table V: the agreement across kernels under pow2 scales).

The F3 order is computed here independently of the oracle: the exact integer
accumulator from a float64 matrix product (every partial sum is an integer
below 2^53, so it is exact), the scale product and the final multiply as
numpy binary32 operations (one rounding each), and bf16 rounding to nearest
even from the float32 bits.
"""
import numpy as np
import pytest

import oracle
import workloads as W

TOKENS = 64  # the verify window; F3 disagreements under own scales: 5, 1, 14, 3 (qkv, o, gate_up, down)


def bf16_rne_bits(f32: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(f32, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def f3_order(q, s_a, w, s_w):
    acc = q.astype(np.float64) @ w.astype(np.float64).T
    assert np.abs(acc).max() < 2 ** 31
    acc32 = acc.astype(np.int64).astype(np.float32)  # fl32(acc): round to nearest even
    sc = (s_a[:, None].astype(np.float32) * s_w[None, :].astype(np.float32)).astype(np.float32)
    return bf16_rne_bits((acc32 * sc).astype(np.float32))


def spacing_key(h):
    h = h.astype(np.int64)
    return np.where(h & 0x8000, -(h & 0x7FFF), h & 0x7FFF)


def report(own_bits, p2_bits):
    """pow2 vs own: max |delta| in value, share of outputs that differ, and a
    histogram of the difference in bf16 spacings (0, 1, 2-3, 4-15, >= 16)."""
    a = W.bf16_bits_to_f32(own_bits).astype(np.float64)
    b = W.bf16_bits_to_f32(p2_bits).astype(np.float64)
    d = np.abs(spacing_key(own_bits) - spacing_key(p2_bits))
    edges = [(0, 0), (1, 1), (2, 3), (4, 15), (16, 1 << 30)]
    return {
        "max_abs_delta": float(np.abs(a - b).max()),
        "pct_differ": float(100.0 * (own_bits != p2_bits).mean()),
        "spacings": {f"{lo}-{hi}" if hi < (1 << 30) else f">={lo}": int(((d >= lo) & (d <= hi)).sum())
                     for lo, hi in edges},
    }


@pytest.mark.parametrize("li", range(4))
def test_pow2_makes_the_epilogue_orders_agree(li):
    L = W.qwen3_14b_layer(li, tokens=TOKENS)
    q, s_a = oracle.quantize_token(L.x)
    own = oracle.w8a8(q, s_a, L.w, L.s_w)
    w2, s2 = oracle.pow2_requant(L.w, L.s_w)
    p2 = oracle.w8a8(q, s_a, w2, s2)
    f3_own = int((f3_order(q, s_a, L.w, L.s_w) != own).sum())
    f3_p2 = int((f3_order(q, s_a, w2, s2) != p2).sum())
    assert f3_own > 0, f"{L.name}: the F3 order never differs under the layer's own scales"
    assert f3_p2 == 0, f"{L.name}: {f3_p2} F3-order disagreements under power-of-two scales"
    r = report(own, p2)
    assert r["pct_differ"] > 0.0  # requantizing changes the layer's values
    assert sum(r["spacings"].values()) == own.size
    print(f"{L.name}: F3 disagreements own {f3_own} / {own.size}, pow2 0; pow2 vs own {r}")


def test_f3_helper_matches_a_hand_worked_case():
    """acc = 3, s_a = 1/3 (binary32), s_w = 3: canonical fl(fl(3 * fl(1/3)) * 3)
    = fl(1 * 3) = 3, while the F3 order fl(3 * fl(fl(1/3) * 3)) = 3 too; with
    s_w = 0.1 the two orders give bf16 values one spacing apart or equal, and
    the helper must match a direct binary32 evaluation."""
    q = np.array([[1, 2]], np.int8)
    w = np.array([[1, 1], [3, 0]], np.int8)
    s_a = np.array([np.float32(1) / np.float32(3)], np.float32)
    s_w = np.array([3.0, 0.1], np.float32)
    got = f3_order(q, s_a, w, s_w)
    want = [bf16_rne_bits(np.float32(3) * (s_a[0] * s_w[0]))[()], bf16_rne_bits(np.float32(3) * (s_a[0] * s_w[1]))[()]]
    assert got[0].tolist() == want
