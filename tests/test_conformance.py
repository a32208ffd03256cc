"""The fault-injection conformance suite on the CPU: the oracle is the
reference arm and the candidate arms are the canonical pipeline with one
fault injected (tests/conformance.py).  Every cell must fire exactly the
checks its row of the prediction matrix allows; the null fault fires none.

Source: "Deterministic LLM Inference Across GPU Kernels: Power-of-Two INT8
Quantization Scales and the Limits of Tolerance-Based Conformance",
Tables II-IV and Fig. 2.
"""
import ctypes

import numpy as np
import pytest

import conformance as C
import oracle
import workloads as W


def window(L, b):
    """Tokens 1..b of the layer's pool, and token 0 as the one before them."""
    q, s_a = oracle.quantize_token(L.x[:b + 1])
    return q[1:], s_a[1:], q[0], s_a[0]


def to_pow2(q, s_a, w, s_w, q_prev, s_prev):
    """Both operands requantized to power-of-two scales, codes re-rounded."""
    w2, sw2 = oracle.pow2_requant(w, s_w)
    qq, sa2 = oracle.pow2_requant(np.concatenate([q_prev[None], q]), np.concatenate([[s_prev], s_a]).astype(np.float32))
    return qq[1:], sa2[1:], w2, sw2, qq[0], sa2[0]


def layers():
    tiny = W.tiny_layer()
    o = W.qwen3_8b_layer(1, tokens=9)
    down = W.qwen3_8b_layer(3, tokens=5)
    return [
        ("tiny_b4", tiny.w, tiny.s_w, tiny, 4),
        ("o_rows1024_b8", o.w[:1024], o.s_w[:1024], o, 8),
        ("down_rows384_b4", down.w[:384], down.s_w[:384], down, 4),
    ]


LAYERS = layers()


def reference_arm(q, s_a, w, s_w):
    return C.Arm(q, s_a, w, s_w, oracle.w8a8(q, s_a, w, s_w))


def candidate(fault, q, s_a, w, s_w, q_prev, s_prev):
    if fault == "F9":
        qs, ss = C.stale_activations(q, s_a, q_prev, s_prev)
        return C.cpu_arm("null", qs, ss, w, s_w)
    return C.cpu_arm(fault, q, s_a, w, s_w)


@pytest.mark.parametrize("regime", ["real", "pow2"])
@pytest.mark.parametrize("li", range(len(LAYERS)))
def test_prediction_matrix_on_layers(li, regime):
    name, w, s_w, L, b = LAYERS[li]
    q, s_a, q_prev, s_prev = window(L, b)
    if regime == "pow2":
        q, s_a, w, s_w, q_prev, s_prev = to_pow2(q, s_a, w, s_w, q_prev, s_prev)
        _, bound = C.exact_sums(q, w)
        assert bound.max() < 2 ** 24  # F5's float sums are exact here (see the module docstring)
    ref = reference_arm(q, s_a, w, s_w)
    null = C.cpu_arm("null", q, s_a, w, s_w)
    # the suite's own canonical pipeline is the oracle's, bit for bit
    assert np.array_equal(null.y, ref.y), f"{name}: null arm differs from the oracle"
    for fault in ("null", "F1", "F2", "F3", "F4", "F5", "F9"):
        cand = candidate(fault, q, s_a, w, s_w, q_prev, s_prev)
        v = C.run_checks(ref, cand, regime)
        want = C.expected_firing(fault, regime, v)
        assert v.firing() == want, f"{name} {regime} {fault}: fired {sorted(v.firing())}, predicted {sorted(want)}"
        if fault in ("F2", "F3", "F4"):
            assert v.max_spacings <= 1, (name, regime, fault, v.max_spacings)
        if fault == "F5":
            assert C.f5_moves_explained_by_cancellation(ref, cand), name
        if fault == "F1":
            assert v.max_spacings <= 2, (name, regime, v.max_spacings)
        if fault == "F4":
            assert v.fired["bitwise"], f"{name} {regime}: truncation never observable"
        if regime == "real" and fault in ("F1", "F2", "F5") and b * w.shape[0] >= 4096:
            assert v.fired["bitwise"], f"{name}: {fault} not observable"
    C.clear_cache()


@pytest.mark.parametrize("regime", ["real", "pow2"])
def test_overflow_fault_is_caught_by_the_precondition_checks_only(regime):
    """F6: both arms are int32 pipelines fed the same over-deep operands, so
    their outputs agree bit for bit; only the checks on the operands and the
    accumulator see the fault."""
    q, s_a, w, s_w = C.overflow_operands(W.rng(606), pow2=(regime == "pow2"))
    ref = C.cpu_arm("null", q, s_a, w, s_w)
    cand = C.cpu_arm("F6", q, s_a, w, s_w)
    exact, _ = C.exact_sums(q, w)
    assert exact[0, 0] == 196608 * 16384 and cand.acc[0, 0] == 196608 * 16384 - 2 ** 32
    v = C.run_checks(ref, cand, regime)
    assert v.firing() == C.PREDICTED[("F6", regime)], sorted(v.firing())
    # the library refuses such operands outright: K past 131071 is a range error
    import invariant_quantized_decode_token_amd as iqd
    from invariant_quantized_decode_token_amd import _lib as L

    lib = iqd.load()
    A = 1 << 20  # fake aligned pointers: validation returns before any use
    p = [ctypes.c_void_p(A * i) for i in range(1, 6)]
    st = lib.w8a8_linear(p[0], p[1], p[2], p[3], 2, 6, 196608, p[4], 1, ctypes.c_void_p(0), 0, None)
    assert st == L.IQD_ERR_RANGE
    C.clear_cache()


def test_lm_head_cells_flip_only_at_small_margins():
    """(7) on an LM-head-shaped layer (4096 -> 8192 vocabulary rows, 8 tokens):
    the null fault flips nothing, a stale operand flips argmaxes, and an
    epilogue fault can flip a token only where its top two logits were
    within twice the fault's largest move."""
    L = W.w8a8_layer("lm_head_rows", 4096, 8192, W.SEED_LM_HEAD, 9, outliers=False)
    q, s_a, q_prev, s_prev = window(L, 8)
    logits, am = oracle.lm_head_argmax(q, s_a, L.w, L.s_w)
    ref = C.Arm(q, s_a, L.w, L.s_w, logits, argmax=am)
    assert np.array_equal(C.argmax_rows(logits), am)  # the suite's argmax is the oracle's
    for fault in ("null", "F1", "F2", "F3", "F4", "F5", "F9"):
        cand = candidate(fault, q, s_a, L.w, L.s_w, q_prev, s_prev)
        v = C.run_checks(ref, cand, "real", lm_head=True)
        assert v.firing() == C.expected_firing(fault, "real", v, lm_head=True), (fault, sorted(v.firing()))
        if fault == "F5":
            assert C.f5_moves_explained_by_cancellation(ref, cand)
        if fault == "null":
            assert not v.fired["token_level_risk"]
        elif fault == "F9":
            assert v.fired["token_level_risk"]
        else:
            assert C.token_flips_at_small_margins(ref, cand), fault
    C.clear_cache()


def test_check_primitives():
    """The suite's helpers on hand-made values."""
    assert C.wrap_i32(np.array([2 ** 31, -2 ** 31 - 1, 3 * 2 ** 30, 5])).tolist() == [-2 ** 31, 2 ** 31 - 1,
                                                                                      -2 ** 30, 5]
    a = np.array([0x3F80, 0x3F81, 0xBF80, 0x0000, 0x8000, 0x0001], np.uint16)  # 1, next, -1, +0, -0, min subnormal
    b = np.array([0x3F81, 0x3F80, 0x3F80, 0x8000, 0x0001, 0x8001], np.uint16)
    assert C.spacings(a, b).tolist() == [1, 1, 2 * 0x3F80, 0, 1, 2]
    assert C.is_pow2(np.array([0.5, 2.0 ** -20, 1.0], np.float32))
    assert not C.is_pow2(np.array([0.5, 0.75], np.float32))
    y = np.array([[0x3F80, 0x4000, 0x4000, 0x3F80]], np.uint16)  # tie at 2.0: lowest index
    assert C.argmax_rows(y).tolist() == [1]
    q = np.array([[1, -2, 3]], np.int8)
    w = np.array([[4, 5, -6], [-128, -128, -128]], np.int8)
    acc, bound = C.exact_sums(q, w)
    assert acc.tolist() == [[4 - 10 - 18, -128 + 256 - 384]] and bound.tolist() == [[32, 768]]
    C.clear_cache()
