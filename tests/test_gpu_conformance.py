"""The fault-injection conformance suite on the GPU: the library is the
reference arm; the candidate arm is a second, independently written kernel
(tests/csrc/mutant_linear.hip) with one epilogue fault switched in, or fed
stale activations (F9).  Qwen3-8B-shaped layers at b = 1 and 8 in both scale
regimes, and the LM head (4096 -> 151936) at b = 8.  Every cell must fire
exactly the checks its row of the prediction matrix allows (tests/
conformance.py); the null fault fires none, i.e. the two kernels agree bit
for bit.  (F6 is covered on the CPU: the library refuses its operands.)

Source: "Deterministic LLM Inference Across GPU Kernels: Power-of-Two INT8
Quantization Scales and the Limits of Tolerance-Based Conformance",
Tables II-IV and Fig. 2.
"""
import numpy as np
import pytest

import conformance as C
import mutants
import oracle
import workloads as W
from gpu_util import dev, host, host_bits

pytestmark = pytest.mark.gpu

FAULTS = ("null", "F1", "F2", "F3", "F4", "F5", "F9")


@pytest.fixture(scope="module")
def iqd():
    import invariant_quantized_decode_token_amd as m

    m.load()
    mutants._load()
    return m


def operands(L, b, regime):
    """Tokens 1..b (token 0 is the stale row of F9), quantized by the oracle;
    in the pow2 regime both operands requantized to power-of-two scales."""
    q, s_a = oracle.quantize_token(L.x[:b + 1])
    w, s_w = L.w, L.s_w
    if regime == "pow2":
        w, s_w = oracle.pow2_requant(w, s_w)
        q, s_a = oracle.pow2_requant(q, s_a)
    return q[1:], s_a[1:], w, s_w, q[0], s_a[0]


def gpu_candidate(fault, q, s_a, wd, swd, w, s_w, q_prev, s_prev):
    if fault == "F9":
        q, s_a = C.stale_activations(q, s_a, q_prev, s_prev)
        y, acc = mutants.linear("null", dev(q), dev(s_a), wd, swd)
    else:
        y, acc = mutants.linear(fault, dev(q), dev(s_a), wd, swd)
    return C.Arm(q, s_a, w, s_w, host_bits(y), host(acc))


@pytest.mark.parametrize("regime", ["real", "pow2"])
@pytest.mark.parametrize("li", range(4))
def test_prediction_matrix_qwen3_8b(iqd, li, regime):
    L = W.qwen3_8b_layer(li, tokens=9)
    tally = {}
    for b in (1, 8):
        print(f"conformance {L.name} {regime} b={b}", flush=True)
        q, s_a, w, s_w, q_prev, s_prev = operands(L, b, regime)
        wd, swd = dev(w), dev(s_w)
        ref = C.Arm(q, s_a, w, s_w, host_bits(iqd.w8a8_linear(dev(q), dev(s_a), wd, swd)))
        for fault in FAULTS:
            cand = gpu_candidate(fault, q, s_a, wd, swd, w, s_w, q_prev, s_prev)
            v = C.run_checks(ref, cand, regime)
            want = C.expected_firing(fault, regime, v)
            assert v.firing() == want, f"{L.name} {regime} b={b} {fault}: fired {sorted(v.firing())}, " \
                                       f"predicted {sorted(want)}"
            if fault in ("F2", "F3", "F4"):
                assert v.max_spacings <= 1
            if fault == "F1":
                assert v.max_spacings <= 2
            if fault == "F5":
                assert C.f5_moves_explained_by_cancellation(ref, cand)
            if fault == "F4":
                assert v.fired["bitwise"]
            tally[(fault, b)] = (v.fired["bitwise"], v.max_spacings)
        del wd, swd
        C.clear_cache()
    print(f"  {L.name} {regime}: (observable, max spacings) {tally}", flush=True)


def test_prediction_matrix_lm_head(iqd):
    L = W.lm_head_layer(tokens=9)
    q, s_a, w, s_w, q_prev, s_prev = operands(L, 8, "real")
    wd, swd = dev(w), dev(s_w)
    logits, am = iqd.lm_head_argmax(dev(q), dev(s_a), wd, swd)
    ref = C.Arm(q, s_a, w, s_w, host_bits(logits), argmax=host(am))
    assert np.array_equal(C.argmax_rows(ref.y), ref.argmax)
    for fault in FAULTS:
        print(f"conformance lm_head real b=8 {fault}", flush=True)
        cand = gpu_candidate(fault, q, s_a, wd, swd, w, s_w, q_prev, s_prev)
        v = C.run_checks(ref, cand, "real", lm_head=True)
        assert v.firing() == C.expected_firing(fault, "real", v, lm_head=True), (fault, sorted(v.firing()))
        if fault == "null":
            assert not v.fired["bitwise"] and not v.fired["token_level_risk"]
        elif fault == "F9":
            assert v.fired["token_level_risk"]
        else:
            assert C.token_flips_at_small_margins(ref, cand), fault
        if fault == "F5":
            assert C.f5_moves_explained_by_cancellation(ref, cand)
    C.clear_cache()
