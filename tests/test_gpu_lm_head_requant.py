"""GPU parity of the LM-head verify pass (logits + argmax) and of the
power-of-two weight-scale requantization on Qwen3-14B-shaped layers."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import assert_bits_equal, dev, host, host_bits, sample_rows, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def iqd():
    import invariant_quantized_decode_token_amd as m

    m.load()
    return m


def test_argmax_ties_small(iqd):
    """Crafted rows with exact ties at the maximum and signed zeros."""
    K, N = 32, 300
    q = np.zeros((4, K), np.int8)
    q[:, 0] = 1
    w = np.zeros((N, K), np.int8)
    s_w = np.ones(N, np.float32)
    w[[17, 40, 299], 0] = 5          # token rows 0..3 tie at 5 * s
    w[[3, 250], 0] = -3
    s_a = np.array([1.0, 0.5, -1.0, 0.0], np.float32)  # row 2: max is the -3s -> +3, rows 3: all zero
    ol, oa = oracle.lm_head_argmax(q, s_a, w, s_w)
    lg, am = iqd.lm_head_argmax(dev(q), dev(s_a), dev(w), dev(s_w))
    assert_bits_equal(host_bits(lg), ol, "tie logits")
    assert_bits_equal(host(am), oa, "tie argmax")
    assert host(am).tolist() == [17, 17, 3, 0]


def test_lm_head_small_full_oracle(iqd):
    g = W.rng(77)
    N, K = 5003, 512
    w = W.int8_weights(g, N, K)
    s_w = W.log_uniform_scales(g, N)
    x = W.normal_bf16(g, 20, K)
    oq, osa = oracle.quantize_token(x)
    for b in (1, 3, 8, 16, 20):
        ol, oa = oracle.lm_head_argmax(oq[:b], osa[:b], w, s_w)
        lg, am = iqd.lm_head_argmax(dev(oq[:b]), dev(osa[:b]), dev(w), dev(s_w))
        assert_bits_equal(host_bits(lg), ol, f"logits b={b}")
        assert_bits_equal(host(am), oa, f"argmax b={b}")
        _, am2 = iqd.lm_head_argmax(dev(oq[:b]), dev(osa[:b]), dev(w), dev(s_w), logits=False)
        assert_bits_equal(host(am2), oa, f"argmax without logits b={b}")


def test_lm_head_verify_replay(iqd):
    """64 hidden states replayed in consecutive chunks of b: 0 argmax flips and
    0 logit differences against b = 1; sampled vocab rows and two full rows
    against the oracle."""
    t = torch()
    L = W.lm_head_layer(tokens=64)
    N = L.N
    oq, osa = oracle.quantize_token(L.x)
    q, sa = iqd.quantize_activations(dev(L.x))
    assert_bits_equal(host(q), oq, "q")
    w, sw = dev(L.w), dev(L.s_w)
    logits = {}
    am = {}
    for b in (1, 2, 3, 5, 8):
        lg = t.empty((64, N), dtype=t.bfloat16, device="cuda")
        ag = t.empty((64,), dtype=t.int32, device="cuda")
        for t0 in range(0, 64, b):
            t1 = min(64, t0 + b)
            iqd.lm_head_argmax(q[t0:t1], sa[t0:t1], w, sw, logits=lg[t0:t1], argmax=ag[t0:t1])
        logits[b] = host_bits(lg)
        am[b] = host(ag)
    for b in (2, 3, 5, 8):
        flips = int((am[b] != am[1]).sum())
        assert flips == 0, f"b={b}: {flips} argmax flips"
        assert_bits_equal(logits[b], logits[1], f"logits b={b} vs b=1")
    rows = sample_rows(N, 64, 5001)
    ol = oracle.w8a8(oq, osa, L.w[rows], L.s_w[rows])
    assert_bits_equal(logits[1][:, rows], ol, "sampled logits vs oracle")
    ol2, oa2 = oracle.lm_head_argmax(oq[:2], osa[:2], L.w, L.s_w)
    assert_bits_equal(logits[1][:2], ol2, "full logits rows 0-1")
    assert_bits_equal(am[1][:2], oa2, "argmax rows 0-1")
    # argmax equals the host argmax of the returned logits on every row
    f = W.bf16_bits_to_f32(logits[1])
    assert np.array_equal(am[1], np.argmax(f, axis=1).astype(np.int32))


@pytest.mark.parametrize("li", range(4))
def test_qwen3_14b_pow2_requant(iqd, li):
    """Requantization bit-exact vs the oracle; both scale sets invariant over
    b in {1, 2, 4, 8, 512} and equal to the oracle on sampled rows; with
    power-of-two scales the epilogue equals the F3 scale order exactly."""
    t = torch()
    L = W.qwen3_14b_layer(li, tokens=512)
    N = L.N
    ow, os_ = oracle.pow2_requant(L.w, L.s_w)
    w, sw = dev(L.w), dev(L.s_w)
    w2, sw2 = iqd.pow2_requantize(w, sw)
    assert_bits_equal(host(w2), ow, f"{L.name} requantized weights")
    assert_bits_equal(host(sw2).view(np.uint32), os_.view(np.uint32), f"{L.name} pow2 scales")
    oq, osa = oracle.quantize_token(L.x)
    q, sa = iqd.quantize_activations(dev(L.x))
    rows = sample_rows(N, 32, 4001 + li)
    for name, (wd, swd, hw, hs) in {"own": (w, sw, L.w, L.s_w), "pow2": (w2, sw2, ow, os_)}.items():
        y1 = t.empty((512, N), dtype=t.bfloat16, device="cuda")
        for i in range(512):
            iqd.w8a8_linear(q[i:i + 1], sa[i:i + 1], wd, swd, y=y1[i:i + 1])
        ref = host_bits(y1)
        assert_bits_equal(ref[:, rows], oracle.w8a8(oq, osa, hw[rows], hs[rows]), f"{L.name} {name} vs oracle")
        for b in (2, 4, 8):
            out = t.empty((64, N), dtype=t.bfloat16, device="cuda")
            for t0 in range(0, 64, b):
                iqd.w8a8_linear(q[t0:t0 + b], sa[t0:t0 + b], wd, swd, y=out[t0:t0 + b])
            assert_bits_equal(host_bits(out), ref[:64], f"{L.name} {name} b={b}")
        y512 = iqd.w8a8_linear(q, sa, wd, swd)
        assert_bits_equal(host_bits(y512), ref, f"{L.name} {name} b=512")
