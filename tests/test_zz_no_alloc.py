"""The LM head entry point that allocates nothing (lm_head_argmax_static):
through the C ABI, equal to lm_head_argmax bit for bit on two calls in a row
(the second smaller, so stale scratch from the first would show), with and
without logits; a request larger than the static scratch is refused with
nothing written."""
import numpy as np
import pytest

import invariant_quantized_decode_token_amd as iqd
from invariant_quantized_decode_token_amd import _lib as L
import workloads as W
from gpu_util import assert_bits_equal, dev, host, host_bits, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    return iqd.load()


def operands(seed, b, N, K):
    g = W.rng(seed)
    w = W.int8_weights(g, N, K)
    s_w = W.log_uniform_scales(g, N)
    q = W.int8_weights(g, b, K)
    s_a = W.log_uniform_scales(g, b, 1e-4, 1e-2)
    return dev(q), dev(s_a), dev(w), dev(s_w)


def test_static_scratch_equals_workspace_path(lib):
    t = torch()
    # first the LM head shape (4096 -> 151936, b = 8: 2.4 MB of logits in the
    # scratch), then a smaller one (the scratch still holds the first call's data)
    for seed, b, N, K in ((5101, 8, 151936, 4096), (5102, 3, 5003, 512)):
        q, s_a, w, s_w = operands(seed, b, N, K)
        ref_lg, ref_am = iqd.lm_head_argmax(q, s_a, w, s_w)
        _, am = iqd.lm_head_argmax_static(q, s_a, w, s_w, logits=False)  # logits in the scratch
        t.cuda.synchronize()
        assert_bits_equal(host(am), host(ref_am), f"argmax, logits in the scratch, b={b} N={N}")
        lg2, am2 = iqd.lm_head_argmax_static(q, s_a, w, s_w)  # caller's logits, keys in the scratch
        t.cuda.synchronize()
        assert_bits_equal(host_bits(lg2), host_bits(ref_lg), f"logits b={b} N={N}")
        assert_bits_equal(host(am2), host(ref_am), f"argmax b={b} N={N}")


def test_static_scratch_rejects_sizes_beyond_it(lib):
    t = torch()
    b, N, K = 16, 300000, 64  # 9.6 MB of logits > IQD_STATIC_SCRATCH_BYTES
    assert 2 * b * N > L.IQD_STATIC_SCRATCH_BYTES
    q, s_a, w, s_w = operands(5103, b, N, K)
    am = t.full((b,), -7, dtype=t.int32, device="cuda")
    with pytest.raises(iqd.IqdError) as e:
        iqd.lm_head_argmax_static(q, s_a, w, s_w, logits=False, argmax=am)
    assert e.value.status == L.IQD_ERR_WORKSPACE
    t.cuda.synchronize()
    assert np.all(host(am) == -7)
    # with the caller's logits the scratch holds only the argmax keys: accepted
    lg, am2 = iqd.lm_head_argmax_static(q, s_a, w, s_w)
    ref_lg, ref_am = iqd.lm_head_argmax(q, s_a, w, s_w)
    t.cuda.synchronize()
    assert_bits_equal(host(am2), host(ref_am), "argmax, large N with caller logits")
