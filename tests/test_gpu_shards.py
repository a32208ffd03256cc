"""The per-GPU shards of a tensor-parallel layer, run on one GPU.

Output rows are independent, so column parallelism (the weight rows split
over g GPUs) needs no cross-GPU arithmetic: each shard's call gives, bit for
bit, its rows of the whole layer's output, and an all-gather of b x N/g bf16
values per GPU completes it.  For the LM head split over the vocabulary,
each shard yields its logits and its (maximum, lowest local index); the
global argmax is the largest maximum, the lowest shard on a tie, which is
the whole head's answer.  (Row parallelism, K split over GPUs, exchanges
int32 partial sums whose exact sum is order-free: that is the split-K path,
covered in test_gpu_w8a8.py.)

Shapes: the Qwen3-8B qkv, o and gate_up split 8 ways (4096 -> 768, 512 and
3072 per GPU) and the Qwen3-8B LM head split 8 ways (4096 -> 18992).
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import assert_bits_equal, dev, host, host_bits, sample_rows

pytestmark = pytest.mark.gpu

G = 8  # shards


@pytest.fixture(scope="module")
def iqd():
    import invariant_quantized_decode_token_amd as m

    m.load()
    return m


@pytest.mark.parametrize("li", [0, 1, 2])
def test_column_shards_equal_whole_layer(iqd, li):
    L = W.qwen3_8b_layer(li, tokens=8)
    assert L.N % G == 0
    ns = L.N // G
    oq, osa = oracle.quantize_token(L.x)
    q, sa = iqd.quantize_activations(dev(L.x))
    wd, swd = dev(L.w), dev(L.s_w)
    for b in (1, 3, 8):
        whole = host_bits(iqd.w8a8_linear(q[:b], sa[:b], wd, swd))
        parts = [host_bits(iqd.w8a8_linear(q[:b], sa[:b], wd[s * ns:(s + 1) * ns], swd[s * ns:(s + 1) * ns]))
                 for s in range(G)]
        assert_bits_equal(np.concatenate(parts, axis=1), whole, f"{L.name} b={b}: shards vs whole")
        # the fused entry point on a shard equals its rows of the whole layer too
        s = G - 1
        fused = host_bits(iqd.w8a8_linear_bf16(dev(L.x[:b]), wd[s * ns:], swd[s * ns:]))
        assert_bits_equal(fused, whole[:, s * ns:], f"{L.name} b={b}: fused last shard")
    rows = sample_rows(ns, 24, li)
    last = slice((G - 1) * ns, L.N)
    assert_bits_equal(parts[G - 1][:, rows], oracle.w8a8(oq[:8], osa[:8], L.w[last][rows], L.s_w[last][rows]),
                      f"{L.name}: last shard vs oracle")


def _bf16_value(h: np.ndarray) -> np.ndarray:
    return (h.astype(np.uint32) << 16).view(np.float32)


def test_lm_head_vocab_shards(iqd):
    L = W.lm_head_layer(tokens=4)
    N, K = L.N, L.K
    assert N % G == 0
    ns = N // G
    w = L.w.copy()
    s_w = L.s_w.copy()
    oq, osa = oracle.quantize_token(L.x)
    # a tie across shards for token 0: the same row (and scale) in shards 2
    # and 5, aligned with token 0's codes and given the largest scale; the
    # lower global index must win
    r_a, r_b = 2 * ns + 17, 5 * ns + 3
    w[r_a] = (np.sign(oq[0]).astype(np.int32) * 127).astype(np.int8)
    w[r_b] = w[r_a]
    s_w[r_a] = s_w[r_b] = np.float32(np.max(np.abs(s_w)) * 64)
    q, sa = iqd.quantize_activations(dev(L.x))
    wd, swd = dev(w), dev(s_w)
    b = 4
    lg_whole, am_whole = iqd.lm_head_argmax(q[:b], sa[:b], wd, swd)
    lg_whole, am_whole = host_bits(lg_whole), host(am_whole)
    logits, best = [], []
    for s in range(G):
        lg, am = iqd.lm_head_argmax(q[:b], sa[:b], wd[s * ns:(s + 1) * ns], swd[s * ns:(s + 1) * ns])
        lg, am = host_bits(lg), host(am)
        logits.append(lg)
        best.append((_bf16_value(lg[np.arange(b), am]), am + s * ns))
    assert_bits_equal(np.concatenate(logits, axis=1), lg_whole, "LM head shards: logits vs whole")
    # global argmax: the largest shard maximum, the lowest shard on a tie
    glob = np.empty(b, np.int64)
    for t in range(b):
        vals = np.array([best[s][0][t] for s in range(G)])
        s_win = int(np.flatnonzero(vals == vals.max())[0])
        glob[t] = best[s_win][1][t]
    assert glob.tolist() == am_whole.tolist(), (glob, am_whole)
    assert glob[0] == r_a, "the tie across shards goes to the lower global index"
    # the winning shard's argmax against the oracle's
    for t in range(b):
        s_win = int(glob[t]) // ns
        sl = slice(s_win * ns, (s_win + 1) * ns)
        ol, oa = oracle.lm_head_argmax(oq[t:t + 1], osa[t:t + 1], w[sl], s_w[sl])
        assert int(oa[0]) + s_win * ns == int(glob[t])
