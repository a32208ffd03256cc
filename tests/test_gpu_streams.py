"""Concurrent calls on two streams: the library keeps no state between calls,
so the same entry points (split-K linears with their own workspaces, the
LM-head argmax, decode attention with its merge) enqueued on two streams at
once, with different inputs, give each stream the bits it gets alone."""
import numpy as np
import pytest

import workloads as W
from gpu_util import assert_bits_equal, dev, host, host_bits, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def iqd():
    import invariant_quantized_decode_token_amd as m

    m.load()
    return m


def make_job(iqd, seed):
    t = torch()
    g = W.rng(seed)
    N, K = 3000, 4096
    w = dev(W.int8_weights(g, N, K))
    sw = dev(W.log_uniform_scales(g, N))
    x = dev(W.normal_bf16(g, 8, K))
    q, sa = iqd.quantize_activations(x)
    qb, db = iqd.quantize_activations(x, group=32)
    wq, dw = W.q8_0_weights(g, N, K)
    wq, dw = dev(wq), dev(dw, "fp16")
    att = W.attn_case(seed, 4, 2000, Hq=8, Hkv=2)
    qa, ka, va = dev(att.q), dev(att.k), dev(att.v)
    outs = {"w8a8": t.empty((8, N), dtype=t.bfloat16, device="cuda"),
            "bq8": t.empty((8, N), dtype=t.bfloat16, device="cuda"),
            "logits": t.empty((8, N), dtype=t.bfloat16, device="cuda"),
            "argmax": t.empty((8,), dtype=t.int32, device="cuda"),
            "attn": t.empty_like(qa)}
    ws = {"w8a8": t.empty((iqd.workspace_bytes(iqd.IQD_OP_W8A8, 8, N, K, 8),), dtype=t.uint8, device="cuda"),
          "bq8": t.empty((iqd.workspace_bytes(iqd.IQD_OP_BLOCKQ8, 8, N, K, 4),), dtype=t.uint8, device="cuda"),
          "head": t.empty((iqd.workspace_bytes(iqd.IQD_OP_LM_HEAD, 8, N, K, 1),), dtype=t.uint8, device="cuda"),
          "attn": t.empty((max(16, iqd.attn_workspace_bytes(4, 8, 2, 128, att.pos0)),), dtype=t.uint8,
                          device="cuda")}

    def run():
        for _ in range(3):
            iqd.w8a8_linear(q, sa, w, sw, split_k=8, y=outs["w8a8"], workspace=ws["w8a8"])
            iqd.blockq8_linear(qb, db, wq, dw, split_k=4, y=outs["bq8"], workspace=ws["bq8"])
            iqd.lm_head_argmax(q, sa, w, sw, logits=outs["logits"], argmax=outs["argmax"], workspace=ws["head"])
            iqd.attn_decode(qa, ka, va, att.pos0, float(att.scale), out=outs["attn"], workspace=ws["attn"])

    def snap():
        return {k: (host(v) if v.dtype == t.int32 else host_bits(v)) for k, v in outs.items()}
    return run, snap


def test_two_streams_at_once_equal_each_alone(iqd):
    t = torch()
    jobs = [make_job(iqd, 101), make_job(iqd, 202)]
    alone = []
    for run, snap in jobs:
        run()
        t.cuda.synchronize()
        alone.append(snap())
    assert not np.array_equal(alone[0]["w8a8"], alone[1]["w8a8"])  # different inputs
    streams = [t.cuda.Stream(), t.cuda.Stream()]
    for rep in range(3):
        for s in streams:
            s.wait_stream(t.cuda.current_stream())
        for (run, _), s in zip(jobs, streams):
            with t.cuda.stream(s):
                run()
        t.cuda.synchronize()
        for i, (_, snap) in enumerate(jobs):
            got = snap()
            for k in got:
                assert_bits_equal(got[k], alone[i][k], f"rep {rep} stream {i} {k}")
