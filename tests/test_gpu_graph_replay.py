"""Graph capture: the entry points a serving loop captures (quantize + linear
in one call, the linear with split-K, block-quantized split-K, the LM-head
argmax, decode attention with the chunk merge, FP8 with split-K, kq6
and kq4 superblocks with split-K) recorded in
one HIP graph and replayed three times with eager work in between; every
replay must equal the eager results bit for bit (no workspace state may leak
from one replay into the next)."""
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


def test_graph_replays_equal_eager(iqd):
    t = torch()
    L = W.qwen3_8b_layer(1, tokens=8)  # o: 4096 -> 4096
    x = dev(L.x)
    w, sw = dev(L.w), dev(L.s_w)
    Lb = W.blockq8_layer(0, tokens=8)
    wb, dwb = dev(Lb.w), dev(Lb.d_w, "fp16")
    xb = dev(Lb.x)
    Ll = W.w8a8_layer("head_rows", 4096, 20000, W.SEED_LM_HEAD, 5, outliers=False)
    wl, swl = dev(Ll.w), dev(Ll.s_w)
    xl = dev(Ll.x)
    att = W.attn_case(W.SEED_ATTN + 77, 4, 1000, capacity=1100)
    qa, ka, va = dev(att.q), dev(att.k), dev(att.v)
    Lk = W.kq6_layer(0, tokens=8)
    qlk, qhk, sck, dk = dev(Lk.ql), dev(Lk.qh), dev(Lk.sc), dev(Lk.d, "fp16")
    qk, dak = iqd.quantize_activations(dev(Lk.x), group=32)
    L4 = W.kq4_layer(0, tokens=8)
    ql4, scm4, dm4 = dev(L4.ql), dev(L4.scm), dev(L4.dm, "fp16")
    q4, da4 = iqd.quantize_activations(dev(L4.x), group=32)
    Lf = W.fp8_layer(0, tokens=8)
    wf, swf = dev(Lf.w), dev(Lf.s_w)
    xf = dev(Lf.x)

    # persistent buffers: inputs derived once, outputs written by every run
    q, sa = iqd.quantize_activations(x)
    qb, db = iqd.quantize_activations(xb, group=32)
    ql, sl = iqd.quantize_activations(xl)
    qf, sf = iqd.quantize_fp8(xf)
    outs = {
        "bf16": t.empty((8, L.N), dtype=t.bfloat16, device="cuda"),
        "split": t.empty((5, L.N), dtype=t.bfloat16, device="cuda"),
        "bq8": t.empty((8, Lb.N), dtype=t.bfloat16, device="cuda"),
        "logits": t.empty((5, Ll.N), dtype=t.bfloat16, device="cuda"),
        "argmax": t.empty((5,), dtype=t.int32, device="cuda"),
        "attn": t.empty_like(qa),
        "fp8": t.empty((8, Lf.N), dtype=t.bfloat16, device="cuda"),
        "kq6": t.empty((8, Lk.N), dtype=t.bfloat16, device="cuda"),
        "kq4": t.empty((8, L4.N), dtype=t.bfloat16, device="cuda"),
    }
    ws = {
        "split": t.zeros((iqd.workspace_bytes(iqd.IQD_OP_W8A8, 5, L.N, L.K, 4),), dtype=t.uint8, device="cuda"),
        "bq8": t.zeros((iqd.workspace_bytes(iqd.IQD_OP_BLOCKQ8, 8, Lb.N, Lb.K, 4),), dtype=t.uint8, device="cuda"),
        "head": t.zeros((iqd.workspace_bytes(iqd.IQD_OP_LM_HEAD, 5, Ll.N, Ll.K, 1),), dtype=t.uint8, device="cuda"),
        "attn": t.zeros((iqd.attn_workspace_bytes(4, 32, 8, 128, att.pos0),), dtype=t.uint8, device="cuda"),
        "fp8": t.zeros((iqd.workspace_bytes(iqd.IQD_OP_FP8, 8, Lf.N, Lf.K, 2),), dtype=t.uint8, device="cuda"),
        "kq6": t.zeros((iqd.workspace_bytes(iqd.IQD_OP_KQ6, 8, Lk.N, Lk.K, 4),), dtype=t.uint8, device="cuda"),
        "kq4": t.zeros((iqd.workspace_bytes(iqd.IQD_OP_KQ4, 8, L4.N, L4.K, 2),), dtype=t.uint8, device="cuda"),
        "bf16": t.zeros((iqd.workspace_bytes(iqd.IQD_OP_W8A8_BF16, 8, L.N, L.K, 1) + 16,), dtype=t.uint8,
                        device="cuda"),
    }
    assert ws["attn"].numel() > 0  # 1000 cells: the merge runs

    def run():
        iqd.w8a8_linear_bf16(x, w, sw, y=outs["bf16"], workspace=ws["bf16"])
        iqd.w8a8_linear(q[:5], sa[:5], w, sw, split_k=4, y=outs["split"], workspace=ws["split"])
        iqd.blockq8_linear(qb, db, wb, dwb, split_k=4, y=outs["bq8"], workspace=ws["bq8"])
        iqd.lm_head_argmax(ql, sl, wl, swl, logits=outs["logits"], argmax=outs["argmax"], workspace=ws["head"])
        iqd.attn_decode(qa, ka, va, att.pos0, float(att.scale), out=outs["attn"], workspace=ws["attn"])
        iqd.fp8_linear(qf, sf, wf, swf, split_k=2, y=outs["fp8"], workspace=ws["fp8"])
        iqd.kq6_linear(qk, dak, qlk, qhk, sck, dk, split_k=4, y=outs["kq6"], workspace=ws["kq6"])
        iqd.kq4_linear(q4, da4, ql4, scm4, dm4, split_k=2, y=outs["kq4"], workspace=ws["kq4"])

    def snapshot():
        t.cuda.synchronize()
        return {k: (host(v) if v.dtype == t.int32 else host_bits(v)) for k, v in outs.items()}

    run()
    eager = snapshot()
    s = t.cuda.Stream()
    s.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(s):
        run()
    t.cuda.current_stream().wait_stream(s)
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        run()
    for rep in range(3):
        for v in outs.values():
            v.zero_()  # eager work between replays; stale outputs cannot pass
        g.replay()
        got = snapshot()
        for k in eager:
            assert_bits_equal(got[k], eager[k], f"replay {rep}: {k}")
        run()  # and eager calls in between leave the graph's results unchanged
        again = snapshot()
        for k in eager:
            assert_bits_equal(again[k], eager[k], f"eager after replay {rep}: {k}")
    np.testing.assert_array_equal(eager["argmax"], host(outs["argmax"]))
