#!/usr/bin/env python3
"""Benchmark: W8A8 mat-vec weight GB/s on Qwen3-8B-shaped decode linears at b = 1..8.

One step is a speculative-verify sweep over the four W8A8 decode layers of a
Qwen3-8B-shaped transformer block (qkv 4096->6144, o 4096->4096, gate_up
4096->24576, down 12288->4096) at every width b = 1..8: for each (b, layer)
the bf16 activations are quantized per token and the int8 weights are
streamed once, in one w8a8_linear_bf16 call (one kernel; the same bits as
quantize_activations followed by w8a8_linear, whose step time is reported
as config.separate_calls_ms_per_step).  The 32 (b, layer) passes use
8 distinct copies of the weights (1.5 GB) so that no pass finds its weights
in the 256 MB Infinity Cache.  Inputs are seeded synthetic data resident in
HBM before timing; the step is replayed from a HIP graph.

value = weight bytes streamed per step (int8 weights + fp32 scales) / step
time, in GB/s.  The roofline object times the dominant kernels, the 32 W8A8
mat-vec launches of a step (on the step's quantized activations), alone with
HIP events on the stream they run on.  The cpu_baseline
object times the CPU oracle on the same step.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--detail]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W8A8 matvec weight GB/s (% HBM peak) at b=1..8; batch-variant rows = 0"
HBM_PEAK_GBS = 8000.0
COPIES = 8
B_LIST = list(range(1, 9))
PREFILL_SPLITS = (1, 2, 4)  # K splits timed for the b = 512 pass; the fastest is reported


def committed_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (profiles/<kernel>_traffic.json: FETCH_SIZE and WRITE_SIZE per dispatch,
    scaled by a known-size copy), or None if the kernel sources changed since
    the counters were taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", f"{kernel}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    h = hashlib.sha256()
    for src in rec["sources"]:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    return rec["traffic_bytes_per_launch"] if h.hexdigest() == rec["source_sha256"] else None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    p.add_argument("--detail", action="store_true", help="per-(layer, b) kernel timings")
    p.add_argument("--no-prefill", action="store_true", help="skip timing the b=512 prefill pass")
    p.add_argument("--extra", action="store_true", help="also time the block-q8, LM-head, FP8 and attention paths")
    p.add_argument("--calib", action="store_true",
                   help="end with one 256 MiB device-to-device copy (a known-size kernel for HBM counter scaling)")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import invariant_quantized_decode_token_amd as iqd
    import workloads as W

    iqd.load()  # fails loudly when the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---- inputs, resident in HBM ------------------------------------------
    layers = [W.qwen3_8b_layer(i, tokens=8) for i in range(4)]
    wsets, swsets = [], []
    for L in layers:
        w0 = torch.from_numpy(L.w).to(dev)
        wsets.append([w0] + [w0.clone() for _ in range(COPIES - 1)])
        swsets.append(torch.from_numpy(L.s_w).to(dev))
    xs = [torch.from_numpy(L.x.view(np.int16)).view(torch.bfloat16).to(dev) for L in layers]
    qs = [torch.empty((8, L.K), dtype=torch.int8, device=dev) for L in layers]
    sas = [torch.empty((8,), dtype=torch.float32, device=dev) for L in layers]
    ys = [torch.empty((8, L.N), dtype=torch.bfloat16, device=dev) for L in layers]

    def layer_bytes(L):
        return L.N * L.K + 4 * L.N

    def linear_bytes(L, b):  # what one w8a8_linear call must move: weights, scales, q, s_a in, bf16 y out
        return L.N * L.K + 4 * L.N + b * L.K + 4 * b + 2 * b * L.N

    step_weight_bytes = sum(layer_bytes(L) for L in layers) * len(B_LIST)

    def step():
        """The decode step: per (b, layer) one w8a8_linear_bf16 call, which
        quantizes the bf16 activations and runs the linear in one kernel."""
        for bi, b in enumerate(B_LIST):
            c = bi % COPIES
            for li, L in enumerate(layers):
                iqd.w8a8_linear_bf16(xs[li][:b], wsets[li][c], swsets[li], y=ys[li][:b])

    def step_separate():
        """The same step as two calls per (b, layer): quantize_activations,
        then w8a8_linear (reported for comparison)."""
        for bi, b in enumerate(B_LIST):
            c = bi % COPIES
            for li, L in enumerate(layers):
                iqd.quantize_activations(xs[li][:b], q=qs[li][:b], scale=sas[li][:b])
                iqd.w8a8_linear(qs[li][:b], sas[li][:b], wsets[li][c], swsets[li], y=ys[li][:b])

    def capture(fn):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    def time_graph(g, reps):
        st = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(st)
        for _ in range(reps):
            g.replay()
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps  # ms per replay

    # ---- the step ------------------------------------------------------------
    g_step = capture(step)
    for _ in range(args.warmup):
        g_step.replay()
    torch.cuda.synchronize()
    ms = time_graph(g_step, args.steps)
    value = step_weight_bytes / (ms * 1e-3) / 1e9

    # ---- the same work as separate quantize + linear calls -------------------------
    g_sep = capture(step_separate)
    for _ in range(3):
        g_sep.replay()
    ms_sep = time_graph(g_sep, args.steps)

    # ---- dominant kernel alone: the 32 W8A8 mat-vec launches of a step ------------
    # (w8a8_linear on the step's quantized activations: k_w8a8_matvec at b = 1
    # and on small matrices at b = 2, k_w8a8_mfvec otherwise)
    for li, L in enumerate(layers):
        iqd.quantize_activations(xs[li], q=qs[li], scale=sas[li])

    def step_linear():
        for bi, b in enumerate(B_LIST):
            c = bi % COPIES
            for li, L in enumerate(layers):
                iqd.w8a8_linear(qs[li][:b], sas[li][:b], wsets[li][c], swsets[li], y=ys[li][:b])
    g_mv = capture(step_linear)
    for _ in range(3):
        g_mv.replay()
    ms_mv = time_graph(g_mv, args.steps)
    n_launch = len(B_LIST) * len(layers)
    mv_bytes = sum(linear_bytes(L, b) for b in B_LIST for L in layers)
    avg_us = ms_mv * 1e3 / n_launch
    achieved = mv_bytes / n_launch / (avg_us * 1e-6) / 1e9
    traffic = committed_traffic("w8a8_decode_matvec")

    # ---- practical ceiling: a device-to-device copy of 1 GiB (read + write bytes) --------
    # (not in a --calib run, whose one known-size copy scales the HBM counters)
    copy_gbs = None
    if not args.calib:
        csrc = torch.empty(2 ** 29, dtype=torch.int16, device=dev)
        cdst = torch.empty_like(csrc)
        g_cp = capture(lambda: cdst.copy_(csrc))
        g_cp.replay()
        copy_gbs = round(2 * csrc.numel() * 2 / (time_graph(g_cp, 10) * 1e-3) / 1e9, 1)
        del csrc, cdst, g_cp

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded int8 weights, log-uniform fp32 scales, N(0,1) bf16 activations with 1% x20 "
                "outlier channels)",
        "config": {
            "workload": "Qwen3-8B-shaped W8A8 decode linears qkv 4096->6144, o 4096->4096, gate_up "
                        "4096->24576, down 12288->4096; per-token quantization + linear (one "
                        "w8a8_linear_bf16 call) at every b=1..8",
            "b": B_LIST,
            "weight_copies": COPIES,
            "weight_bytes_per_step": step_weight_bytes,
            "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
            "tokens_per_s_equiv": round(sum(B_LIST) / (ms * 1e-3), 1),
            "separate_calls_ms_per_step": round(ms_sep, 5),
        },
        "roofline": {
            "kernel": "W8A8 decode mat-vec, the 32 launches of a step alone (k_w8a8_matvec dot4 at b=1 and on "
                      "small matrices at b=2, k_w8a8_mfvec matrix cores otherwise)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "avg_launch_us": round(avg_us, 3),
            "copy_GBs": copy_gbs,  # a 1 GiB device-to-device copy, read + write bytes: a practical ceiling
            "launches_per_step": n_launch,
        },
        "cpu_baseline": None,
    }

    if args.detail:
        det = []
        for li, L in enumerate(layers):
            for b in B_LIST:
                def one(li=li, L=L, b=b):
                    for c in range(COPIES):
                        iqd.w8a8_linear_bf16(xs[li][:b], wsets[li][c], swsets[li], y=ys[li][:b])

                def lin(li=li, L=L, b=b):
                    for c in range(COPIES):
                        iqd.w8a8_linear(qs[li][:b], sas[li][:b], wsets[li][c], swsets[li], y=ys[li][:b])
                g = capture(one)
                g.replay()
                us = time_graph(g, 20) * 1e3 / COPIES
                g2 = capture(lin)
                g2.replay()
                us2 = time_graph(g2, 20) * 1e3 / COPIES
                det.append({"layer": L.name, "b": b, "us": round(us, 3),
                            "weight_GBs": round(layer_bytes(L) / (us * 1e-6) / 1e9, 1),
                            "linear_only_us": round(us2, 3)})
        out["detail"] = det

    if not args.no_prefill:
        pre = []
        for li, L in enumerate(layers):
            T = 512
            Lp = W.qwen3_8b_layer(li, tokens=T)
            xp = torch.from_numpy(Lp.x.view(np.int16)).view(torch.bfloat16).to(dev)
            qp, sp = iqd.quantize_activations(xp)
            yp = torch.empty((T, L.N), dtype=torch.bfloat16, device=dev)
            wsp = torch.empty((iqd.workspace_bytes(iqd.IQD_OP_W8A8, T, L.N, L.K, max(PREFILL_SPLITS)),),
                              dtype=torch.uint8, device=dev)
            per_split = {}
            for split in PREFILL_SPLITS:
                def pf(li=li, split=split):
                    for c in range(COPIES):
                        iqd.w8a8_linear(qp, sp, wsets[li][c], swsets[li], split_k=split, y=yp, workspace=wsp)
                g = capture(pf)
                g.replay()
                per_split[split] = time_graph(g, 5) * 1e3 / COPIES
            best = min(per_split, key=per_split.get)
            us = per_split[best]
            tops = 2.0 * T * L.N * L.K / (us * 1e-6) / 1e12
            pre.append({"layer": L.name, "b": T, "split_k": best, "us": round(us, 2), "TOPS": round(tops, 1),
                        "mfma_frac": round(tops / 5000.0, 4),
                        "us_by_split": {str(k): round(v, 2) for k, v in per_split.items()}})
            del wsp
        out["prefill"] = pre

    if args.extra:
        ext = []
        def copies_past_cache(nbytes):  # weight copies in rotation: more than 512 MB, past the 256 MB cache
            return max(2, -(-512 * 2 ** 20 // int(nbytes)))

        for i in range(2):
            Lb = W.blockq8_layer(i, tokens=16)
            by = Lb.N * Lb.K * (1 + 2 / 32)
            nc = copies_past_cache(by)
            wq = torch.from_numpy(Lb.w).to(dev)
            wqs = [wq] + [wq.clone() for _ in range(nc - 1)]
            dw = torch.from_numpy(Lb.d_w.view(np.int16)).view(torch.float16).to(dev)
            xb = torch.from_numpy(Lb.x.view(np.int16)).view(torch.bfloat16).to(dev)
            qb, db = iqd.quantize_activations(xb, group=32)
            for b in (1, 4, 8, 16):
                yb = torch.empty((b, Lb.N), dtype=torch.bfloat16, device=dev)

                def bq(b=b, yb=yb):
                    for c in range(nc):
                        iqd.blockq8_linear(qb[:b], db[:b], wqs[c], dw, y=yb)
                g = capture(bq)
                g.replay()
                us = time_graph(g, 10) * 1e3 / nc
                ext.append({"op": "blockq8_linear", "K": Lb.K, "N": Lb.N, "b": b, "us": round(us, 2),
                            "weight_GBs": round(by / (us * 1e-6) / 1e9, 1)})
            del wqs, wq
        # kq6 superblocks (6.5625 bits per weight) on the Qwen3-8B o and down shapes
        for i in range(len(W.KQ6_SHAPES)):
            Lk = W.kq6_layer(i, tokens=16)
            by = Lk.N * Lk.K * (0.5 + 0.25 + 1 / 16) + Lk.N * (Lk.K // 256) * 2
            nc = copies_past_cache(by)
            planes = [(torch.from_numpy(Lk.ql).to(dev), torch.from_numpy(Lk.qh).to(dev), torch.from_numpy(Lk.sc).to(dev))]
            planes += [tuple(p.clone() for p in planes[0]) for _ in range(nc - 1)]
            dk = torch.from_numpy(Lk.d.view(np.int16)).view(torch.float16).to(dev)
            xk = torch.from_numpy(Lk.x.view(np.int16)).view(torch.bfloat16).to(dev)
            qk, dak = iqd.quantize_activations(xk, group=32)
            for b in (1, 4, 8):
                yk = torch.empty((b, Lk.N), dtype=torch.bfloat16, device=dev)

                def kq(b=b, yk=yk):
                    for c in range(nc):
                        iqd.kq6_linear(qk[:b], dak[:b], *planes[c], dk, y=yk)
                g = capture(kq)
                g.replay()
                us = time_graph(g, 10) * 1e3 / nc
                ext.append({"op": "kq6_linear", "K": Lk.K, "N": Lk.N, "b": b, "us": round(us, 2),
                            "weight_GBs": round(by / (us * 1e-6) / 1e9, 1)})
            del planes
        # kq4 superblocks (4.625 bits per weight) on the same shapes
        for i in range(len(W.KQ6_SHAPES)):
            L4 = W.kq4_layer(i, tokens=16)
            by = L4.N * L4.K * (0.5 + 1 / 16) + L4.N * (L4.K // 256) * 4
            nc = copies_past_cache(by)
            planes = [(torch.from_numpy(L4.ql).to(dev), torch.from_numpy(L4.scm).to(dev))]
            planes += [tuple(p.clone() for p in planes[0]) for _ in range(nc - 1)]
            dm4 = torch.from_numpy(L4.dm.view(np.int16)).view(torch.float16).to(dev)
            x4 = torch.from_numpy(L4.x.view(np.int16)).view(torch.bfloat16).to(dev)
            q4, da4 = iqd.quantize_activations(x4, group=32)
            for b in (1, 4, 8):
                y4 = torch.empty((b, L4.N), dtype=torch.bfloat16, device=dev)

                def k4(b=b, y4=y4):
                    for c in range(nc):
                        iqd.kq4_linear(q4[:b], da4[:b], planes[c][0], planes[c][1], dm4, y=y4)
                g = capture(k4)
                g.replay()
                us = time_graph(g, 10) * 1e3 / nc
                ext.append({"op": "kq4_linear", "K": L4.K, "N": L4.N, "b": b, "us": round(us, 2),
                            "weight_GBs": round(by / (us * 1e-6) / 1e9, 1)})
            del planes
        Ll = W.lm_head_layer(tokens=8)
        wl = torch.from_numpy(Ll.w).to(dev)
        swl = torch.from_numpy(Ll.s_w).to(dev)
        xl = torch.from_numpy(Ll.x.view(np.int16)).view(torch.bfloat16).to(dev)
        ql, sl = iqd.quantize_activations(xl)
        for b in (1, 2, 3, 5, 8):
            am = torch.empty((b,), dtype=torch.int32, device=dev)
            lg = torch.empty((b, Ll.N), dtype=torch.bfloat16, device=dev)

            def lh(b=b, am=am, lg=lg):
                for _ in range(4):  # 622 MB of weights: far past the 256 MB Infinity Cache
                    iqd.lm_head_argmax(ql[:b], sl[:b], wl, swl, logits=lg, argmax=am)
            g = capture(lh)
            g.replay()
            us = time_graph(g, 10) * 1e3 / 4
            by = Ll.N * Ll.K + 4 * Ll.N
            ext.append({"op": "lm_head_argmax", "K": Ll.K, "N": Ll.N, "b": b, "us": round(us, 2),
                        "weight_GBs": round(by / (us * 1e-6) / 1e9, 1)})
        # FP8 (E4M3) W8A8 on the Qwen3-8B layers (weights 1 byte each, as int8)
        for li in range(4):
            Lf = W.fp8_layer(li, tokens=8)
            wf0 = torch.from_numpy(Lf.w).to(dev)
            wfs = [wf0] + [wf0.clone() for _ in range(COPIES - 1)]
            swf = torch.from_numpy(Lf.s_w).to(dev)
            qf, sf = iqd.quantize_fp8(torch.from_numpy(Lf.x.view(np.int16)).view(torch.bfloat16).to(dev))
            for b in (1, 4, 8):
                yf = torch.empty((b, Lf.N), dtype=torch.bfloat16, device=dev)

                def f8(b=b, yf=yf):
                    for c in range(COPIES):
                        iqd.fp8_linear(qf[:b], sf[:b], wfs[c], swf, y=yf)
                g = capture(f8)
                g.replay()
                us = time_graph(g, 10) * 1e3 / COPIES
                by = Lf.N * Lf.K + 4 * Lf.N
                ext.append({"op": "fp8_linear", "layer": Lf.name, "K": Lf.K, "N": Lf.N, "b": b, "us": round(us, 2),
                            "weight_GBs": round(by / (us * 1e-6) / 1e9, 1)})
            del wfs, wf0
        # the W8A8 decode mat-vec on Qwen3-14B-shaped layers (shapes the launch tables were not tuned on)
        for li in range(4):
            L14 = W.qwen3_14b_layer(li, tokens=8)
            by = L14.N * L14.K + 4 * L14.N
            nc = copies_past_cache(by)
            w0 = torch.from_numpy(L14.w).to(dev)
            w14 = [w0] + [w0.clone() for _ in range(nc - 1)]
            s14 = torch.from_numpy(L14.s_w).to(dev)
            x14 = torch.from_numpy(L14.x.view(np.int16)).view(torch.bfloat16).to(dev)
            q14, sa14 = iqd.quantize_activations(x14)
            for b in (1, 4, 8):
                y14 = torch.empty((b, L14.N), dtype=torch.bfloat16, device=dev)

                def m14(b=b, y14=y14):
                    for c in range(nc):
                        iqd.w8a8_linear(q14[:b], sa14[:b], w14[c], s14, y=y14)
                g = capture(m14)
                g.replay()
                us = time_graph(g, 10) * 1e3 / nc
                ext.append({"op": "w8a8_linear", "model": "Qwen3-14B", "layer": L14.name, "K": L14.K, "N": L14.N,
                            "b": b, "us": round(us, 2), "weight_GBs": round(by / (us * 1e-6) / 1e9, 1)})
            del w14, w0
        # decode attention, Qwen3-8B heads (32 query, 8 kv, D = 128): enough cache
        # copies in rotation to exceed the 256 MB Infinity Cache
        name, Hq, Hkv, D = W.QWEN3_8B_ATTN
        for cells in (4096, 32768):
            kv_bytes = cells * Hkv * D * 2 * 2
            ncopy = max(2, min(32, -(-512 * 2 ** 20 // kv_bytes)))
            case = W.attn_case(W.SEED_ATTN + cells, 8, cells)
            ks = [torch.from_numpy(case.k.view(np.int16)).view(torch.bfloat16).to(dev) for _ in range(ncopy)]
            vs = [torch.from_numpy(case.v.view(np.int16)).view(torch.bfloat16).to(dev) for _ in range(ncopy)]
            qa = torch.from_numpy(case.q.view(np.int16)).view(torch.bfloat16).to(dev)
            for b in (1, 2, 4, 8):
                oa = torch.empty((b, Hq, D), dtype=torch.bfloat16, device=dev)
                wsa = torch.empty((max(16, iqd.attn_workspace_bytes(b, Hq, Hkv, D, cells - b)),), dtype=torch.uint8,
                                  device=dev)

                def at(b=b, oa=oa, wsa=wsa):
                    for c in range(ncopy):
                        iqd.attn_decode(qa[:b], ks[c], vs[c], cells - b, float(case.scale), out=oa, workspace=wsa)
                g = capture(at)
                g.replay()
                us = time_graph(g, 10) * 1e3 / ncopy
                ext.append({"op": "attn_decode", "cells": cells, "Hq": Hq, "Hkv": Hkv, "D": D, "b": b,
                            "us": round(us, 2), "kv_GBs": round(kv_bytes / (us * 1e-6) / 1e9, 1)})
            del ks, vs
        out["extra"] = ext

    if not args.no_cpu:
        import oracle

        ncores = os.cpu_count() or 1
        nthreads = min(ncores, 16)
        hosts = [(oracle.quantize_token, L) for L in layers]
        t0 = time.time()
        passes = 0
        while passes < 1 or time.time() - t0 < 10.0:
            for b in B_LIST:
                for L in layers:
                    q, s = oracle.quantize_token(L.x[:b])
                    oracle.w8a8(q, s, L.w, L.s_w, nthreads=nthreads)
            passes += 1
        dt = time.time() - t0
        out["cpu_baseline"] = {
            "value": round(step_weight_bytes * passes / dt / 1e9, 3),
            "unit": "GB/s",
            "cores": nthreads,
            "kind": "oracle",
            "sample": f"{passes} full step(s): quantize + W8A8 linear for the 4 layers at b=1..8, "
                      f"{dt:.1f} s wall",
        }

    if args.calib:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        src.fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
