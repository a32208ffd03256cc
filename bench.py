#!/usr/bin/env python3
"""Benchmark: W8A8 mat-vec weight GB/s on Qwen3-8B-shaped decode linears at b = 1..8.

One step is a speculative-verify sweep over the four W8A8 decode layers of a
Qwen3-8B-shaped transformer block (qkv 4096->6144, o 4096->4096, gate_up
4096->24576, down 12288->4096) at every width b = 1..8: for each (b, layer)
the bf16 activations are quantized per token and the int8 weights are
streamed once, in one w8a8_linear_bf16 call (the same bits as
quantize_activations followed by w8a8_linear, whose step time is reported as
config.separate_calls_ms_per_step).  The 32 (b, layer) passes use 8 distinct
copies of the weights (1.5 GB) so that no pass finds its weights in the
256 MB Infinity Cache.  Inputs are seeded synthetic data resident in HBM
before timing; the step is replayed from a HIP graph.

Before anything is timed, the timed inputs are gated: every output row of
every (layer, b) call of the step, and of a b = 512 prefill pass, is compared
bit for bit with the same token computed alone (b = 1): `batch_variant_rows`
counts the rows that differ.  The CPU-oracle leg (`cpu_baseline`, which times
the oracle on the same step) also compares every output of the step with the
oracle's: `mismatches` counts the differing bf16 outputs.  Both must be 0;
the run exits with status 1 otherwise (after printing its line).

value = weight bytes streamed per step (int8 weights + fp32 scales) / step
time (the median of 10 timed groups of steps, each group one replay of a
graph that holds its steps back to back), in GB/s.  The roofline object
times the dominant kernels, the 32 W8A8 mat-vec launches of a step (on the
step's quantized activations), alone with HIP events on the stream they run
on, next to a plain streaming read of the same weight bytes per launch (the
practical ceiling of launches of those sizes).  `configs` times the other
configurations: the tiny layer, the block-q8 layers, the Qwen3-14B layers
with their own and power-of-two scales (plus the pow2-vs-own deviation and
the F3-order agreement), the LM head, and a synthetic Qwen3-8B decode step
(36 blocks x 4 linears + LM head) in tokens/s.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-prefill]
                       [--no-configs] [--detail] [--extra] [--calib]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W8A8 matvec weight GB/s (% HBM peak) at b=1..8; batch-variant rows = 0"
HBM_PEAK_GBS = 8000.0
MFMA_I8_PEAK_TOPS = 5000.0
COPIES = 8
B_LIST = list(range(1, 9))
PREFILL_T = 512
PREFILL_SPLITS = (1, 2, 4)  # K splits timed for the b = 512 pass; the fastest is reported
REPEATS = 10                # timed groups of steps; value uses their median
QWEN3_8B_BLOCKS = 36


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


def log(msg: str):
    """One progress line per finished phase, on stderr (the JSON line is stdout's only line)."""
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


class LoggedRows(list):
    """Result rows that print a progress line as each one is added, so a long
    run (under a profiler's counters, every dispatch serialised) shows it is
    alive between phases."""

    KEYS = ("config", "op", "layer", "K", "N", "b", "cells", "Hq")

    def append(self, row):
        super().append(row)
        log("timed " + ", ".join(f"{k}={row[k]}" for k in self.KEYS if k in row))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline (and the oracle gate)")
    p.add_argument("--detail", action="store_true", help="per-(layer, b) kernel timings")
    p.add_argument("--no-prefill", action="store_true", help="skip timing the b=512 prefill pass")
    p.add_argument("--no-configs", action="store_true", help="skip the other configurations")
    p.add_argument("--extra", action="store_true", help="also time the FP8, k-quant and attention paths")
    p.add_argument("--no-shards", action="store_true",
                   help="with --extra, leave out the 8-way shard lines")
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

    def to_dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def bits(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    def capture(fn, rep=1):
        """A HIP graph of `rep` back-to-back runs of fn.  Each graph replay
        costs about 4-5 us of fixed GPU time on MI355X (measured: a plain read
        of 16.8 MB per launch took 4.34 us per launch in replays of 8 launches,
        3.84 us in replays of 128), which a decode loop pays once per captured
        step of hundreds of launches; timed graphs therefore hold many launches."""
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(rep):
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

    def time_fn(fn, reps=10):
        """ms per run of fn: fn is captured `rep` times into one graph, with
        rep chosen so that a replay lasts at least about 1 ms of GPU time
        (at most 64 runs), and the result is the median of 10 timed repeats of
        `reps` replays each, divided by rep; time_fn.last keeps (median, minimum)."""
        g = capture(fn)
        g.replay()
        one = time_graph(g, 3)
        rep = max(1, min(64, int(1.0 / max(one, 1e-3))))
        if rep > 1:
            del g
            g = capture(fn, rep)
            g.replay()
        ts = sorted(time_graph(g, reps) / rep for _ in range(10))
        med = 0.5 * (ts[4] + ts[5])
        time_fn.last = (med, ts[0])
        return med

    def copies_past_cache(nbytes):  # weight copies in rotation: at least 1 GiB, well past the 256 MB cache
        return max(2, -(-(1 << 30) // int(nbytes)))

    # ---- inputs, resident in HBM ------------------------------------------
    layers = [W.qwen3_8b_layer(i, tokens=PREFILL_T) for i in range(4)]  # x[:8] are the step's tokens
    wsets, swsets = [], []
    for L in layers:
        w0 = torch.from_numpy(L.w).to(dev)
        wsets.append([w0] + [w0.clone() for _ in range(COPIES - 1)])
        swsets.append(torch.from_numpy(L.s_w).to(dev))
    xs_all = [to_dev_bf16(L.x) for L in layers]
    xs = [x[:8] for x in xs_all]
    qs = [torch.empty((8, L.K), dtype=torch.int8, device=dev) for L in layers]
    sas = [torch.empty((8,), dtype=torch.float32, device=dev) for L in layers]
    ys = {(li, b): torch.empty((b, L.N), dtype=torch.bfloat16, device=dev)
          for li, L in enumerate(layers) for b in B_LIST}

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
                iqd.w8a8_linear_bf16(xs[li][:b], wsets[li][c], swsets[li], y=ys[(li, b)])

    def step_separate():
        """The same step as two calls per (b, layer): quantize_activations,
        then w8a8_linear (reported for comparison)."""
        for bi, b in enumerate(B_LIST):
            c = bi % COPIES
            for li, L in enumerate(layers):
                iqd.quantize_activations(xs[li][:b], q=qs[li][:b], scale=sas[li][:b])
                iqd.w8a8_linear(qs[li][:b], sas[li][:b], wsets[li][c], swsets[li], y=ys[(li, b)])

    # ---- gate: every row of the timed calls against the same token alone --------
    # (b = 1 rows for the 8 step tokens and the 512 prefill tokens; then the
    # step's own calls and a b = 512 pass, row by row)
    batch_variant_rows = 0
    rows_checked = 0
    b1_rows = []
    for li, L in enumerate(layers):
        y1 = torch.empty((PREFILL_T, L.N), dtype=torch.bfloat16, device=dev)
        for t in range(PREFILL_T):
            iqd.w8a8_linear_bf16(xs_all[li][t:t + 1], wsets[li][0], swsets[li], y=y1[t:t + 1])
        b1_rows.append(bits(y1))
    step()
    torch.cuda.synchronize()
    step_out = {k: bits(v) for k, v in ys.items()}
    for (li, b), out in step_out.items():
        batch_variant_rows += int(np.any(out != b1_rows[li][:b], axis=1).sum())
        rows_checked += b
    for li, L in enumerate(layers):
        qp, sp = iqd.quantize_activations(xs_all[li])
        y512 = bits(iqd.w8a8_linear(qp, sp, wsets[li][0], swsets[li]))
        batch_variant_rows += int(np.any(y512 != b1_rows[li], axis=1).sum())
        rows_checked += PREFILL_T
        del qp, sp
    log(f"gate: {batch_variant_rows} batch-variant rows of {rows_checked}")
    gate = {"batch_variant_rows": batch_variant_rows, "rows_checked": rows_checked,
            "what": "every output row of the 32 timed (layer, b) calls and of a b=512 prefill pass per layer, "
                    "bitwise against the same token computed alone (b=1)"}

    # ---- the step: REPEATS timed groups, median and minimum ---------------------
    # Each group of n steps is one replay of a graph holding n back-to-back
    # steps (32 launches each), timed between HIP events: exactly K = args.steps
    # steps are timed in all.
    groups = max(1, min(REPEATS, args.steps))
    per = [args.steps // groups + (1 if i < args.steps % groups else 0) for i in range(groups)]

    def time_groups(fn):
        """ms per step of each timed group: one replay of a graph of n steps per group."""
        graphs = {n: capture(fn, n) for n in sorted(set(per))}
        for g in graphs.values():
            g.replay()
        torch.cuda.synchronize()
        res = [time_graph(graphs[n], 1) / n for n in per]
        graphs.clear()
        return res

    g_warm = capture(step)
    for _ in range(args.warmup):
        g_warm.replay()
    torch.cuda.synchronize()
    del g_warm
    group_ms = time_groups(step)
    ms = statistics.median(group_ms)
    ms_min = min(group_ms)
    value = step_weight_bytes / (ms * 1e-3) / 1e9
    log(f"step: {ms:.4f} ms (median of {groups}), {value:.0f} GB/s")

    # ---- the same work as separate quantize + linear calls -------------------------
    ms_sep = statistics.median(time_groups(step_separate))

    # ---- dominant kernel alone: the 32 W8A8 mat-vec launches of a step ------------
    # (w8a8_linear on the step's quantized activations: k_w8a8_matvec at b = 1
    # and on small matrices at b = 2, k_w8a8_mfvec otherwise)
    for li, L in enumerate(layers):
        iqd.quantize_activations(xs[li], q=qs[li], scale=sas[li])

    def step_linear():
        for bi, b in enumerate(B_LIST):
            c = bi % COPIES
            for li, L in enumerate(layers):
                iqd.w8a8_linear(qs[li][:b], sas[li][:b], wsets[li][c], swsets[li], y=ys[(li, b)])
    mv_ms = time_groups(step_linear)
    ms_mv = statistics.median(mv_ms)
    n_launch = len(B_LIST) * len(layers)
    mv_bytes = sum(linear_bytes(L, b) for b in B_LIST for L in layers)
    avg_us = ms_mv * 1e3 / n_launch
    achieved = mv_bytes / n_launch / (avg_us * 1e-6) / 1e9
    traffic = committed_traffic("w8a8_decode_matvec")
    log(f"mat-vec launches alone: {avg_us:.3f} us per launch, {achieved:.0f} GB/s")

    # ---- practical ceiling of these launch sizes: a plain streaming read of each
    # layer's weight bytes, launched as the step launches its mat-vecs ------------
    sink = torch.zeros(1, dtype=torch.int32, device=dev)

    def step_read():
        for bi, b in enumerate(B_LIST):
            c = bi % COPIES
            for li in range(len(layers)):
                iqd.read_ceiling(wsets[li][c], sink)
    ms_rd = statistics.median(time_groups(step_read))
    read_us_by_layer = {}
    for li, L in enumerate(layers):
        def rd(li=li):
            for c in range(COPIES):
                iqd.read_ceiling(wsets[li][c], sink)
        read_us_by_layer[L.name] = round(time_fn(rd, 20) * 1e3 / COPIES, 3)
    read_bytes = sum(L.N * L.K for L in layers) * len(B_LIST)
    ceiling_gbs = read_bytes / (ms_rd * 1e-3) / 1e9
    log(f"read ceiling of the same launches: {ceiling_gbs:.0f} GB/s")

    # ---- practical ceiling of a copy: a device-to-device copy of 1 GiB (read + write bytes) --------
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
        "mismatches": None,
        "batch_variant_rows": batch_variant_rows,
        "config": {
            "workload": "Qwen3-8B-shaped W8A8 decode linears qkv 4096->6144, o 4096->4096, gate_up "
                        "4096->24576, down 12288->4096; per-token quantization + linear (one "
                        "w8a8_linear_bf16 call) at every b=1..8",
            "b": B_LIST,
            "weight_copies": COPIES,
            "weight_bytes_per_step": step_weight_bytes,
            "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
            "tokens_per_s_equiv": round(sum(B_LIST) / (ms * 1e-3), 1),
            "timing": f"{groups} timed groups of {per[0]} step(s), each group one replay of a graph of its "
                      "steps back to back, between HIP events; ms_per_step is their median",
            "ms_per_step_min": round(ms_min, 5),
            "ms_per_step_groups": [round(v, 5) for v in group_ms],
            "separate_calls_ms_per_step": round(ms_sep, 5),
        },
        "gate": gate,
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
            "algorithmic_bytes_per_launch": round(mv_bytes / n_launch),
            # a plain streaming read of the same weight bytes, launched as the
            # step launches its 32 mat-vecs: the part of the peak that launches
            # of these sizes reach with no arithmetic and no output
            "read_ceiling_GBs": round(ceiling_gbs, 1),
            "read_ceiling_frac": round(ceiling_gbs / HBM_PEAK_GBS, 4),
            "read_ceiling_us_by_layer": read_us_by_layer,
            "read_time_over_matvec_time": round(ms_rd / ms_mv, 4),
            "copy_GBs": copy_gbs,  # a 1 GiB device-to-device copy, read + write bytes
            "launches_per_step": n_launch,
        },
        "cpu_baseline": None,
    }

    if args.detail:
        det = []
        for li, L in enumerate(layers):
            for b in B_LIST:
                def one(li=li, b=b):
                    for c in range(COPIES):
                        iqd.w8a8_linear_bf16(xs[li][:b], wsets[li][c], swsets[li], y=ys[(li, b)])

                def lin(li=li, b=b):
                    for c in range(COPIES):
                        iqd.w8a8_linear(qs[li][:b], sas[li][:b], wsets[li][c], swsets[li], y=ys[(li, b)])
                us = time_fn(one, 20) * 1e3 / COPIES
                us2 = time_fn(lin, 20) * 1e3 / COPIES
                det.append({"layer": L.name, "b": b, "us": round(us, 3),
                            "weight_GBs": round(layer_bytes(L) / (us * 1e-6) / 1e9, 1),
                            "linear_only_us": round(us2, 3)})
        out["detail"] = det

    if not args.no_prefill:
        pre = []
        for li, L in enumerate(layers):
            T = PREFILL_T
            qp, sp = iqd.quantize_activations(xs_all[li])
            yp = torch.empty((T, L.N), dtype=torch.bfloat16, device=dev)
            wsp = torch.empty((iqd.workspace_bytes(iqd.IQD_OP_W8A8, T, L.N, L.K, max(PREFILL_SPLITS)),),
                              dtype=torch.uint8, device=dev)
            per_split = {}
            for split in PREFILL_SPLITS:
                def pf(li=li, split=split):
                    for c in range(COPIES):
                        iqd.w8a8_linear(qp, sp, wsets[li][c], swsets[li], split_k=split, y=yp, workspace=wsp)
                per_split[split] = time_fn(pf, 5) * 1e3 / COPIES
            best = min(per_split, key=per_split.get)
            us = per_split[best]
            tops = 2.0 * T * L.N * L.K / (us * 1e-6) / 1e12
            row = {"layer": L.name, "b": T, "split_k": best, "us": round(us, 2), "TOPS": round(tops, 1),
                   "mfma_frac": round(tops / MFMA_I8_PEAK_TOPS, 4),
                   "us_by_split": {str(k): round(v, 2) for k, v in per_split.items()}}
            # Context only: the vendor int8 GEMM (torch._int_mm, hipBLASLt) on the same operands and weight
            # copies, timed eagerly (median of 5); int32 output, no scale epilogue.
            try:
                def vend(li=li):
                    for c in range(COPIES):
                        torch._int_mm(qp, wsets[li][c].t())
                vend()  # eager, outside any graph: the library may record work a graph replay mishandles
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                vts = []
                for _ in range(5):
                    e0.record()
                    vend()
                    e1.record()
                    torch.cuda.synchronize()
                    vts.append(e0.elapsed_time(e1))
                vus = sorted(vts)[2] * 1e3 / COPIES
                row["vendor_int8_gemm"] = {"us": round(vus, 2), "mfma_frac": round(
                    2.0 * T * L.N * L.K / (vus * 1e-6) / 1e12 / MFMA_I8_PEAK_TOPS, 4)}
            except RuntimeError as e:
                row["vendor_int8_gemm"] = {"error": str(e)[:120]}
            pre.append(row)
            del wsp, qp, sp
        out["prefill"] = pre
        log("prefill timed")

    if not args.no_configs:
        out["configs"] = run_configs(iqd, W, np, torch, dev, to_dev_bf16, bits, time_fn, copies_past_cache,
                                     layers, wsets, swsets, xs)
        log("configs timed")

    if args.extra:
        out["extra"] = run_extra(iqd, W, np, torch, dev, time_fn, copies_past_cache, args.no_shards)
        log("extra timed")

    if not args.no_cpu:
        out["cpu_baseline"], out["mismatches"], out["gate"]["oracle"] = run_cpu_baseline(
            np, layers, step_out, step_weight_bytes)
        log(f"cpu baseline: {out['cpu_baseline']['value']} GB/s, {out['mismatches']} mismatches vs the oracle")

    if args.calib:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        src.fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()

    print(json.dumps(out), flush=True)
    if out["batch_variant_rows"] != 0 or (out["mismatches"] or 0) != 0:
        print(f"GATE FAILED: batch_variant_rows={out['batch_variant_rows']} mismatches={out['mismatches']}",
              file=sys.stderr, flush=True)
        sys.exit(1)


def run_configs(iqd, W, np, torch, dev, to_dev_bf16, bits, time_fn, copies_past_cache, layers, wsets, swsets, xs):
    """The other configurations: per-call µs, weight GB/s, % of 8 TB/s and
    tokens/s (b / µs per call)."""
    res = LoggedRows()

    def row(cfg, op, name, K, N, b, us, wbytes, **kw):
        # us: the median of 10 timed repeats (the time_fn call just made); us_min: their minimum, per call
        med, mn = time_fn.last
        us_min = us * mn / med
        r = {"config": cfg, "op": op, "layer": name, "K": K, "N": N, "b": b, "us": round(us, 3),
             "us_min": round(us_min, 3),
             "weight_GBs": round(wbytes / (us * 1e-6) / 1e9, 1),
             "pct_hbm_peak": round(100.0 * wbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
             "tokens_per_s": round(b / (us * 1e-6), 1)}
        r.update(kw)
        res.append(r)

    # C1: the tiny layer, b = 1..5 (its 128 KB of weights stay in the caches)
    L = W.tiny_layer()
    w, sw = torch.from_numpy(L.w).to(dev), torch.from_numpy(L.s_w).to(dev)
    x = to_dev_bf16(L.x)
    for b in range(1, 6):
        y = torch.empty((b, L.N), dtype=torch.bfloat16, device=dev)

        def f(b=b, y=y):
            for _ in range(16):
                iqd.w8a8_linear_bf16(x[:b], w, sw, y=y)
        row("C1 tiny", "w8a8_linear_bf16", "tiny", L.K, L.N, b, time_fn(f, 10) * 1e3 / 16, L.N * L.K + 4 * L.N,
            note="weights cache-resident")

    # C3: block-q8 (fp16 block scales), b in {1, 4, 8, 16}
    for i in range(2):
        Lb = W.blockq8_layer(i, tokens=16)
        by = Lb.N * Lb.K * (1 + 2 / 32)
        nc = copies_past_cache(by)
        wq = torch.from_numpy(Lb.w).to(dev)
        wqs = [wq] + [wq.clone() for _ in range(nc - 1)]
        dw = torch.from_numpy(Lb.d_w.view(np.int16)).view(torch.float16).to(dev)
        qb, db = iqd.quantize_activations(to_dev_bf16(Lb.x), group=32)
        for b in (1, 4, 8, 16):
            yb = torch.empty((b, Lb.N), dtype=torch.bfloat16, device=dev)

            def bq(b=b, yb=yb):
                for c in range(nc):
                    iqd.blockq8_linear(qb[:b], db[:b], wqs[c], dw, y=yb)
            row("C3 blockq8", "blockq8_linear", Lb.name, Lb.K, Lb.N, b, time_fn(bq) * 1e3 / nc, by)
        del wqs, wq

    # C4: Qwen3-14B-shaped layers, own scales and power-of-two scales; plus the
    # pow2-vs-own deviation and the F3-order agreement over a 64-token window
    rep = []
    for li in range(4):
        L14 = W.qwen3_14b_layer(li, tokens=64)
        by = L14.N * L14.K + 4 * L14.N
        nc = copies_past_cache(by)
        w0 = torch.from_numpy(L14.w).to(dev)
        s0 = torch.from_numpy(L14.s_w).to(dev)
        w2, s2 = iqd.pow2_requantize(w0, s0)
        x14 = to_dev_bf16(L14.x)
        q14, sa14 = iqd.quantize_activations(x14)
        outs = {}
        for scales, (wb, sb) in (("own", (w0, s0)), ("pow2", (w2, s2))):
            outs[scales] = bits(iqd.w8a8_linear(q14, sa14, wb, sb))
            wl = [wb] + [wb.clone() for _ in range(nc - 1)]
            for b in (1, 8):
                y14 = torch.empty((b, L14.N), dtype=torch.bfloat16, device=dev)

                def m14(b=b, y14=y14, wl=wl, sb=sb):
                    for c in range(nc):
                        iqd.w8a8_linear_bf16(x14[:b], wl[c], sb, y=y14)
                row("C4 Qwen3-14B", "w8a8_linear_bf16", L14.name, L14.K, L14.N, b, time_fn(m14) * 1e3 / nc, by,
                    scales=scales)
            del wl
        rep.append(pow2_report(np, L14.name, bits, q14, sa14, (w0, s0), (w2, s2), outs))
        log(f"C4 {L14.name} timed")
        del w0, w2, s0, s2
    res.append({"config": "C4 Qwen3-14B", "op": "pow2 vs own scales, 64 tokens", "layers": rep})

    # C5: the LM head (logits + argmax), b in {1, 2, 3, 5, 8}
    Ll = W.lm_head_layer(tokens=8)
    wl = torch.from_numpy(Ll.w).to(dev)
    swl = torch.from_numpy(Ll.s_w).to(dev)
    ql, sl = iqd.quantize_activations(to_dev_bf16(Ll.x))
    lm_bytes = Ll.N * Ll.K + 4 * Ll.N
    for b in (1, 2, 3, 5, 8):
        am = torch.empty((b,), dtype=torch.int32, device=dev)
        lg = torch.empty((b, Ll.N), dtype=torch.bfloat16, device=dev)

        def lh(b=b, am=am, lg=lg):
            for _ in range(4):  # 622 MB of weights: far past the 256 MB Infinity Cache
                iqd.lm_head_argmax(ql[:b], sl[:b], wl, swl, logits=lg, argmax=am)
        row("C5 LM head", "lm_head_argmax", "lm_head", Ll.K, Ll.N, b, time_fn(lh) * 1e3 / 4, lm_bytes)

    # A synthetic Qwen3-8B decode step: 36 blocks of the four linears (each block
    # its own copy of the weights, 6.9 GB) and the LM head, per b.
    blocks = [[wsets[li][0].clone() for li in range(4)] for _ in range(QWEN3_8B_BLOCKS)]
    ybuf = {b: [torch.empty((b, L.N), dtype=torch.bfloat16, device=dev) for L in layers] for b in range(1, 9)}
    step_bytes = QWEN3_8B_BLOCKS * sum(L.N * L.K + 4 * L.N for L in layers) + lm_bytes
    for b in range(1, 9):
        am = torch.empty((b,), dtype=torch.int32, device=dev)

        def full(b=b, am=am):
            for blk in blocks:
                for li in range(4):
                    iqd.w8a8_linear_bf16(xs[li][:b], blk[li], swsets[li], y=ybuf[b][li])
            iqd.lm_head_argmax(ql[:b], sl[:b], wl, swl, logits=False, argmax=am)
        us = time_fn(full, 5) * 1e3
        res.append({"config": "synthetic Qwen3-8B decode step", "op": "36 x (qkv, o, gate_up, down) "
                    "w8a8_linear_bf16 + lm_head_argmax", "b": b, "us": round(us, 1),
                    "weight_GBs": round(step_bytes / (us * 1e-6) / 1e9, 1),
                    "pct_hbm_peak": round(100.0 * step_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
                    "tokens_per_s": round(b / (us * 1e-6), 1), "weight_bytes": step_bytes})
    del blocks, wl
    return res


def pow2_report(np, name, bits, q, s_a, own, p2, outs):
    """pow2 vs own scales on the same tokens: max |delta|, share of outputs
    that differ, a histogram in bf16 spacings; and how many outputs the F3
    order acc * (s_a * s_w) would change, for each scale set (the accumulator
    from a float64 product of the int8 operands, exact since every partial
    sum is an integer below 2^53; the scale product and the last multiply in
    binary32; bf16 by rounding to nearest even)."""
    qh = q.cpu().numpy().astype(np.float64)
    sa = s_a.cpu().numpy().astype(np.float32)

    def f3(w, s):
        acc = qh @ w.cpu().numpy().astype(np.float64).T
        a32 = acc.astype(np.int64).astype(np.float32)
        prod = (a32 * (sa[:, None] * s.cpu().numpy().astype(np.float32)[None, :])).astype(np.float32)
        u = prod.view(np.uint32).astype(np.uint64)
        return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)

    def key(h):
        h = h.astype(np.int64)
        return np.where(h & 0x8000, -(h & 0x7FFF), h & 0x7FFF)

    a, b = outs["own"], outs["pow2"]
    d = np.abs(key(a) - key(b))
    fa = (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    fb = (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return {"layer": name, "outputs": int(a.size),
            "pow2_vs_own": {"max_abs_delta": float(np.abs(fa - fb).max()),
                            "pct_differ": round(100.0 * float((a != b).mean()), 3),
                            "spacings_hist": {"0": int((d == 0).sum()), "1": int((d == 1).sum()),
                                              "2-3": int(((d >= 2) & (d <= 3)).sum()),
                                              "4-15": int(((d >= 4) & (d <= 15)).sum()),
                                              ">=16": int((d >= 16).sum())}},
            "f3_order_disagreements": {"own": int((f3(*own) != a).sum()), "pow2": int((f3(*p2) != b).sum())}}


def run_extra(iqd, W, np, torch, dev, time_fn, copies_past_cache, no_shards=False):
    ext = LoggedRows()
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
            us = time_fn(kq) * 1e3 / nc
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
            us = time_fn(k4) * 1e3 / nc
            ext.append({"op": "kq4_linear", "K": L4.K, "N": L4.N, "b": b, "us": round(us, 2),
                        "weight_GBs": round(by / (us * 1e-6) / 1e9, 1)})
        del planes
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
            us = time_fn(f8) * 1e3 / COPIES
            by = Lf.N * Lf.K + 4 * Lf.N
            ext.append({"op": "fp8_linear", "layer": Lf.name, "K": Lf.K, "N": Lf.N, "b": b, "us": round(us, 2),
                        "weight_GBs": round(by / (us * 1e-6) / 1e9, 1)})
        del wfs, wf0
    # decode attention, Qwen3-8B heads (32 query, 8 kv, D = 128): cache copies
    # in rotation totalling at least 1 GiB, well past the 256 MB Infinity Cache
    name, Hq, Hkv, D = W.QWEN3_8B_ATTN
    for cells in (4096, 32768):
        kv_bytes = cells * Hkv * D * 2 * 2
        ncopy = max(2, min(64, -(-(1 << 30) // kv_bytes)))
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
            us = time_fn(at) * 1e3 / ncopy
            ext.append({"op": "attn_decode", "cells": cells, "Hq": Hq, "Hkv": Hkv, "D": D, "b": b,
                        "us": round(us, 2), "kv_GBs": round(kv_bytes / (us * 1e-6) / 1e9, 1)})
        del ks, vs
    if not no_shards:
        ext += run_shards(iqd, W, np, torch, dev, time_fn, copies_past_cache)
    return ext


def run_shards(iqd, W, np, torch, dev, time_fn, copies_past_cache):
    """One GPU's share of an 8-way tensor-parallel Qwen3-8B decode layer at
    its real shape: column shards of qkv, o and gate_up (N / 8 weight rows),
    a K shard of down (K / 8, whose int32 partial sums an exact all-reduce
    would add; timed here as the same mat-vec with its epilogue) and a
    vocabulary shard of the LM head (151936 / 8 rows).  Weight copies in
    rotation past the cache, as for the other rows."""
    G = 8
    res = LoggedRows()
    for li in range(4):
        L = W.qwen3_8b_layer(li, tokens=8)
        if L.name == "down":
            w = np.ascontiguousarray(L.w[:, : L.K // G])
            x, K, N, kind = L.x[:, : L.K // G], L.K // G, L.N, "K shard"
        else:
            w = np.ascontiguousarray(L.w[: L.N // G])
            x, K, N, kind = L.x, L.K, L.N // G, "column shard"
        s_w = np.ascontiguousarray(L.s_w[:N])
        nc = copies_past_cache(N * K)
        w0 = torch.from_numpy(w).to(dev)
        wsl = [w0] + [w0.clone() for _ in range(nc - 1)]
        swd = torch.from_numpy(s_w).to(dev)
        xd = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
        for b in (1, 8):
            y = torch.empty((b, N), dtype=torch.bfloat16, device=dev)
            wsp = torch.empty((max(16, iqd.workspace_bytes(iqd.IQD_OP_W8A8_BF16, b, N, K, 1)),), dtype=torch.uint8,
                              device=dev)

            def f(b=b, y=y, wsp=wsp):
                for c in range(nc):
                    iqd.w8a8_linear_bf16(xd[:b], wsl[c], swd, y=y, workspace=wsp)
            us = time_fn(f) * 1e3 / nc
            res.append({"op": "shard_8way", "layer": L.name, "kind": kind, "K": K, "N": N, "b": b, "us": round(us, 2),
                        "weight_GBs": round((N * K + 4 * N) / (us * 1e-6) / 1e9, 1)})
        del wsl, w0
    Lh = W.lm_head_layer(tokens=8)
    N = Lh.N // G
    nc = copies_past_cache(N * Lh.K)
    w0 = torch.from_numpy(np.ascontiguousarray(Lh.w[:N])).to(dev)
    wsl = [w0] + [w0.clone() for _ in range(nc - 1)]
    swd = torch.from_numpy(np.ascontiguousarray(Lh.s_w[:N])).to(dev)
    q, sa = iqd.quantize_activations(torch.from_numpy(Lh.x.view(np.int16)).view(torch.bfloat16).to(dev))
    for b in (1, 8):
        am = torch.empty((b,), dtype=torch.int32, device=dev)
        wsp = torch.empty((iqd.workspace_bytes(iqd.IQD_OP_LM_HEAD, b, N, Lh.K, 1),), dtype=torch.uint8, device=dev)

        def fh(b=b, am=am, wsp=wsp):
            for c in range(nc):
                iqd.lm_head_argmax(q[:b], sa[:b], wsl[c], swd, logits=False, argmax=am, workspace=wsp)
        us = time_fn(fh) * 1e3 / nc
        res.append({"op": "shard_8way", "layer": "lm_head", "kind": "vocabulary shard", "K": Lh.K, "N": N, "b": b,
                    "us": round(us, 2), "weight_GBs": round((N * Lh.K + 4 * N) / (us * 1e-6) / 1e9, 1)})
    del wsl, w0
    return res


def run_cpu_baseline(np, layers, step_out, step_weight_bytes):
    """The CPU oracle on the same step (quantize + W8A8 linear, 4 layers,
    b = 1..8), on the host's CPU share of threads, repeated for at least 10 s;
    one step on 1 thread.  Its outputs are also compared with the GPU's
    outputs of the step, every element."""
    import oracle

    nthreads = oracle.default_threads()
    mism = 0
    checked = 0
    t0 = time.time()
    passes = 0
    while passes < 1 or time.time() - t0 < 10.0:
        for b in B_LIST:
            for li, L in enumerate(layers):
                q, s = oracle.quantize_token(L.x[:b])
                y = oracle.w8a8(q, s, L.w, L.s_w, nthreads=nthreads)
                if passes == 0:
                    mism += int((y != step_out[(li, b)]).sum())
                    checked += y.size
        passes += 1
    dt = time.time() - t0
    t1 = time.time()
    for b in B_LIST:
        for L in layers:
            q, s = oracle.quantize_token(L.x[:b])
            oracle.w8a8(q, s, L.w, L.s_w, nthreads=1)
    dt1 = time.time() - t1
    base = {
        "value": round(step_weight_bytes * passes / dt / 1e9, 3),
        "unit": "GB/s",
        "cores": nthreads,
        "kind": "oracle",
        "sample": f"{passes} full step(s): quantize + W8A8 linear for the 4 layers at b=1..8, {dt:.1f} s wall",
        "one_thread_GBs": round(step_weight_bytes / dt1 / 1e9, 3),
        "nproc": os.cpu_count(),
        "cpu_model": cpu_model(),
        "threads_note": "threads = OMP_NUM_THREADS when set (the host's CPU share for one GPU), else every core; "
                        "threads split output rows only",
    }
    gate = {"mismatches": mism, "outputs_checked": checked,
            "what": "every bf16 output of the 32 timed (layer, b) calls against the CPU oracle"}
    return base, mism, gate


if __name__ == "__main__":
    main()
