#!/usr/bin/env python3
"""Decode-matmul benchmark on one MI355X: packed-ternary (PQ2) weights x
group-128 INT8 activations, the attention-QKV projection shape (K=5120,
N=10240) at M = 1, 2, 3, 4 activation columns.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-prefill]
                    [--calibrate]

A step is one pass of the per-call hot path over one batch: for each M in
1..4, quantise the bf16 activations to INT8 (pq2_quantize_act_i8) and run the
small-m matmul on the tile-layout weights (pq2_matmul_small_m_tiles, the
fastest path over M = 1..4).  The same calls on the row-major prepared planes
(pq2_matmul_small_m), their plane-order variant and both one-launch fused
entry points are timed per M and reported beside it; every path gives the
same output bits, which the run checks.  Weight preparation
(pq2_prepare_tiles / pq2_prepare_planes) is one-time and outside the timing.
Every step reads the next of R weight copies (>= 1 GiB in total per layout,
four times the 256 MB Infinity Cache), so weights stream from HBM.  Steps
are captured as HIP graphs (one graph of R consecutive steps, as a decode
loop runs its calls inside one larger graph, and one of the remainder) and
replayed; exactly K steps are timed with HIP events between a synchronize
on each side.

value = algorithmic bytes of the timed steps / their time (GB/s), where a
call's algorithmic bytes are what the method must move: packed weights
(34 B / 128 weights) + bf16 activations + q + xs (quantiser) and
weights + q + xs + y (matmul).  The per-M matmul kernel duration (HIP events
around graph replays of back-to-back launches on the launch stream) gives the
roofline entry.  The CPU oracle, timed on a bounded sample of the same work,
gives cpu_baseline.  --calibrate adds a plain elementwise copy of 64 MiB
(float32 negate, 64 MiB read + 64 MiB written, five times) so that
rocprofv3 FETCH_SIZE / WRITE_SIZE counts can be scaled to bytes.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_BYTES_PER_S = 8.0e12       # MI355X HBM3E, published peak
PEAK_INT8_OPS_PER_S = 5.0e15        # MI355X dense INT8 MFMA, published peak
ROTATION_BYTES = 1 << 30
METRIC = "µs/call and achieved HBM GB/s (% of peak) for M=1..4 packed-ternary matmul"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def weight_bytes(n, k):
    return n * (k // 128) * 34


def matmul_bytes(m, n, k):
    return weight_bytes(n, k) + m * k + m * (k // 128) * 4 + m * n * 4


def quantize_bytes(m, k):
    return m * k * 2 + m * k + m * (k // 128) * 4


def source_digest():
    """Digest of the sources of the tile-layout small-m kernel."""
    h = hashlib.sha256()
    for f in ("tiles.hip", "small_m_common.h", "pq2_device.h"):
        with open(os.path.join(ROOT, "gemm_int8_act_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(digest):
    """HBM bytes per launch of the tile-layout small-m kernel from the
    committed rocprofv3 counter summary, if it was taken on the current
    kernel source."""
    path = os.path.join(ROOT, "profiles", "small_m_tiles_qkv_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            parts = line.split()
            if len(parts) == 2 and not line.startswith("#"):
                vals[parts[0]] = parts[1]
    if vals.get("kernel_source_digest") != digest:
        return None
    try:
        return float(vals["hbm_bytes_per_launch_avg_m1to4"])
    except (KeyError, ValueError):
        return None


class Graph:
    """A captured HIP graph of a callable, replayed on the capture stream."""

    def __init__(self, torch, fn, stream):
        self.g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            fn()  # warm (first-call attribute setup happens outside capture)
        torch.cuda.synchronize()
        with torch.cuda.graph(self.g, stream=stream):
            fn()

    def replay(self):
        self.g.replay()


def time_graph(torch, graph, stream, reps):
    """Milliseconds per replay, HIP events on the replay stream."""
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        graph.replay()
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(reps):
            graph.replay()
        end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / reps


def cpu_baseline(raw, x, n, k, ms, budget_s):
    """The CPU oracle on the same work (quantise + matmul per M), repeated up
    to the time budget; single thread."""
    import oracle
    import workloads
    bits = workloads.bf16_bits(x)
    done_bytes = 0
    reps = 0
    t0 = time.perf_counter()
    while True:
        for m in ms:
            q, xs = oracle.quantize_act_i8(bits[:m])
            oracle.matmul_raw(q, xs, raw, n, k)
            done_bytes += quantize_bytes(m, k) + matmul_bytes(m, n, k)
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {
        "value": done_bytes / dt / 1e9,
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{reps} repetition(s) of quantise+matmul at M={list(ms)} on the full K={k} N={n} "
                  f"shape, {dt:.1f} s single-threaded",
        "ms_per_step": dt / reps * 1e3,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work")
    ap.add_argument("--reps", type=int, default=20, help="graph replays per per-M timing")
    ap.add_argument("--calibrate", action="store_true",
                    help="also run a plain 64 MiB copy kernel (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch

    import gemm_int8_act_amd as pq2
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = workloads.WORKLOADS["qkv"]
    n, k, ms = w.n, w.k, (1, 2, 3, 4)
    raw_np, x_cpu = workloads.workload_inputs("qkv")
    wb = weight_bytes(n, k)
    tb = pq2.pq2_tiles_bytes(n, k)
    copies = max(2, math.ceil(ROTATION_BYTES / wb))
    log(f"[bench] qkv K={k} N={n} weights {wb} B, {copies} copies per layout "
        f"({copies * wb / 2**30:.2f} GiB planes, {copies * tb / 2**30:.2f} GiB tiles)")

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        raw = torch.from_numpy(raw_np).to(dev)
        pool = torch.empty((copies, wb), dtype=torch.uint8, device=dev)
        tpool = torch.empty((copies, tb), dtype=torch.uint8, device=dev)
        rpool = torch.empty((copies,) + tuple(raw.shape), dtype=torch.uint8, device=dev)  # raw rows, read in place
        pq2.pq2_prepare_planes(raw, n, k, pool[0], stream=stream)
        pq2.pq2_prepare_tiles(raw, n, k, tpool[0], stream=stream)
        for c in range(copies):
            if c:
                pool[c].copy_(pool[0])
                tpool[c].copy_(tpool[0])
            rpool[c].copy_(raw)
        x = x_cpu.to(dev)
        bufs = {}
        pbufs = {}
        for m in ms:
            bufs[m] = (torch.empty((m, k), dtype=torch.int8, device=dev),
                       torch.empty((m, k // 128), dtype=torch.float32, device=dev),
                       torch.empty((m, n), dtype=torch.float32, device=dev))
            pbufs[m] = (torch.empty((m, k), dtype=torch.int8, device=dev),
                        torch.empty((m, k // 128), dtype=torch.float32, device=dev),
                        torch.empty((m, k // 128), dtype=torch.int32, device=dev),
                        torch.empty((m, n), dtype=torch.float32, device=dev))
    torch.cuda.synchronize()

    def step_fn(c):
        def f():
            for m in ms:
                q, xs, y = bufs[m]
                pq2.pq2_gemv_tiles(x[:m], tpool[c], y, q, xs, stream=stream)
        return f

    # One graph holds `copies` consecutive steps (step i reads copy i), as a
    # decode loop runs its calls inside one larger graph; a second graph of
    # the first r steps makes the count exact.
    def steps_fn(count):
        def f():
            for c in range(count):
                step_fn(c)()
        return f

    def run_steps(count, graphs):
        full, rest = divmod(count, copies)
        for _ in range(full):
            graphs[copies].replay()
        if rest:
            graphs[rest].replay()

    step_bytes = sum(quantize_bytes(m, k) + matmul_bytes(m, n, k) for m in ms)
    graphs = {copies: Graph(torch, steps_fn(copies), stream)}
    for count in {args.warmup % copies, args.steps % copies} - {0}:
        graphs[count] = Graph(torch, steps_fn(count), stream)

    # Warmup, then exactly K timed steps.
    with torch.cuda.stream(stream):
        run_steps(args.warmup, graphs)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        start.record(stream)
        run_steps(args.steps, graphs)
        end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    for y in (bufs[m][2] for m in ms):
        assert torch.isfinite(y).all(), "non-finite output"
    del graphs

    # Per-M call timings: graphs of `copies` back-to-back calls, one per copy.
    per_m = {}
    reps = args.reps

    def per_call_us(body):
        return time_graph(torch, Graph(torch, body, stream), stream, reps) / copies * 1e3

    for m in ms:
        q, xs, y = bufs[m]
        qp, pxs, qsum, py = pbufs[m]
        ys = {key: torch.empty((m, n), dtype=torch.float32, device=dev)
              for key in ("planes", "tiles_fused", "planes_fused", "raw")}
        xm = x[:m]

        def calls(kind, m=m, q=q, xs=xs, y=y, qp=qp, pxs=pxs, qsum=qsum, py=py, xm=xm):
            def body():
                for c in range(copies):
                    if kind == "tiles_mm":
                        pq2.pq2_matmul_small_m_tiles(q, xs, tpool[c], y, stream=stream)
                    elif kind == "tiles_call":
                        pq2.pq2_quantize_act_i8(xm, q, xs, stream=stream)
                        pq2.pq2_matmul_small_m_tiles(q, xs, tpool[c], y, stream=stream)
                    elif kind == "gemv":
                        pq2.pq2_gemv_tiles(xm, tpool[c], y, q, xs, stream=stream)
                    elif kind == "tiles_fused":
                        pq2.pq2_matmul_small_m_tiles_fused(xm, tpool[c], ys["tiles_fused"], stream=stream)
                    elif kind == "planes_mm":
                        pq2.pq2_matmul_small_m(q, xs, pool[c], ys["planes"], stream=stream)
                    elif kind == "planes_call":
                        pq2.pq2_quantize_act_i8(xm, q, xs, stream=stream)
                        pq2.pq2_matmul_small_m(q, xs, pool[c], ys["planes"], stream=stream)
                    elif kind == "planes_order_mm":
                        pq2.pq2_matmul_small_m_planes(qp, pxs, qsum, pool[c], py, stream=stream)
                    elif kind == "planes_order_call":
                        pq2.pq2_quantize_act_i8_planes(xm, qp, pxs, qsum, stream=stream)
                        pq2.pq2_matmul_small_m_planes(qp, pxs, qsum, pool[c], py, stream=stream)
                    elif kind == "planes_fused":
                        pq2.pq2_matmul_small_m_fused(xm, pool[c], ys["planes_fused"], stream=stream)
                    elif kind == "raw_mm":
                        pq2.pq2_matmul_small_m_raw(q, xs, rpool[c], ys["raw"], stream=stream)
            return body

        t = {kind: per_call_us(calls(kind)) for kind in
             ("tiles_mm", "tiles_call", "gemv", "tiles_fused", "planes_mm", "planes_call", "planes_order_mm",
              "planes_order_call", "planes_fused", "raw_mm")}
        torch.cuda.synchronize()
        for key, other in (("planes", ys["planes"]), ("plane order", py), ("tiles fused", ys["tiles_fused"]),
                           ("planes fused", ys["planes_fused"]), ("raw reader", ys["raw"])):
            assert torch.equal(other.view(torch.int32), y.view(torch.int32)), \
                f"{key} output differs from the tile-layout output at M={m}"
        gbs = matmul_bytes(m, n, k) / (t["tiles_mm"] * 1e-6) / 1e9
        pgbs = matmul_bytes(m, n, k) / (t["planes_mm"] * 1e-6) / 1e9
        per_m[str(m)] = {
            "matmul_us": round(t["tiles_mm"], 3),
            "matmul_GBps": round(gbs, 1),
            "matmul_pct_peak": round(100 * gbs * 1e9 / PEAK_HBM_BYTES_PER_S, 1),
            "complete_call_us": round(t["tiles_call"], 3),
            "gemv_call_us": round(t["gemv"], 3),
            "fused_call_us": round(t["tiles_fused"], 3),
            "planes_matmul_us": round(t["planes_mm"], 3),
            "planes_matmul_GBps": round(pgbs, 1),
            "planes_complete_call_us": round(t["planes_call"], 3),
            "planes_fused_call_us": round(t["planes_fused"], 3),
            "plane_order_matmul_us": round(t["planes_order_mm"], 3),
            "plane_order_complete_call_us": round(t["planes_order_call"], 3),
            "raw_matmul_us": round(t["raw_mm"], 3),
            "matmul_bytes": matmul_bytes(m, n, k),
        }
        log(f"[bench] M={m}: tiles matmul {t['tiles_mm']:.3f} us ({gbs:.0f} GB/s, "
            f"{100 * gbs * 1e9 / PEAK_HBM_BYTES_PER_S:.1f}% of 8 TB/s), call {t['tiles_call']:.3f}, "
            f"gemv {t['gemv']:.3f}, "
            f"fused {t['tiles_fused']:.3f}; planes matmul {t['planes_mm']:.3f} ({pgbs:.0f} GB/s), "
            f"call {t['planes_call']:.3f}, fused {t['planes_fused']:.3f}; plane order matmul "
            f"{t['planes_order_mm']:.3f}, call {t['planes_order_call']:.3f}; raw reader matmul {t['raw_mm']:.3f}")

    # Smaller activation groups (page "Kernel experiments", section C, Tests
    # 8 and 9): the tile matmul and the complete call with 64- and 32-element
    # activation groups, beside the group-128 figures above.
    agroups = {}
    for ag in (64, 32):
        agroups[str(ag)] = {}
        for m in ms:
            xm = x[:m]
            qg = torch.empty((m, k), dtype=torch.int8, device=dev)
            xsg = torch.empty((m, k // ag), dtype=torch.float32, device=dev)
            yg = torch.empty((m, n), dtype=torch.float32, device=dev)
            with torch.cuda.stream(stream):
                pq2.pq2_quantize_act_i8_g(xm, qg, xsg, ag, stream=stream)

            def g_calls(call, m=m, xm=xm, qg=qg, xsg=xsg, yg=yg, ag=ag):
                def body():
                    for c in range(copies):
                        if call:
                            pq2.pq2_quantize_act_i8_g(xm, qg, xsg, ag, stream=stream)
                        pq2.pq2_matmul_small_m_tiles_g(qg, xsg, tpool[c], yg, ag, stream=stream)
                return body

            mm_us, call_us = per_call_us(g_calls(False)), per_call_us(g_calls(True))
            torch.cuda.synchronize()
            assert torch.isfinite(yg).all(), "non-finite output"
            agroups[str(ag)][str(m)] = {
                "matmul_us": round(mm_us, 3),
                "complete_call_us": round(call_us, 3),
                "matmul_vs_group128": round(mm_us / per_m[str(m)]["matmul_us"], 3),
            }
        log(f"[bench] activation groups of {ag}: matmul us " +
            ", ".join(f"M={m} {v['matmul_us']:.3f}" for m, v in agroups[str(ag)].items()))

    # Read ceiling: each layout's decode-engine weight loads with no
    # arithmetic (pq2_read_probe), over the same rotating copies.
    probe = {}
    for name, layout, wpool in (("tiles", pq2.LAYOUT_TILES, tpool), ("planes", pq2.LAYOUT_PLANES, pool)):
        pout = torch.empty((pq2.pq2_read_probe_words(layout, n, k),), dtype=torch.int32, device=dev)

        def probe_calls(layout=layout, wpool=wpool, pout=pout):
            def body():
                for c in range(copies):
                    pq2.pq2_read_probe(wpool[c], layout, n, k, pout, stream=stream)
            return body

        p_us = per_call_us(probe_calls())
        probe[name] = {"us": round(p_us, 3), "weight_GBps": round(wb / (p_us * 1e-6) / 1e9, 1)}
    torch.cuda.synchronize()
    log(f"[bench] read probe (weights only, no arithmetic): tiles {probe['tiles']['us']:.3f} us "
        f"({probe['tiles']['weight_GBps']:.0f} GB/s), planes {probe['planes']['us']:.3f} us "
        f"({probe['planes']['weight_GBps']:.0f} GB/s)")

    tot_bytes = sum(v["matmul_bytes"] for v in per_m.values())
    tot_us = sum(v["matmul_us"] for v in per_m.values())
    achieved = tot_bytes / (tot_us * 1e-6) / 1e9
    ptot_us = sum(v["planes_matmul_us"] for v in per_m.values())
    digest = source_digest()
    traffic = stored_traffic(digest)
    roofline = {
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": PEAK_HBM_BYTES_PER_S / 1e9,
        "unit": "GB/s",
        "frac": round(achieved * 1e9 / PEAK_HBM_BYTES_PER_S, 4),
        "traffic": traffic,
        "kernel": "small_m_tiles_kernel (pq2_matmul_small_m_tiles), mean over one launch each at M=1..4",
        "algorithmic_bytes_per_launch_avg": tot_bytes / len(ms),
        "mean_launch_us": round(tot_us / len(ms), 3),
        "kernel_source_digest": digest,
        "planes_kernel_achieved": round(tot_bytes / (ptot_us * 1e-6) / 1e9, 1),
        "planes_kernel_mean_launch_us": round(ptot_us / len(ms), 3),
        # The same layout's weight loads alone (pq2_read_probe): the mean
        # launch as a multiple of that read time.
        "read_probe_us": probe["tiles"]["us"],
        "mean_launch_vs_read_probe": round((tot_us / len(ms)) / probe["tiles"]["us"], 3),
    }

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": "attention QKV projection K=5120 N=10240, M=1,2,3,4 (x -> y per M with pq2_gemv_tiles: "
                        "fused quantise + tile matmul at M=1, quantiser + tile matmul at M=2..4)",
            "k": k, "n": n, "ms": list(ms),
            "weight_copies": copies, "rotation_bytes": copies * tb,
        },
        "us_per_call": per_m,
        "activation_groups_us_per_call": agroups,
        "read_probe_us_per_call": probe,
        "roofline": roofline,
    }

    if not args.no_prefill:
        result["prefill"] = bench_prefill(torch, pq2, workloads, dev, stream)
    if args.calibrate:
        calibration_copy(torch, dev, stream)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(raw_np, x_cpu, n, k, ms, args.cpu_budget)
    print(json.dumps(result), flush=True)


def calibration_copy(torch, dev, stream):
    """A plain elementwise copy of known size (64 MiB read, 64 MiB written per
    launch), the yardstick for the FETCH_SIZE / WRITE_SIZE counters."""
    with torch.cuda.stream(stream):
        src = torch.ones(16 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log(f"[bench] calibration copy: 5 x {src.numel() * 4} bytes read and written")


def bench_prefill(torch, pq2, workloads, dev, stream):
    """MFMA prefill at the gate (N=6144) and up (N=17408) shapes, M=256..1024:
    from the tile layout (the decode step's weights), and from the planes with
    natural- and plane-order activations; all give the same bits."""
    out = {}
    for name in ("prefill_gate", "prefill_up"):
        w = workloads.WORKLOADS[name]
        raw_np, x_cpu = workloads.workload_inputs(name)
        with torch.cuda.stream(stream):
            planes = torch.empty(weight_bytes(w.n, w.k), dtype=torch.uint8, device=dev)
            tiles = torch.empty(pq2.pq2_tiles_bytes(w.n, w.k), dtype=torch.uint8, device=dev)
            raw = torch.from_numpy(raw_np).to(dev)
            pq2.pq2_prepare_planes(raw, w.n, w.k, planes, stream=stream)
            pq2.pq2_prepare_tiles(raw, w.n, w.k, tiles, stream=stream)
            x = x_cpu.to(dev)
        torch.cuda.synchronize()
        for m in w.ms:
            q = torch.empty((m, w.k), dtype=torch.int8, device=dev)
            qp = torch.empty((m, w.k), dtype=torch.int8, device=dev)
            xs = torch.empty((m, w.k // 128), dtype=torch.float32, device=dev)
            qsum = torch.empty((m, w.k // 128), dtype=torch.int32, device=dev)
            y = torch.empty((m, w.n), dtype=torch.float32, device=dev)
            with torch.cuda.stream(stream):
                pq2.pq2_quantize_act_i8(x[:m], q, xs, stream=stream)
                pq2.pq2_quantize_act_i8_planes(x[:m], qp, xs, qsum, stream=stream)

            def f(q=q, xs=xs, y=y):
                for _ in range(10):
                    pq2.pq2_matmul_prefill(q, xs, planes, y, stream=stream)

            def fp(qp=qp, xs=xs, y=y):
                for _ in range(10):
                    pq2.pq2_matmul_prefill_planes(qp, xs, planes, y, stream=stream)

            yt = torch.empty((m, w.n), dtype=torch.float32, device=dev)

            def ft(q=q, xs=xs, yt=yt):
                for _ in range(10):
                    pq2.pq2_matmul_prefill_tiles(q, xs, tiles, yt, stream=stream)

            t_us = time_graph(torch, Graph(torch, f, stream), stream, 5) / 10 * 1e3
            tp_us = time_graph(torch, Graph(torch, fp, stream), stream, 5) / 10 * 1e3
            tt_us = time_graph(torch, Graph(torch, ft, stream), stream, 5) / 10 * 1e3
            # Smaller activation groups (one scale per 64 or 32 activations),
            # same weights: the tile-layout prefill with per-group rescales.
            ag_us = {}
            for agroup in (64, 32):
                qg = torch.empty((m, w.k), dtype=torch.int8, device=dev)
                xsg = torch.empty((m, w.k // agroup), dtype=torch.float32, device=dev)
                yg = torch.empty((m, w.n), dtype=torch.float32, device=dev)
                with torch.cuda.stream(stream):
                    pq2.pq2_quantize_act_i8_g(x[:m], qg, xsg, agroup, stream=stream)

                def fg(qg=qg, xsg=xsg, yg=yg, agroup=agroup):
                    for _ in range(10):
                        pq2.pq2_matmul_prefill_tiles_g(qg, xsg, tiles, yg, agroup, stream=stream)

                ag_us[agroup] = time_graph(torch, Graph(torch, fg, stream), stream, 5) / 10 * 1e3
            torch.cuda.synchronize()
            assert torch.equal(yt.view(torch.int32), y.view(torch.int32)), f"prefill from tiles differs at M={m}"
            ops = 2.0 * m * w.n * w.k
            tops = ops / (tt_us * 1e-6) / 1e12
            out[f"{name}_m{m}"] = {"us": round(tt_us, 2), "TOPS": round(tops, 1),
                                   "pct_int8_peak": round(100 * tops * 1e12 / PEAK_INT8_OPS_PER_S, 1),
                                   "planes_us": round(t_us, 2), "planes_plane_order_us": round(tp_us, 2),
                                   "agroup64_us": round(ag_us[64], 2), "agroup32_us": round(ag_us[32], 2)}
            log(f"[bench] {name} M={m}: tile layout {tt_us:.1f} us, {tops:.0f} TOPS (planes {t_us:.1f} us, "
                f"planes with plane-order input {tp_us:.1f} us; activation groups 64 / 32: "
                f"{ag_us[64]:.1f} / {ag_us[32]:.1f} us)")
        del planes, tiles
    return out


if __name__ == "__main__":
    main()
