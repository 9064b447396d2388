#!/usr/bin/env python3
"""Decode-matmul benchmark on one MI355X: packed-ternary (PQ2) weights x
group-128 INT8 activations at M = 1..4 activation columns.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-prefill]
                    [--variants] [--calibrate] [--configs up,qkv,down]

The headline workload is the FFN up projection (K=5120, N=17408), the
largest single-GPU decode shape of the measurement plan.  A step is one
complete call y = W x for each of M = 1, 2, 3, 4 (pq2_gemv_tiles: one fused
quantise + tile matmul launch at M = 1, the quantiser and the tile matmul at
M = 2, 3, 4 at this shape), every call on its own copy of the tile-layout
weights: the
copies (a multiple of 4, >= 1 GiB in total, four times the 256 MB Infinity
Cache) are read in turn, so no call re-reads bytes another call of the last
GiB has read, and every call streams its weights from HBM.  Steps are
captured as HIP graphs (one graph reading every copy once, and one of the
remainder) and replayed; exactly K steps are timed with HIP events between a
synchronize on each side.  Weight preparation is one-time and untimed.

value = algorithmic bytes of the timed calls / their time (GB/s), where a
call's algorithmic bytes are what the method must move for the matmul:
packed weights (34 B / 128 weights) + q + xs + y.  Beside the headline, the
attention QKV (K=5120, N=10240) and FFN down (K=17408, N=5120) shapes are
timed the same way per call, and for each shape and M the tile matmul alone
(the roofline kernel), over the same rotating copies:

  * roofline per config: algorithmic bytes per launch / mean launch time of
    small_m_tiles_kernel (HIP events around graphs of back-to-back launches
    on the launch stream), against 8 TB/s; traffic from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary when its kernel digest matches;
  * ceilings: a linear stream read of the same bytes (pq2_stream_probe,
    shaped like no engine), its best over the shapes the stream sweep found
    best at these sizes (pq2_stream_probe_cfg), the same with one store per
    wave, the decode
    engine's own weight loads (pq2_read_probe), the empty-kernel launch floor
    (pq2_empty_probe), and a fit t = t0 + B / BW of the stream read over
    4..192 MB.

The CPU oracle, timed on a bounded sample of the same work on one thread and
on every core of the affinity mask (rows split between threads, bitwise the
same result), gives cpu_baseline.  --calibrate adds a plain copy kernel of
64 MiB (the yardstick for FETCH_SIZE / WRITE_SIZE); --variants times the
other decode paths (planes, plane order, fused, raw reader, activation
groups) at the QKV shape.
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
VALU_LANE_OPS_PER_S = 16 * 1024 * 2.4e9   # fp32 VALU: 16 lanes per SIMD per clock, 1024 SIMDs, 2.4 GHz
ROTATION_BYTES = 1 << 30
METRIC = "µs/call and achieved HBM GB/s (% of peak) for M=1..4 packed-ternary matmul"
HEADLINE = "up"
DECODE_MS = (1, 2, 3, 4)
WARMUP_MS = 25.0         # replays before each timing
SPLITK_MIN_K = 8192      # split k is timed beside the tile matmul above this k (down)
STREAM_WORKGROUPS = 2048
STREAM_FIT_MB = (4, 8, 16, 24, 48, 96, 192)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def weight_bytes(n, k):
    return n * (k // 128) * 34


def matmul_bytes(m, n, k):
    return weight_bytes(n, k) + m * k + m * (k // 128) * 4 + m * n * 4


def source_digest():
    """Digest of the sources of the tile-layout small-m kernel."""
    h = hashlib.sha256()
    for f in ("tiles.hip", "small_m_common.h", "pq2_device.h"):
        with open(os.path.join(ROOT, "gemm_int8_act_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_summary(name, digest):
    """Key/value lines of a committed profile summary (profiles/<name>), or
    None when it is missing or was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            parts = line.split()
            if len(parts) == 2 and not line.startswith("#"):
                vals[parts[0]] = parts[1]
    return vals if vals.get("kernel_source_digest") == digest else None


def stored_trace(digest):
    """Indented key/value lines of the committed kernel-trace summary, if it
    was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "small_m_tiles_kernel_trace.md")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            parts = line.split()
            if line.startswith("    ") and len(parts) == 2:
                vals[parts[0]] = parts[1]
    return vals if vals.get("kernel_source_digest") == digest else None


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


def time_graph(torch, graph, stream, reps, repeats=5):
    """Milliseconds per replay (median of `repeats` runs of `reps` replays),
    HIP events on the replay stream."""
    out = []
    with torch.cuda.stream(stream):
        # Warm-up of at least WARMUP_MS of replays: the clocks settle after a
        # spell of host-side work (a shorter warm-up left the first shape of
        # a series 5% slow).
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        graph.replay()
        end.record(stream)
        end.synchronize()
        for _ in range(max(0, math.ceil(WARMUP_MS / max(start.elapsed_time(end), 1e-3)) - 1)):
            graph.replay()
        torch.cuda.synchronize()
        for _ in range(repeats):
            start = torch.cuda.Event(enable_timing=True)
            end = torch.cuda.Event(enable_timing=True)
            start.record(stream)
            for _ in range(reps):
                graph.replay()
            end.record(stream)
            end.synchronize()
            out.append(start.elapsed_time(end) / reps)
    out.sort()
    return out[len(out) // 2]


def per_call_us(torch, stream, body, calls, reps):
    """µs per call of a graph of `calls` back-to-back calls."""
    return time_graph(torch, Graph(torch, body, stream), stream, reps) / calls * 1e3


class Config:
    """One decode shape on the device: rotating tile-layout copies, the
    activations, per-M scratch and outputs."""

    def __init__(self, torch, pq2, workloads, name, dev, stream, ms=DECODE_MS):
        w = workloads.WORKLOADS[name]
        self.name, self.n, self.k, self.ms = name, w.n, w.k, ms
        # The shape's other column counts (FFN up M = 8, FFN down M = 16):
        # timed per call beside M = 1..4, outside the roofline's mean.
        self.extra_ms = tuple(m for m in w.ms if m not in ms)
        all_ms = tuple(ms) + self.extra_ms
        self.raw_np, x_cpu = workloads.workload_inputs(name)
        self.x_cpu = x_cpu[: max(all_ms)].contiguous()
        self.wb = weight_bytes(self.n, self.k)
        self.tb = pq2.pq2_tiles_bytes(self.n, self.k)
        per = len(ms)
        self.copies = per * max(1, math.ceil(ROTATION_BYTES / self.tb / per))
        with torch.cuda.stream(stream):
            raw = torch.from_numpy(self.raw_np).to(dev)
            self.tpool = torch.empty((self.copies, self.tb), dtype=torch.uint8, device=dev)
            pq2.pq2_prepare_tiles(raw, self.n, self.k, self.tpool[0], stream=stream)
            for c in range(1, self.copies):
                self.tpool[c].copy_(self.tpool[0])
            self.x = self.x_cpu.to(dev)
            self.q = {m: torch.empty((m, self.k), dtype=torch.int8, device=dev) for m in all_ms}
            self.xs = {m: torch.empty((m, self.k // 128), dtype=torch.float32, device=dev) for m in all_ms}
            self.y = {m: torch.empty((m, self.n), dtype=torch.float32, device=dev) for m in all_ms}
            self.ymm = {m: torch.empty((m, self.n), dtype=torch.float32, device=dev) for m in all_ms}
            for m in all_ms:
                pq2.pq2_quantize_act_i8(self.x[:m], self.q[m], self.xs[m], stream=stream)
        torch.cuda.synchronize()
        log(f"[bench] {name} K={self.k} N={self.n}: weights {self.wb} B, {self.copies} tile copies "
            f"({self.copies * self.tb / 2**30:.2f} GiB)")

    def gemv(self, pq2, m, c, stream):
        pq2.pq2_gemv_tiles(self.x[:m], self.tpool[c], self.y[m], self.q[m], self.xs[m], stream=stream)

    def matmul(self, pq2, m, c, stream):
        pq2.pq2_matmul_small_m_tiles(self.q[m], self.xs[m], self.tpool[c], self.ymm[m], stream=stream)


def measure_config(torch, pq2, cfg, stream, reps, digest):
    """Per-M tile matmul and complete call, and the read ceilings, over the
    config's rotating copies."""
    n, k, copies = cfg.n, cfg.k, cfg.copies
    per_m = {}
    for m in cfg.ms + cfg.extra_ms:
        mm_us = per_call_us(torch, stream, lambda m=m: [cfg.matmul(pq2, m, c, stream) for c in range(copies)],
                            copies, reps)
        call_us = per_call_us(torch, stream, lambda m=m: [cfg.gemv(pq2, m, c, stream) for c in range(copies)],
                              copies, reps)
        torch.cuda.synchronize()
        assert torch.equal(cfg.y[m].view(torch.int32), cfg.ymm[m].view(torch.int32)), \
            f"{cfg.name} M={m}: complete call and tile matmul differ"
        b = matmul_bytes(m, n, k)
        per_m[str(m)] = {
            "matmul_us": round(mm_us, 3),
            "matmul_GBps": round(b / (mm_us * 1e-6) / 1e9, 1),
            "matmul_pct_peak": round(100 * b / (mm_us * 1e-6) / PEAK_HBM_BYTES_PER_S, 1),
            "gemv_call_us": round(call_us, 3),
            "gemv_call_GBps": round(b / (call_us * 1e-6) / 1e9, 1),
            "matmul_bytes": b,
        }
        if k > SPLITK_MIN_K:
            # Cross-workgroup split k (one 1024-element segment per wave, the
            # last workgroup of a tile adds the slices in index order): a
            # different summation order, so compared within a relative 1e-4.
            dev = cfg.x.device
            part = torch.empty((pq2.pq2_tiles_splitk_partial_floats(m, n, k),), dtype=torch.float32, device=dev)
            ctr = torch.zeros((pq2.pq2_tiles_splitk_counter_words(n),), dtype=torch.int32, device=dev)
            ysk = torch.empty((m, n), dtype=torch.float32, device=dev)
            sk_us = per_call_us(torch, stream, lambda m=m: [pq2.pq2_matmul_small_m_tiles_splitk(
                cfg.q[m], cfg.xs[m], cfg.tpool[c], ysk, part, ctr, stream=stream) for c in range(copies)],
                copies, reps)
            torch.cuda.synchronize()
            assert torch.allclose(ysk, cfg.ymm[m], rtol=1e-4, atol=1e-6), f"{cfg.name} M={m}: split k differs"
            assert int(ctr.abs().sum()) == 0, "split-k counters not reset"
            per_m[str(m)]["splitk_matmul_us"] = round(sk_us, 3)
        log(f"[bench] {cfg.name} M={m}: tile matmul {mm_us:.3f} us ({per_m[str(m)]['matmul_GBps']:.0f} GB/s, "
            f"{per_m[str(m)]['matmul_pct_peak']:.1f}% of 8 TB/s), complete call {call_us:.3f} us"
            + (f", split-k matmul {per_m[str(m)]['splitk_matmul_us']:.3f} us" if k > SPLITK_MIN_K else ""))

    # Ceilings at the same bytes, over the same copies.
    words = pq2.pq2_stream_probe_words(STREAM_WORKGROUPS)
    sout = torch.empty((words,), dtype=torch.int32, device=cfg.x.device)
    pout = torch.empty((pq2.pq2_read_probe_words(pq2.LAYOUT_TILES, n, k),), dtype=torch.int32, device=cfg.x.device)
    stream_us = per_call_us(torch, stream, lambda: [pq2.pq2_stream_probe(
        cfg.tpool[c], cfg.tb, STREAM_WORKGROUPS, sout, False, 0x7FFFFFFF, stream=stream) for c in range(copies)],
        copies, reps)
    stream_store_us = per_call_us(torch, stream, lambda: [pq2.pq2_stream_probe(
        cfg.tpool[c], cfg.tb, STREAM_WORKGROUPS, sout, True, stream=stream) for c in range(copies)], copies, reps)
    engine_read_us = per_call_us(torch, stream, lambda: [pq2.pq2_read_probe(
        cfg.tpool[c], pq2.LAYOUT_TILES, n, k, pout, stream=stream) for c in range(copies)], copies, reps)
    # The best read of the same bytes over the shapes the stream sweep found
    # best at these sizes (about 8 loads in flight per SIMD, non-temporal).
    best_us, best_shape = None, None
    cout = torch.empty((1 << 13,), dtype=torch.int32, device=cfg.x.device)
    for policy, ws, loads in BEST_STREAM_SHAPES:
        waves = 4
        us = per_call_us(torch, stream, lambda policy=policy, ws=ws, loads=loads: [pq2.pq2_stream_probe_cfg(
            cfg.tpool[c], cfg.tb, ws * 256, waves, loads, policy, cout, False, 0x7FFFFFFF, stream=stream)
            for c in range(copies)], copies, reps)
        if best_us is None or us < best_us:
            best_us, best_shape = us, f"{STREAM_POLICIES[policy]}, {ws} waves per SIMD, {loads} loads per lane"
    torch.cuda.synchronize()
    ceilings = {
        "stream_read_us": round(stream_us, 3),
        "stream_read_GBps": round(cfg.tb / (stream_us * 1e-6) / 1e9, 1),
        "stream_read_best_us": round(best_us, 3),
        "stream_read_best_frac": round(cfg.tb / (best_us * 1e-6) / PEAK_HBM_BYTES_PER_S, 4),
        "stream_read_best_shape": best_shape,
        "stream_read_plus_store_us": round(stream_store_us, 3),
        "engine_read_probe_us": round(engine_read_us, 3),
        "bytes": cfg.tb,
    }
    log(f"[bench] {cfg.name} ceilings: stream read {stream_us:.3f} us ({ceilings['stream_read_GBps']:.0f} GB/s), "
        f"best shape {best_us:.3f} us ({best_shape}), + one store per wave {stream_store_us:.3f} us, "
        f"engine read probe {engine_read_us:.3f} us")

    tot_b = sum(per_m[str(m)]["matmul_bytes"] for m in cfg.ms)
    tot_us = sum(per_m[str(m)]["matmul_us"] for m in cfg.ms)
    achieved = tot_b / (tot_us * 1e-6) / 1e9
    mean_us = tot_us / len(cfg.ms)
    traffic = stored_summary(f"small_m_tiles_{cfg.name}_traffic.txt", digest)
    trace = stored_trace(digest)
    traced_us = float(trace[f"traced_mean_launch_us_{cfg.name}"]) if trace and \
        f"traced_mean_launch_us_{cfg.name}" in trace else None
    roofline = {
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": PEAK_HBM_BYTES_PER_S / 1e9,
        "unit": "GB/s",
        "frac": round(achieved * 1e9 / PEAK_HBM_BYTES_PER_S, 4),
        "traffic": float(traffic["hbm_bytes_per_launch_avg_m1to4"]) if traffic else None,
        "kernel": f"small_m_tiles_kernel (pq2_matmul_small_m_tiles), {cfg.name} K={k} N={n}, "
                  f"mean over one launch each at M={','.join(map(str, cfg.ms))}",
        "algorithmic_bytes_per_launch_avg": tot_b / len(cfg.ms),
        "mean_launch_us": round(mean_us, 3),
        "kernel_source_digest": digest,
        "stream_read_us": ceilings["stream_read_us"],
        "mean_launch_vs_stream_read": round(mean_us / stream_us, 3),
        "stream_read_best_us": ceilings["stream_read_best_us"],
        "mean_launch_vs_best_stream_read": round(mean_us / best_us, 3),
        # The same kernel's mean duration per dispatch under rocprofv3
        # --kernel-trace (committed summary, same kernel source), and the
        # fraction of 8 TB/s it implies.
        "traced_mean_launch_us": traced_us,
        "traced_frac": round(tot_b / len(cfg.ms) / (traced_us * 1e-6) / PEAK_HBM_BYTES_PER_S, 4) if traced_us else None,
        "stream_read_frac": round(cfg.tb / (stream_us * 1e-6) / PEAK_HBM_BYTES_PER_S, 4),
    }
    return per_m, ceilings, roofline


def headline_step(torch, pq2, cfg, stream, steps, warmup):
    """Exactly `steps` complete steps (M = 1..4, each call on its own copy)."""
    per = len(cfg.ms)
    steps_per_graph = cfg.copies // per

    def steps_fn(count):
        def f():
            for s in range(count):
                for i, m in enumerate(cfg.ms):
                    cfg.gemv(pq2, m, (s * per + i) % cfg.copies, stream)
        return f

    graphs = {steps_per_graph: Graph(torch, steps_fn(steps_per_graph), stream)}
    for count in {warmup % steps_per_graph, steps % steps_per_graph} - {0}:
        graphs[count] = Graph(torch, steps_fn(count), stream)

    def run(count):
        full, rest = divmod(count, steps_per_graph)
        for _ in range(full):
            graphs[steps_per_graph].replay()
        if rest:
            graphs[rest].replay()

    with torch.cuda.stream(stream):
        run(warmup)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        start.record(stream)
        run(steps)
        end.record(stream)
    torch.cuda.synchronize()
    for m in cfg.ms:
        assert torch.isfinite(cfg.y[m]).all(), "non-finite output"
    return start.elapsed_time(end) / steps


def launch_floor_and_stream_fit(torch, pq2, dev, stream, reps):
    """Empty-kernel graph floor and the stream read over 4..192 MB, fitted as
    t = t0 + B / BW (least squares)."""
    floor = {}
    for wg, waves in ((1, 1), (1088, 5)):
        floor[f"{wg}x{waves}"] = round(per_call_us(
            torch, stream, lambda wg=wg, waves=waves: [pq2.pq2_empty_probe(wg, waves, stream=stream)
                                                       for _ in range(200)], 200, reps), 3)
    buf = torch.empty((3 << 29,), dtype=torch.uint8, device=dev)  # 1.5 GiB
    buf.fill_(0x5A)
    out = torch.empty((pq2.pq2_stream_probe_words(STREAM_WORKGROUPS),), dtype=torch.int32, device=dev)
    pts = []
    for mb in STREAM_FIT_MB:
        nb = mb << 20
        copies = buf.numel() // nb
        us = per_call_us(torch, stream, lambda nb=nb, copies=copies: [pq2.pq2_stream_probe(
            buf[c * nb:(c + 1) * nb], nb, STREAM_WORKGROUPS, out, False, 0x7FFFFFFF, stream=stream)
            for c in range(copies)], copies, reps)
        pts.append((nb, us))
    torch.cuda.synchronize()
    del buf
    nbar = sum(b for b, _ in pts) / len(pts)
    tbar = sum(t for _, t in pts) / len(pts)
    slope = sum((b - nbar) * (t - tbar) for b, t in pts) / sum((b - nbar) ** 2 for b, _ in pts)
    t0 = tbar - slope * nbar
    fit = {"t0_us": round(t0, 3), "bw_GBps": round(1e-3 / slope, 1),
           "points": [{"MiB": b >> 20, "us": round(t, 3), "GBps": round(b / (t * 1e-6) / 1e9, 1)} for b, t in pts]}
    log(f"[bench] launch floor (empty kernel, graph): {floor}; stream read fit t = {t0:.3f} us + B / "
        f"{fit['bw_GBps']:.0f} GB/s over {', '.join(str(b >> 20) for b, _ in pts)} MiB")
    return floor, fit


def stream_sweep(torch, pq2, dev, stream, reps):
    """The stream read probe over 4..192 MiB and 256..8192 workgroups (four
    waves each), graphs of back-to-back launches over a rotating 1.5 GiB
    buffer, plus the empty-kernel floor: µs per launch."""
    buf = torch.empty((3 << 29,), dtype=torch.uint8, device=dev)
    buf.fill_(0x5A)
    out = torch.empty((pq2.pq2_stream_probe_words(8192),), dtype=torch.int32, device=dev)
    table = []
    for mb in STREAM_FIT_MB:
        nb = mb << 20
        copies = buf.numel() // nb
        row = {"MiB": mb}
        for wg in (256, 512, 1024, 2048, 4096, 8192):
            us = per_call_us(torch, stream, lambda nb=nb, copies=copies, wg=wg: [pq2.pq2_stream_probe(
                buf[c * nb:(c + 1) * nb], nb, wg, out, False, 0x7FFFFFFF, stream=stream) for c in range(copies)],
                copies, reps)
            row[str(wg)] = round(us, 3)
        table.append(row)
        log(f"[bench] stream sweep {row}")
    floor = {f"{wg}x{w}": round(per_call_us(torch, stream, lambda wg=wg, w=w: [
        pq2.pq2_empty_probe(wg, w, stream=stream) for _ in range(200)], 200, reps), 3)
        for wg, w in ((1, 1), (256, 1), (1088, 5), (2048, 4), (8192, 4))}
    log(f"[bench] empty-kernel floor {floor}")
    shape = stream_shape_sweep(torch, pq2, buf, stream, reps)
    del buf
    return {"stream_read_us": table, "launch_floor_us": floor, "stream_shape_us": shape}


# Shapes of the configurable stream read: the decode weight sizes (QKV, FFN
# up/down) and a large read; waves per SIMD (256 CUs x 4 SIMDs: workgroups of
# four waves, or 256 workgroups of one or two below one wave per SIMD); loads
# in flight per lane.
STREAM_SHAPE_BYTES = (13926400, 23674880, 192 << 20)
STREAM_SHAPE_WAVES_PER_SIMD = (0.25, 0.5, 1, 2, 4, 8)
STREAM_SHAPE_LOADS = (1, 2, 4, 8, 16)
STREAM_POLICIES = ("buffer", "buffer_nt", "lds", "lds_nt")
# (policy, waves per SIMD in workgroups of four, loads per lane): the best
# shapes of the sweep at the decode weight sizes.
BEST_STREAM_SHAPES = ((1, 8, 1), (1, 4, 2), (1, 2, 4), (3, 8, 1))


def stream_shape_sweep(torch, pq2, buf, stream, reps):
    """pq2_stream_probe_cfg over bytes x load instruction and cache policy x
    waves per SIMD x loads in flight per lane, then
    the workgroup size (1..16 waves) at 2 and 4 waves per SIMD: µs per launch
    in graphs of back-to-back launches over the rotating buffer."""
    out = torch.empty((1 << 16,), dtype=torch.int32, device=buf.device)

    def timed(nb, wg, waves, loads, policy):
        copies = buf.numel() // nb
        return round(per_call_us(torch, stream, lambda: [pq2.pq2_stream_probe_cfg(
            buf[c * nb:(c + 1) * nb], nb, wg, waves, loads, policy, out, False, 0x7FFFFFFF, stream=stream)
            for c in range(copies)], copies, reps), 3)

    grid = []
    for nb in STREAM_SHAPE_BYTES:
        for policy, pname in enumerate(STREAM_POLICIES):
            for loads in STREAM_SHAPE_LOADS:
                row = {"bytes": nb, "policy": pname, "loads_per_lane": loads}
                for ws in STREAM_SHAPE_WAVES_PER_SIMD:
                    waves = min(4, int(ws * 4))  # below one wave per SIMD: 256 smaller workgroups
                    row[str(ws)] = timed(nb, int(ws * 1024) // waves, waves, loads, policy)
                grid.append(row)
                log(f"[bench] stream shape {row}")
    wg_size = []
    for ws in (2, 4):
        for loads in (1, 4):
            row = {"bytes": 23674880, "policy": "buffer_nt", "waves_per_simd": ws, "loads_per_lane": loads}
            for waves in (1, 2, 4, 8, 16):
                if waves * loads <= 64:
                    row[str(waves)] = timed(23674880, ws * 1024 // waves, waves, loads, 1)
            wg_size.append(row)
            log(f"[bench] stream workgroup size {row}")
    return {"grid": grid, "workgroup_size": wg_size}


def cpu_baseline(raw, x, n, k, ms, budget_s):
    """The CPU oracle on the same work (quantise + matmul per M) for a bounded
    time, on one thread and on T threads that split the weight rows; the two
    results must be bitwise equal."""
    import concurrent.futures

    import numpy as np

    import oracle
    import workloads
    bits = workloads.bf16_bits(x)
    qs = {m: oracle.quantize_act_i8(bits[:m]) for m in ms}
    # Every core of the affinity mask, but no more threads than the machine's CPU
    # share (OMP_NUM_THREADS, 16 where unset).
    cores = min(len(os.sched_getaffinity(0)), int(os.environ.get("OMP_NUM_THREADS") or 16))

    def matmul_rows(m, r0, r1):
        q, xs = qs[m]
        return oracle.matmul_raw(q, xs, raw[r0:r1], r1 - r0, k)[0]

    def run(threads, pool):
        done_bytes, reps, results = 0, 0, {}
        t0 = time.perf_counter()
        while True:
            for m in ms:
                oracle.quantize_act_i8(bits[:m])
                if threads == 1:
                    results[m] = matmul_rows(m, 0, n)
                else:
                    cuts = [n * i // threads for i in range(threads + 1)]
                    parts = list(pool.map(lambda i, m=m: matmul_rows(m, cuts[i], cuts[i + 1]), range(threads)))
                    results[m] = np.concatenate(parts, axis=1)
                done_bytes += matmul_bytes(m, n, k)
            reps += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        return done_bytes / (time.perf_counter() - t0) / 1e9, reps, time.perf_counter() - t0, results

    single, reps1, dt1, r1 = run(1, None)
    with concurrent.futures.ThreadPoolExecutor(max_workers=cores) as pool:
        multi, repsT, dtT, rT = run(cores, pool)
    for m in ms:
        assert np.array_equal(r1[m].view(np.uint64), rT[m].view(np.uint64)), "threaded oracle differs"
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": round(multi, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{repsT} repetition(s) of quantise+matmul at M={list(ms)} on the full K={k} N={n} shape "
                  f"in {dtT:.1f} s on {cores} threads (weight rows split, bitwise equal to one thread)",
        "single_thread": {"value": round(single, 4), "cores": 1,
                          "sample": f"{reps1} repetition(s) in {dt1:.1f} s"},
        "cpu_model": model,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle work per thread count")
    ap.add_argument("--reps", type=int, default=20, help="graph replays per timing")
    ap.add_argument("--configs", default="up,qkv,down", help="decode shapes to measure (headline first)")
    ap.add_argument("--variants", action="store_true", help="also time the other decode paths at the QKV shape")
    ap.add_argument("--stream-sweep", action="store_true",
                    help="only sweep the stream read probe over sizes and grid widths and print the table")
    ap.add_argument("--only", default=None,
                    help="profiling runs: measure this one decode shape (per-call timings and ceilings; "
                         "no headline step, prefill, floor or CPU baseline), or 'prefill' for the prefill "
                         "timings only, and print its JSON")
    ap.add_argument("--prefill-agroups", action="store_true",
                    help="with --only prefill: also time activation groups of 64 and 32")
    ap.add_argument("--calibrate", action="store_true",
                    help="also run a plain 64 MiB copy kernel (counter calibration; with --only)")
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
    stream = torch.cuda.Stream()
    digest = source_digest()
    if args.stream_sweep:
        print(json.dumps(stream_sweep(torch, pq2, dev, stream, args.reps)), flush=True)
        return
    if args.only == "prefill":
        line = {"only": "prefill", "prefill": bench_prefill(torch, pq2, workloads, dev, stream, args.reps,
                                                             args.prefill_agroups)}
        if args.calibrate:
            calibration_copy(torch, dev, stream)
        print(json.dumps(line), flush=True)
        return
    if args.only:
        cfg = Config(torch, pq2, workloads, args.only, dev, stream)
        per_m, ceil, roof = measure_config(torch, pq2, cfg, stream, args.reps, digest)
        if args.calibrate:
            calibration_copy(torch, dev, stream)
        line = {"only": args.only, "us_per_call": per_m, "ceilings": ceil, "roofline": roof}
        if args.variants and args.only == "qkv":
            line["variants"] = bench_variants(torch, pq2, workloads, cfg, dev, stream, args.reps)
        print(json.dumps(line), flush=True)
        return
    names = [c for c in args.configs.split(",") if c]
    if HEADLINE not in names:
        names.insert(0, HEADLINE)

    results, rooflines, ceilings = {}, {}, {}
    ms_per_step = value = None
    head = None
    for name in names:
        cfg = Config(torch, pq2, workloads, name, dev, stream)
        if name == HEADLINE:
            ms_per_step = headline_step(torch, pq2, cfg, stream, args.steps, args.warmup)
            step_bytes = sum(matmul_bytes(m, cfg.n, cfg.k) for m in cfg.ms)
            value = step_bytes / (ms_per_step * 1e-3) / 1e9
            head = cfg
            log(f"[bench] headline {name}: {ms_per_step * 1e3:.3f} us per step of M={list(cfg.ms)}, "
                f"{value:.0f} GB/s")
        per_m, ceil, roof = measure_config(torch, pq2, cfg, stream, args.reps, digest)
        results[name] = {"k": cfg.k, "n": cfg.n, "weight_copies": cfg.copies,
                         "rotation_bytes": cfg.copies * cfg.tb, "us_per_call": per_m}
        ceilings[name], rooflines[name] = ceil, roof
        if args.variants and name == "qkv":
            results[name]["variants"] = bench_variants(torch, pq2, workloads, cfg, dev, stream, args.reps)
        if name != HEADLINE:
            del cfg
            torch.cuda.empty_cache()

    floor, fit = launch_floor_and_stream_fit(torch, pq2, dev, stream, args.reps)
    roofline = dict(rooflines[HEADLINE])
    roofline["per_config"] = {k: v for k, v in rooflines.items() if k != HEADLINE}

    # pq2_gemv_tiles' choice (the C library's rule, restated for the label).
    fused_ms = [m for m in head.ms if m <= 2 and head.k <= 8192 and m * -(-head.n // 16) <= 1600]
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
            "workload": f"FFN up projection K={head.k} N={head.n}, M=1,2,3,4: x -> y per M with pq2_gemv_tiles "
                        f"(one fused quantise + tile matmul launch at M={','.join(map(str, fused_ms))}, quantiser "
                        f"launch + tile matmul at M={','.join(map(str, [m for m in head.ms if m not in fused_ms]))}), "
                        "each call on its own weight copy",
            "k": head.k, "n": head.n, "ms": list(head.ms),
            "weight_copies": head.copies, "rotation_bytes": head.copies * head.tb,
        },
        "decode": results,
        "ceilings": ceilings,
        "launch_floor_us": floor,
        "stream_read_fit": fit,
        "roofline": roofline,
    }
    del head
    torch.cuda.empty_cache()
    if not args.no_prefill:
        result["prefill"] = bench_prefill(torch, pq2, workloads, dev, stream, 5)
    if args.calibrate:
        calibration_copy(torch, dev, stream)
    if not args.no_cpu_baseline:
        w = workloads.WORKLOADS[HEADLINE]
        raw_np, x_cpu = workloads.workload_inputs(HEADLINE)
        result["cpu_baseline"] = cpu_baseline(raw_np, x_cpu, w.n, w.k, DECODE_MS, args.cpu_budget)
    print(json.dumps(result), flush=True)


def bench_variants(torch, pq2, workloads, cfg, dev, stream, reps):
    """The other decode paths at one shape, same rotating weights (planes,
    plane-order activations, the fused launches, the raw-block reader,
    activation groups of 64 and 32); every path's output bits are checked
    against the tile matmul's (groups 64 and 32: finite only)."""
    n, k, copies = cfg.n, cfg.k, cfg.copies
    wb = weight_bytes(n, k)
    with torch.cuda.stream(stream):
        raw = torch.from_numpy(cfg.raw_np).to(dev)
        pool = torch.empty((copies, wb), dtype=torch.uint8, device=dev)
        pq2.pq2_prepare_planes(raw, n, k, pool[0], stream=stream)
        # The raw-block reader rotates its own copies of the raw rows too.
        rpool = torch.empty((copies, raw.numel()), dtype=torch.uint8, device=dev)
        for c in range(copies):
            if c:
                pool[c].copy_(pool[0])
            rpool[c].copy_(raw.view(-1))
    torch.cuda.synchronize()
    out = {}
    for m in cfg.ms:
        xm, q, xs, y = cfg.x[:m], cfg.q[m], cfg.xs[m], cfg.ymm[m]
        qp = torch.empty_like(q)
        pxs = torch.empty_like(xs)
        qsum = torch.empty((m, k // 128), dtype=torch.int32, device=dev)
        ys = {key: torch.empty((m, n), dtype=torch.float32, device=dev)
              for key in ("planes", "plane_order", "tiles_fused", "planes_fused", "raw")}
        with torch.cuda.stream(stream):
            pq2.pq2_quantize_act_i8_planes(xm, qp, pxs, qsum, stream=stream)
        bodies = {
            "planes_matmul_us": lambda: [pq2.pq2_matmul_small_m(q, xs, pool[c], ys["planes"], stream=stream)
                                         for c in range(copies)],
            "plane_order_matmul_us": lambda: [pq2.pq2_matmul_small_m_planes(qp, pxs, qsum, pool[c],
                                                                           ys["plane_order"], stream=stream)
                                              for c in range(copies)],
            "tiles_fused_call_us": lambda: [pq2.pq2_matmul_small_m_tiles_fused(xm, cfg.tpool[c], ys["tiles_fused"],
                                                                              stream=stream) for c in range(copies)],
            "planes_fused_call_us": lambda: [pq2.pq2_matmul_small_m_fused(xm, pool[c], ys["planes_fused"],
                                                                         stream=stream) for c in range(copies)],
            "raw_matmul_us": lambda: [pq2.pq2_matmul_small_m_raw(q, xs, rpool[c].view(n, -1), ys["raw"],
                                                                 stream=stream) for c in range(copies)],
        }
        t = {key: round(per_call_us(torch, stream, body, copies, reps), 3) for key, body in bodies.items()}
        torch.cuda.synchronize()
        for key, yv in ys.items():
            assert torch.equal(yv.view(torch.int32), y.view(torch.int32)), f"{key} differs at M={m}"
        for ag in (64, 32):
            qg = torch.empty((m, k), dtype=torch.int8, device=dev)
            xsg = torch.empty((m, k // ag), dtype=torch.float32, device=dev)
            yg = torch.empty((m, n), dtype=torch.float32, device=dev)
            with torch.cuda.stream(stream):
                pq2.pq2_quantize_act_i8_g(xm, qg, xsg, ag, stream=stream)
            t[f"agroup{ag}_matmul_us"] = round(per_call_us(torch, stream, lambda qg=qg, xsg=xsg, yg=yg, ag=ag: [
                pq2.pq2_matmul_small_m_tiles_g(qg, xsg, cfg.tpool[c], yg, ag, stream=stream)
                for c in range(copies)], copies, reps), 3)
            t[f"agroup{ag}_two_launch_call_us"] = round(per_call_us(torch, stream, lambda qg=qg, xsg=xsg, yg=yg, ag=ag: [
                (pq2.pq2_quantize_act_i8_g(xm, qg, xsg, ag, stream=stream),
                 pq2.pq2_matmul_small_m_tiles_g(qg, xsg, cfg.tpool[c], yg, ag, stream=stream))
                for c in range(copies)], copies, reps), 3)
            yf = torch.empty((m, n), dtype=torch.float32, device=dev)
            t[f"agroup{ag}_fused_call_us"] = round(per_call_us(torch, stream, lambda yf=yf, ag=ag: [
                pq2.pq2_matmul_small_m_tiles_fused_g(xm, cfg.tpool[c], yf, ag, stream=stream)
                for c in range(copies)], copies, reps), 3)
            torch.cuda.synchronize()
            assert torch.isfinite(yg).all()
            assert torch.equal(yf.view(torch.int32), yg.view(torch.int32)), f"fused agroup {ag} differs at M={m}"
        out[str(m)] = t
        log(f"[bench] variants {cfg.name} M={m}: {t}")
    del pool, rpool
    return out


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


def bench_prefill(torch, pq2, workloads, dev, stream, reps=5, agroups=False):
    """MFMA prefill at the gate (N=6144) and up (N=17408) shapes, M=256..1024,
    from the tile layout, over weight copies that together exceed the 256 MB
    Infinity Cache (each launch reads the next copy).  With agroups, also
    with activation groups of 64 and 32 (pq2_matmul_prefill_tiles_g)."""
    out = {}
    for name in ("prefill_gate", "prefill_up"):
        w = workloads.WORKLOADS[name]
        raw_np, x_cpu = workloads.workload_inputs(name)
        tb = pq2.pq2_tiles_bytes(w.n, w.k)
        copies = max(2, math.ceil((320 << 20) / tb))
        with torch.cuda.stream(stream):
            tiles = torch.empty((copies, tb), dtype=torch.uint8, device=dev)
            pq2.pq2_prepare_tiles(torch.from_numpy(raw_np).to(dev), w.n, w.k, tiles[0], stream=stream)
            for c in range(1, copies):
                tiles[c].copy_(tiles[0])
            x = x_cpu.to(dev)
        torch.cuda.synchronize()
        for m in w.ms:
            q = torch.empty((m, w.k), dtype=torch.int8, device=dev)
            xs = torch.empty((m, w.k // 128), dtype=torch.float32, device=dev)
            y = torch.empty((m, w.n), dtype=torch.float32, device=dev)
            with torch.cuda.stream(stream):
                pq2.pq2_quantize_act_i8(x[:m], q, xs, stream=stream)
            us = per_call_us(torch, stream, lambda q=q, xs=xs, y=y: [
                pq2.pq2_matmul_prefill_tiles(q, xs, tiles[c], y, stream=stream) for c in range(copies)],
                copies, reps)
            torch.cuda.synchronize()
            assert torch.isfinite(y).all()
            ops = 2.0 * m * w.n * w.k
            tops = ops / (us * 1e-6) / 1e12
            # The rescale's own bound: 3 VALU per (m, n, group), issued at 16
            # lanes per SIMD per clock (a wave64 instruction over 4 cycles).
            rescale_us = 3.0 * m * w.n * (w.k // 128) / VALU_LANE_OPS_PER_S * 1e6
            out[f"{name}_m{m}"] = {"us": round(us, 2), "TOPS": round(tops, 1),
                                   "pct_int8_peak": round(100 * tops * 1e12 / PEAK_INT8_OPS_PER_S, 1),
                                   "rescale_bound_us": round(rescale_us, 1),
                                   "rescale_bound_frac": round(rescale_us / us, 3),
                                   "weight_copies": copies}
            log(f"[bench] {name} M={m}: tile-layout prefill {us:.1f} us, {tops:.0f} TOPS "
                f"({out[f'{name}_m{m}']['pct_int8_peak']:.1f}% of 5 POP/s; rescale bound {rescale_us:.1f} us, "
                f"{100 * rescale_us / us:.0f}% of the call)")
            for ag in ((64, 32) if agroups else ()):
                qg = torch.empty((m, w.k), dtype=torch.int8, device=dev)
                xsg = torch.empty((m, w.k // ag), dtype=torch.float32, device=dev)
                with torch.cuda.stream(stream):
                    pq2.pq2_quantize_act_i8_g(x[:m], qg, xsg, ag, stream=stream)
                usg = per_call_us(torch, stream, lambda qg=qg, xsg=xsg, y=y, ag=ag: [
                    pq2.pq2_matmul_prefill_tiles_g(qg, xsg, tiles[c], y, ag, stream=stream) for c in range(copies)],
                    copies, reps)
                torch.cuda.synchronize()
                assert torch.isfinite(y).all()
                out[f"{name}_m{m}"][f"agroup{ag}_us"] = round(usg, 2)
                log(f"[bench] {name} M={m}: activation groups of {ag}: {usg:.1f} us ({100 * (usg / us - 1):+.0f}%)")
        del tiles
        torch.cuda.empty_cache()
    return out


if __name__ == "__main__":
    main()
