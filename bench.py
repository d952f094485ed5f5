#!/usr/bin/env python3
"""Benchmark of the weight-only FP4 / FP8 matmul library on one MI355X.

Headline (one JSON line on stdout): the FP4 decode GEMV, M in {1, 2, 4, 8},
N = K = 5120, block 16, BF16 activations N(0,1), bias.  One step = the four
GEMV calls (one per M), each on its own copy of the weights; 73 copies
(about 1 GiB) rotate so every call streams its weights from HBM rather than
from the 256 MB last-level cache.  Steps run as captured HIP graphs of eight
steps each, so host launch overhead does not sit between the kernels.

    value    = packed weight + scale bytes per step / step time  [GB/s]
    roofline = the GEMV kernel: algorithmic bytes (weights, scales,
               activations, bias, output) per launch / mean launch time
               (timed region / launches, HIP events on the launch stream),
               against the 8 TB/s HBM3E peak
    cpu_baseline = the CPU oracle on the same workload (GB/s of weights), plus
               one oracle call on 64 rows of each M = 8192 prefill workload
               (TFLOP/s of that sample, full-size time extrapolated)

"extra" reports the spread of the headline (each graph replay timed on its
own), the other workloads (small FP16 GEMV, FP4 prefill GEMM with the dequant
+ hipBLASLt baseline beside it, FP8 GEMV and prefill, wide-output GEMV, the
dequant kernel, the W8A8 and W4A4 modes; prefill timed over 200 dispatches
after 50 warm-up ones) and
measured HBM read and copy rates, the read rate also at each GEMV's weight
bytes per launch.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       [--no-extra] [--profile-kernel fp4_gemv|copy]
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import fp8_weight_only_fp4w_amd as fw  # noqa: E402
import workloads  # noqa: E402

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense BF16 / FP16 MFMA
ROTATE_BYTES = 1 << 30          # rotate weight copies past the 256 MB MALL
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fp4_gemv_decode_traffic.json")
GEMV_SOURCES = ["fp8_weight_only_fp4w_amd/csrc/gemv.hip", "fp8_weight_only_fp4w_amd/csrc/device.h",
                "fp8_weight_only_fp4w_amd/csrc/nvfp4_block.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------------ inputs on device

def dev_bits(bits, dtype):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda")
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16)


def dev_u8(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def fp4_on_device(p, copies=1):
    """Activations, bias, ws2 once; `copies` distinct device copies of B and scales."""
    B = dev_u8(p.B)
    ws = dev_u8(p.weight_scale)
    Bs = [B] + [B.clone() for _ in range(copies - 1)]
    wss = [ws] + [ws.clone() for _ in range(copies - 1)]
    return dict(A=dev_bits(p.A, p.dtype), B=Bs, ws=wss,
                ws2=torch.tensor([p.weight_scale_2], dtype=torch.float32, device="cuda"),
                bias=None if p.bias is None else dev_bits(p.bias, p.dtype))


def fp8_on_device(p, copies=1):
    B = dev_u8(p.B)
    bs = torch.from_numpy(p.b_scale).to("cuda")
    return dict(A=dev_bits(p.A, p.dtype), B=[B] + [B.clone() for _ in range(copies - 1)],
                bs=[bs] + [bs.clone() for _ in range(copies - 1)],
                bias=None if p.bias is None else dev_bits(p.bias, p.dtype))


def copies_for(weight_bytes):
    return max(1, -(-ROTATE_BYTES // weight_bytes))


# ------------------------------------------------------------------ timing helpers

def capture(fn):
    """Capture fn() (enqueue-only work on the current stream) into a graph."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm the allocator / library outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_graphs(graphs, steps, warmup, min_warm_s=0.0):
    """Replay graphs round-robin: warmup untimed (at least `warmup` replays
    and, in whole rounds over the graphs, at least `min_warm_s` seconds),
    then exactly `steps` timed replays bracketed by synchronisation; returns
    (wall s, event s)."""
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < min_warm_s:
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, start.elapsed_time(stop) / 1e3


def time_rotating(call, R, launches, G=20):
    """Per-launch seconds of call(r) over rotating copies r = 0 .. R-1, from
    graphs of G launches each (HIP events around the timed replays; 20, as
    the headline's graphs hold 20 steps).  The
    untimed warm-up runs for at least 30 ms: right after the inputs are
    built the GPU needs that long to reach its steady rate (the wide GEMV's
    first 64 launches ran 16 % slower than the ones after them)."""
    n = -(-R // G)
    gs = [capture(lambda i=i: [call((i * G + k) % R) for k in range(G)]) for i in range(n)]
    reps = max(1, launches // G)
    _, e = time_graphs(gs, reps, min(reps, 4), min_warm_s=0.03)
    del gs
    return e / (reps * G)


def time_calls(fn_list, steps, warmup):
    """Direct launches (for long kernels where launch overhead is hidden)."""
    for i in range(warmup):
        fn_list[i % len(fn_list)]()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        fn_list[i % len(fn_list)]()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / 1e3


# ------------------------------------------------------------------ headline

STEPS_PER_GRAPH = 20  # steps captured in one graph (80 launches: amortises the graph launch, as a decode step's graph of ~120 GEMVs does)


def gemv_decode(steps, warmup):
    w = workloads.WORKLOADS["fp4_gemv_decode"]
    Ms = w.Ms
    probs = {M: w.make(M=M) for M in Ms}
    p0 = probs[Ms[0]]
    weight_bytes = p0.B.nbytes + p0.weight_scale.nbytes
    R = copies_for(weight_bytes)
    d = fp4_on_device(p0, copies=R)
    A = {M: dev_bits(probs[M].A, "bf16") for M in Ms}
    out = {M: torch.empty(M, w.N, dtype=torch.bfloat16, device="cuda") for M in Ms}

    def step(r):
        for M in Ms:
            fw.fp4w_matmul(A[M], d["B"][r], d["ws"][r], d["ws2"], d["bias"], 16, out=out[M])

    # graphs of STEPS_PER_GRAPH consecutive steps (each step on the next copy
    # of the weights), and single-step graphs for a remainder
    G = max(1, min(STEPS_PER_GRAPH, steps))
    n_groups = -(-R // G)
    groups = [capture(lambda i=i: [step((i * G + k) % R) for k in range(G)]) for i in range(n_groups)]
    singles = [capture(lambda r=r: step(r)) for r in range(min(R, G))]
    for i in range(warmup // G):
        groups[i % n_groups].replay()
    for i in range(warmup % G):
        singles[i % len(singles)].replay()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for i in range(steps // G):
        groups[i % n_groups].replay()
    for i in range(steps % G):
        singles[i % len(singles)].replay()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_step = start.elapsed_time(stop) / 1e3 / steps
    # spread: each replay of a G-step graph timed on its own (events between
    # replays), as mean microseconds per launch within that replay
    n_rep = max(64, steps // G)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_rep)]
    for i, (a, b) in enumerate(evs):
        a.record()
        groups[i % n_groups].replay()
        b.record()
    torch.cuda.synchronize()
    per_launch = np.array([a.elapsed_time(b) * 1e3 / (G * len(Ms)) for a, b in evs])
    per_replay = {"replays": n_rep, "launches_per_replay": G * len(Ms),
                  "us_per_launch_p10": round(float(np.percentile(per_launch, 10)), 3),
                  "us_per_launch_p50": round(float(np.percentile(per_launch, 50)), 3),
                  "us_per_launch_p90": round(float(np.percentile(per_launch, 90)), 3)}
    del groups, singles
    # algorithmic bytes of one step (four launches)
    alg = 0
    for M in Ms:
        alg += weight_bytes + M * w.K * 2 + w.N * 2 + M * w.N * 2 + 4
    # per-M breakdown (graphs of G launches of one M, same rotation)
    per_m = {}
    for M in Ms:
        gs = [capture(lambda i=i, M=M: [fw.fp4w_matmul(A[M], d["B"][(i * G + k) % R], d["ws"][(i * G + k) % R],
                                                        d["ws2"], d["bias"], 16, out=out[M]) for k in range(G)])
              for i in range(n_groups)]
        reps = max(steps // G, 16)
        _, e = time_graphs(gs, reps, 2)
        t = e / (reps * G)
        per_m[str(M)] = {"us": round(t * 1e6, 3), "weight_GBps": round(weight_bytes / t / 1e9, 1)}
        del gs
    return dict(workload=w, Ms=Ms, weight_bytes=weight_bytes, R=R, per_step=per_step, wall=wall,
                alg_bytes_step=alg, per_m=per_m, per_replay=per_replay)


# ------------------------------------------------------------------ CPU baseline

def cpu_baseline(min_seconds=10.0):
    """The CPU oracle, as it stands, on the headline workload: all four M of
    one step (full N), repeated until at least `min_seconds` have passed."""
    from oracle import reference as ref
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = None
    w = workloads.WORKLOADS["fp4_gemv_decode"]
    probs = [w.make(M=M) for M in w.Ms]
    wb = probs[0].B.nbytes + probs[0].weight_scale.nbytes
    done, t0 = 0, time.perf_counter()
    while True:
        for p in probs:
            ref.matmul_fp4_reference(p.A, p.dtype, p.B, p.weight_scale, 16, p.weight_scale_2, p.bias)
            done += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    res = {"value": round(done * wb / el / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": f"{done} oracle calls (M in {list(w.Ms)}, N=K=5120, full output) in {el:.1f} s; "
                     f"float64 dequant + numpy BLAS dgemm; cores = BLAS threads; host has "
                     f"{os.cpu_count()} logical CPUs, affinity {len(os.sched_getaffinity(0))}"}
    # prefill: one oracle call on 64 rows of each M = 8192 prefill workload
    rows = 64
    pre = {}
    for name, wl in (("fp4_prefill", workloads.WORKLOADS["fp4_prefill"]),
                     ("fp8_prefill", workloads.WORKLOADS["fp8_gemv"])):
        p = wl.make(M=rows)
        t0 = time.perf_counter()
        if wl.op == "fp4":
            ref.matmul_fp4_reference(p.A, p.dtype, p.B, p.weight_scale, wl.block_size, p.weight_scale_2, p.bias)
        else:
            ref.matmul_fp8_reference(p.A, p.dtype, p.B, p.b_scale, wl.block_size, p.bias)
        el = time.perf_counter() - t0
        full_m = 8192
        pre[name] = {"value": round(2.0 * rows * wl.N * wl.K / el / 1e12, 6), "unit": "TFLOP/s",
                     "sample_rows": rows, "sample_s": round(el, 2),
                     "extrapolated_full_call_s": round(el * full_m / rows, 1),
                     "extrapolation": f"linear in M from {rows} to {full_m} rows (the oracle's weight decode, "
                                      f"paid once per call, is counted {full_m // rows} times: an upper bound)"}
    res["prefill_sampled"] = pre
    return res


# ------------------------------------------------------------------ extra workloads

def hbm_copy_gbps():
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    t = time_calls([lambda: dst.copy_(src)], 20, 3)
    return round(2 * n * 20 / t / 1e9, 1)


def hbm_read(sizes):
    """Measured HBM read rate from this repository's read-stream kernel
    (libhbmprobe.so): the peak over a 4 GiB buffer, and for each entry of
    `sizes` (name -> bytes per launch) the rate at that many bytes per launch
    over enough rotated slices to pass 1 GiB (past the last-level cache),
    launched back to back from a HIP graph.  Each is the best over grid sizes
    and loads in flight per thread.  For each size it also streams the same
    slices with the decode GEMV's load structure alone (no arithmetic)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "fp8_weight_only_fp4w_amd", "libhbmprobe.so"))
    lib.hbm_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_int, ctypes.c_uint32,
                                   ctypes.c_void_p, ctypes.c_void_p]
    lib.hbm_read_probe.restype = ctypes.c_int
    lib.hbm_lds_stream_probe.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_int, ctypes.c_uint32,
                                         ctypes.c_void_p, ctypes.c_void_p]
    lib.hbm_lds_stream_probe.restype = ctypes.c_int
    grids, unrolls = (256, 512, 1024, 2048), (4, 8)
    big_bytes = 4 << 30
    buf = torch.full((big_bytes,), 1, dtype=torch.uint8, device="cuda")  # every thread's XOR is 0
    sink = torch.empty(max(grids) * 512, dtype=torch.int32, device="cuda")
    key = 0xFFFFFFFF  # never equal to a reduction of these bytes: nothing is stored

    def launch(ptr, nbytes, grid, unroll):
        rc = lib.hbm_read_probe(ctypes.c_void_p(ptr), nbytes, grid, unroll, key, ctypes.c_void_p(sink.data_ptr()),
                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hbm_read_probe failed ({rc})")

    peak = {}
    for g in grids:
        for u in unrolls:
            t = time_calls([lambda g=g, u=u: launch(buf.data_ptr(), big_bytes, g, u)], 10, 2)
            peak[f"grid{g}_u{u}"] = round(big_bytes * 10 / t / 1e9, 1)
    res = {"peak_GBps": max(peak.values()), "peak_config": max(peak, key=peak.get), "buffer_bytes": big_bytes,
           "sweep_4GiB": peak, "at_size": {}}
    for name, nbytes in sizes.items():
        nb = nbytes - nbytes % 16
        slices = max(2, -(-ROTATE_BYTES // nb))
        assert slices * nb <= big_bytes
        sweep = {}
        for g in grids:
            for u in unrolls:
                def body(g=g, u=u):
                    for i in range(slices):
                        launch(buf.data_ptr() + i * nb, nb, g, u)
                body()
                torch.cuda.synchronize()
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph):
                    body()
                graph.replay()
                torch.cuda.synchronize()
                t = time_calls([graph.replay], 5, 1)
                sweep[f"grid{g}_u{u}"] = round(nb * slices * 5 / t / 1e9, 1)
                del graph
        res["at_size"][name] = {"bytes": nb, "slices": slices, "GBps": max(sweep.values()),
                                "config": max(sweep, key=sweep.get), "sweep": sweep}
        # the decode GEMV's load structure alone (8-wave workgroups, 2 KiB
        # units through per-wave LDS rings, 4 in flight), same slices
        lsweep = {}
        for g in (160, 256):
            units = nb // (g * 8 * 2048)
            if units < 1:
                continue
            sb = g * 8 * units * 2048

            def lbody(g=g, units=units):
                for i in range(slices):
                    rc = lib.hbm_lds_stream_probe(ctypes.c_void_p(buf.data_ptr() + i * nb), nb, g, units, key,
                                                  ctypes.c_void_p(sink.data_ptr()),
                                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
                    if rc != 0:
                        raise RuntimeError(f"hbm_lds_stream_probe failed ({rc})")
            lbody()
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                lbody()
            graph.replay()
            torch.cuda.synchronize()
            t = time_calls([graph.replay], 5, 1)
            lsweep[f"grid{g}"] = {"bytes": sb, "us": round(t / 5 / slices * 1e6, 2), "GBps": round(sb * slices * 5 / t / 1e9, 1)}
            del graph
        res["at_size"][name]["gemv_structure"] = lsweep
    del buf, sink
    return res


def mfma_peak():
    """Measured dense BF16 MFMA rate from this repository's probe
    (libmfmaprobe.so): back-to-back independent 32x32x16 MFMAs on 512
    workgroups, one or two waves per SIMD, with operands that change every
    instruction (random BF16 bits) or constant ones.  Under this load the
    clock follows the operand bits, so the random-operand rate is the
    ceiling a GEMM on random data can approach."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "fp8_weight_only_fp4w_amd", "libmfmaprobe.so"))
    lib.mfma_peak_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint32,
                                    ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
    lib.mfma_peak_probe.restype = ctypes.c_int64
    grid, iters = 512, 4000
    sink = torch.empty(grid * 512, dtype=torch.float32, device="cuda")
    key = 0x7FC00123  # a NaN payload no sum of these finite products has: nothing is stored
    res = {"grid": grid, "iters": iters}
    for waves in (1, 2):
        for rnd, label in ((1, "random"), (0, "constant")):
            mfmas = [0]

            def launch(waves=waves, rnd=rnd):
                n = lib.mfma_peak_probe(grid, waves, iters, rnd, 12345, key, ctypes.c_void_p(sink.data_ptr()),
                                        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
                if n <= 0:
                    raise RuntimeError(f"mfma_peak_probe failed ({n})")
                mfmas[0] = n

            t = time_calls([launch], 20, 5)  # about 50 ms timed, so the clock has settled
            res[f"{label}_{waves}wave_TFLOPs"] = round(mfmas[0] * 32768 * 20 / t / 1e12, 1)
    res["random_best_TFLOPs"] = max(res["random_1wave_TFLOPs"], res["random_2wave_TFLOPs"])
    del sink
    return res


def extra_small_gemv(steps, warmup):
    w = workloads.WORKLOADS["fp4_gemv_small"]
    p = w.make()
    d = fp4_on_device(p)
    out = torch.empty(1, w.N, dtype=torch.float16, device="cuda")
    t = time_rotating(lambda r: fw.fp4w_matmul(d["A"], d["B"][0], d["ws"][0], d["ws2"], None, 16, out=out),
                      1, steps)
    return {"us_per_call": round(t * 1e6, 3), "note": "75 KB working set, L2-resident"}


def extra_prefill_fp4(reps=200, warmup=50):
    w = workloads.WORKLOADS["fp4_prefill"]
    p = w.make()
    d = fp4_on_device(p)
    flops = 2.0 * p.M * p.N * p.K
    out = torch.empty(p.M, p.N, dtype=torch.bfloat16, device="cuda")
    t = time_calls([lambda: fw.fp4w_matmul(d["A"], d["B"][0], d["ws"][0], d["ws2"], None, 16, out=out)],
                   reps, warmup) / reps
    res = {"fused_ms": round(t * 1e3, 3), "fused_TFLOPs": round(flops / t / 1e12, 1),
           "fused_frac_of_bf16_peak": round(flops / t / 1e12 / BF16_PEAK_TFLOPS, 4)}
    # baseline: dequant to a [N, K] scratch, then hipBLASLt (torch.matmul)
    scratch = torch.empty(p.N, p.K, dtype=torch.bfloat16, device="cuda")

    def base():
        fw.fp4w_dequant(d["B"][0], d["ws"][0], d["ws2"], 16, out=scratch)
        torch.matmul(d["A"], scratch.t(), out=out)

    tb = time_calls([base], reps, warmup) / reps
    td = time_calls([lambda: fw.fp4w_dequant(d["B"][0], d["ws"][0], d["ws2"], 16, out=scratch)],
                    reps, warmup) / reps
    dq_bytes = p.B.nbytes + p.weight_scale.nbytes + scratch.numel() * 2
    res.update({"baseline_dequant_plus_hipblaslt_ms": round(tb * 1e3, 3),
                "baseline_TFLOPs": round(flops / tb / 1e12, 1),
                "fused_over_baseline_time": round(t / tb, 4), "dispatches": {"warmup": warmup, "timed": reps},
                "dequant_ms": round(td * 1e3, 4), "dequant_GBps": round(dq_bytes / td / 1e9, 1)})
    # The same calls on all-zero activations and weights: the shader clock
    # follows the chip's power draw, which depends on the operand bits, so a
    # shorter time here means the random-data time is power-limited.
    zA, zB = torch.zeros_like(d["A"]), torch.zeros_like(d["B"][0])
    tz = time_calls([lambda: fw.fp4w_matmul(zA, zB, d["ws"][0], d["ws2"], None, 16, out=out)], 50, 10) / 50

    def base_zero():
        fw.fp4w_dequant(zB, d["ws"][0], d["ws2"], 16, out=scratch)
        torch.matmul(zA, scratch.t(), out=out)

    tbz = time_calls([base_zero], 50, 10) / 50
    res["zero_operands"] = {"fused_ms": round(tz * 1e3, 3), "baseline_ms": round(tbz * 1e3, 3),
                            "dispatches": {"warmup": 10, "timed": 50}}
    del scratch, zA, zB
    return res


def extra_fp8(steps, warmup, reps=200, pre_warmup=50):
    w = workloads.WORKLOADS["fp8_gemv"]
    p = w.make(M=4)
    wb = p.B.nbytes + p.b_scale.nbytes
    R = copies_for(wb)
    d = fp8_on_device(p, copies=R)
    out = torch.empty(4, p.N, dtype=torch.bfloat16, device="cuda")
    t = time_rotating(lambda r: fw.fp8w_matmul(d["A"], d["B"][r], d["bs"][r], None, 128, out=out), R, steps)
    res = {"gemv_M4_us": round(t * 1e6, 2), "gemv_M4_weight_GBps": round(wb / t / 1e9, 1)}
    del d
    p8 = w.make(M=8192)
    d = fp8_on_device(p8)
    out = torch.empty(8192, p8.N, dtype=torch.bfloat16, device="cuda")
    flops = 2.0 * p8.M * p8.N * p8.K
    tp = time_calls([lambda: fw.fp8w_matmul(d["A"], d["B"][0], d["bs"][0], None, 128, out=out)],
                    reps, pre_warmup) / reps
    res.update({"prefill_ms": round(tp * 1e3, 3), "prefill_TFLOPs": round(flops / tp / 1e12, 1),
                "prefill_frac_of_bf16_peak": round(flops / tp / 1e12 / BF16_PEAK_TFLOPS, 4),
                "prefill_dispatches": {"warmup": pre_warmup, "timed": reps}})
    # the pages' default path: dequant to an [N, K] scratch, then hipBLASLt (torch.matmul)
    scratch = torch.empty(p8.N, p8.K, dtype=torch.bfloat16, device="cuda")

    def base():
        fw.fp8w_dequant(d["B"][0], d["bs"][0], 128, out=scratch)
        torch.matmul(d["A"], scratch.t(), out=out)

    tb = time_calls([base], reps, pre_warmup) / reps
    td = time_calls([lambda: fw.fp8w_dequant(d["B"][0], d["bs"][0], 128, out=scratch)], reps, pre_warmup) / reps
    dq_bytes = p8.B.nbytes + p8.b_scale.nbytes + scratch.numel() * 2
    res.update({"prefill_baseline_dequant_plus_hipblaslt_ms": round(tb * 1e3, 3),
                "prefill_baseline_TFLOPs": round(flops / tb / 1e12, 1),
                "prefill_over_baseline_time": round(tp / tb, 4),
                "dequant_ms": round(td * 1e3, 4), "dequant_GBps": round(dq_bytes / td / 1e9, 1)})
    # The same calls on all-zero activations and weights: the shader clock
    # follows the chip's power draw, which depends on the operand bits, so a
    # shorter time here means the random-data time is power-limited.
    zA, zB = torch.zeros_like(d["A"]), torch.zeros_like(d["B"][0])
    tz = time_calls([lambda: fw.fp8w_matmul(zA, zB, d["bs"][0], None, 128, out=out)], 50, 10) / 50

    def base_zero():
        fw.fp8w_dequant(zB, d["bs"][0], 128, out=scratch)
        torch.matmul(zA, scratch.t(), out=out)

    tbz = time_calls([base_zero], 50, 10) / 50
    res["prefill_zero_operands"] = {"fused_ms": round(tz * 1e3, 3), "baseline_ms": round(tbz * 1e3, 3),
                                    "dispatches": {"warmup": 10, "timed": 50}}
    del scratch, zA, zB
    return res


def extra_wide(steps, warmup):
    w = workloads.WORKLOADS["fp4_gemv_wide"]
    p = w.make()
    wb = p.B.nbytes + p.weight_scale.nbytes
    R = copies_for(wb)
    d = fp4_on_device(p, copies=R)
    out = torch.empty(4, p.N, dtype=torch.bfloat16, device="cuda")
    t = time_rotating(lambda r: fw.fp4w_matmul(d["A"], d["B"][r], d["ws"][r], d["ws2"], None, 16, out=out),
                      R, min(steps, 64))
    return {"us": round(t * 1e6, 2), "weight_GBps": round(wb / t / 1e9, 1), "copies": R}


def extra_skinny(steps, warmup):
    """8 < M <= 64 (batched decode / short prefill chunks): the skinny MFMA
    kernel, weights rotated past the last-level cache."""
    res = {}
    for N, K in ((4096, 4096), (17408, 5120)):
        for M in (16, 32, 64):
            p = workloads.make_fp4(M, N, K, 16, "bf16", seed=M)
            wb = p.B.nbytes + p.weight_scale.nbytes
            R = copies_for(wb)
            d = fp4_on_device(p, copies=R)
            out = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
            t = time_rotating(lambda r: fw.fp4w_matmul(d["A"], d["B"][r], d["ws"][r], d["ws2"], None, 16,
                                                       out=out), R, min(steps, 64))
            del d
            p8 = workloads.make_fp8(M, N, K, 128, "bf16", seed=M)
            wb8 = p8.B.nbytes + p8.b_scale.nbytes
            R8 = copies_for(wb8)
            d8 = fp8_on_device(p8, copies=R8)
            t8 = time_rotating(lambda r: fw.fp8w_matmul(d8["A"], d8["B"][r], d8["bs"][r], None, 128, out=out),
                               R8, min(steps, 64))
            del d8
            torch.cuda.empty_cache()
            res[f"M{M}_N{N}_K{K}"] = {"fp4_us": round(t * 1e6, 2), "fp4_weight_GBps": round(wb / t / 1e9, 1),
                                      "fp8_us": round(t8 * 1e6, 2), "fp8_weight_GBps": round(wb8 / t8 / 1e9, 1)}
    return res


def extra_w8a8(steps, warmup):
    """Optional W8A8 mode ([FP8 doc] §6): the activation QDQ kernel alone, and
    QDQ + FP8 matmul at the FP8 GEMV workload (M=4) and at the pages' W8A8
    profiling shape (bf16, M=16, N=K=4096, block 128).  a_scale = amax/448."""
    res = {}
    w = workloads.WORKLOADS["fp8_gemv"]
    for label, M, N, K in (("M4_N17408_K5120", 4, w.N, w.K), ("M16_N4096_K4096", 16, 4096, 4096)):
        p = workloads.make_fp8(M, N, K, 128, "bf16", seed=M + 5)
        wb = p.B.nbytes + p.b_scale.nbytes
        R = copies_for(wb)
        d = fp8_on_device(p, copies=R)
        a = d["A"].float().abs().max() / 448.0
        sc = a.reshape(1).to(torch.float32)
        work = torch.empty_like(d["A"])
        out = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        tq = time_rotating(lambda r: fw.fp8w_qdq_activation(d["A"], sc, out=work), 1, steps)
        tw = time_rotating(lambda r: fw.fp8w_matmul_w8a8(d["A"], d["B"][r], d["bs"][r], sc, None, 128,
                                                          out=out, workspace=work), R, steps)
        t0 = time_rotating(lambda r: fw.fp8w_matmul(d["A"], d["B"][r], d["bs"][r], None, 128, out=out),
                           R, steps)
        res[label] = {"qdq_us": round(tq * 1e6, 2), "w8a8_us": round(tw * 1e6, 2),
                      "weight_only_us": round(t0 * 1e6, 2), "weight_GBps_w8a8": round(wb / tw / 1e9, 1)}
        del d
    A = torch.randn(8192, 5120, device="cuda").to(torch.bfloat16)
    work = torch.empty_like(A)
    sc = (A.float().abs().max() / 448.0).reshape(1)
    tq = time_calls([lambda: fw.fp8w_qdq_activation(A, sc, out=work)], 50, 5) / 50
    res["qdq_M8192_K5120"] = {"us": round(tq * 1e6, 2), "GBps": round(4 * A.numel() / tq / 1e9, 1)}
    return res


def extra_w4a4(steps, warmup, reps=50):
    """W4A4 ([FP4 doc] §6): the NVFP4 activation kernels alone at the prefill
    activation shape (M = 8192, K = 5120), and the whole W4A4 matmul (QDQ
    into a workspace + the FP4 matmul) at the prefill workload and at the
    decode workload (M = 4)."""
    res = {}
    A = torch.randn(8192, 5120, device="cuda").to(torch.bfloat16)
    work = torch.empty_like(A)
    codes = torch.empty(8192, 2560, dtype=torch.uint8, device="cuda")
    scales = torch.empty(8192, 320, dtype=torch.uint8, device="cuda")
    tq = time_calls([lambda: fw.fp4w_qdq_activation(A, out=work)], reps, 5) / reps
    tp = time_calls([lambda: fw.fp4w_quantize_activation(A, codes, scales)], reps, 5) / reps
    n = A.numel()
    res["qdq_M8192_K5120"] = {"us": round(tq * 1e6, 2), "GBps": round(4 * n / tq / 1e9, 1)}
    res["quantize_M8192_K5120"] = {"us": round(tp * 1e6, 2), "GBps": round((2 * n + n / 2 + n / 16) / tp / 1e9, 1)}
    del A, work, codes, scales
    p = workloads.WORKLOADS["fp4_prefill"].make()
    d = fp4_on_device(p)
    work = torch.empty_like(d["A"])
    out = torch.empty(p.M, p.N, dtype=torch.bfloat16, device="cuda")
    flops = 2.0 * p.M * p.N * p.K
    tw = time_calls([lambda: fw.fp4w_matmul_w4a4(d["A"], d["B"][0], d["ws"][0], d["ws2"], None, 16, out=out,
                                                 workspace=work)], 20, 5) / 20
    res["prefill_ms"] = round(tw * 1e3, 3)
    res["prefill_TFLOPs"] = round(flops / tw / 1e12, 1)
    del d, work, out
    w = workloads.WORKLOADS["fp4_gemv_decode"]
    p4 = w.make(M=4)
    wb = p4.B.nbytes + p4.weight_scale.nbytes
    R = copies_for(wb)
    d = fp4_on_device(p4, copies=R)
    work = torch.empty_like(d["A"])
    out = torch.empty(4, w.N, dtype=torch.bfloat16, device="cuda")
    t4 = time_rotating(lambda r: fw.fp4w_matmul_w4a4(d["A"], d["B"][r], d["ws"][r], d["ws2"], d["bias"], 16,
                                                      out=out, workspace=work), R, steps)
    res["decode_M4_N5120_K5120_us"] = round(t4 * 1e6, 2)
    return res


def extra_mid_m(steps, warmup):
    """FP4 matmul through the default dispatch at prompt-chunk sizes M = 64 ..
    1024 (N = 17408, K = 5120): where the skinny kernel hands over to the
    prefill GEMM, whose 256 x 256 tiles give these sizes few workgroups (a
    last round of at most half the CUs' worth of tiles is split over two
    workgroups per tile)."""
    N, K = 17408, 5120
    B, ws = workloads.fp4_weights_on_device(N, K, 16, seed=11)
    ws2 = torch.tensor([2.0 ** -8], dtype=torch.float32, device="cuda")
    res = {}
    for M in (64, 65, 128, 256, 512, 1024):
        A = dev_bits(workloads.activations(np.random.default_rng(M), M, K, "bf16", "normal"), "bf16")
        out = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        path = fw.fp4w_path_name(fw.fp4w_select_path(fw.OP_FP4_MATMUL, M, N, K, 16, K // 16))
        n = max(4, min(steps, 20))
        t = time_calls([lambda: fw.fp4w_matmul(A, B, ws, ws2, None, 16, out=out)], n, 2) / n
        res[f"M{M}"] = {"path": path, "us": round(t * 1e6, 1), "TFLOPs": round(2 * M * N * K / t / 1e12, 1)}
    del B, ws
    return res


def decode_step_setup():
    """Device inputs of the decode-step sequence: one weight set per launch,
    one activation per K, one output per shape (FP16, M = 4, no bias)."""
    M = workloads.DECODE_STEP_M
    shapes = workloads.DECODE_STEP_SHAPES
    ws2 = torch.tensor([2.0 ** -8], dtype=torch.float32, device="cuda")
    W = [workloads.fp4_weights_on_device(N, K, 16, seed=7000 + i) for i, (N, K) in enumerate(shapes)]
    A = {}
    for K in sorted({K for _, K in shapes}):
        A[K] = dev_bits(workloads.activations(np.random.default_rng(K), M, K, "fp16", "uniform"), "fp16")
    out = {s: torch.empty(M, s[0], dtype=torch.float16, device="cuda") for s in set(shapes)}

    def step():
        for (N, K), (B, ws) in zip(shapes, W):
            fw.fp4w_matmul(A[K], B, ws, ws2, None, 16, out=out[(N, K)])

    return dict(M=M, shapes=shapes, W=W, A=A, out=out, ws2=ws2, step=step)


def extra_decode_step(steps, warmup):
    """A decode step as 121 back-to-back FP4 GEMV launches (M = 4, FP16): the
    step replayed from one HIP graph, the same launches issued one by one from
    Python, and the sum of the launches timed in isolation (graphs of one
    shape), whose difference to the graph step is the cost of the sequence."""
    st = decode_step_setup()
    shapes, W = st["shapes"], st["W"]
    wbytes = sum(B.numel() + ws.numel() for B, ws in W)
    g = capture(st["step"])
    n = max(4, min(steps, 40))
    _, tg = time_graphs([g], n, max(2, min(warmup, 5)))
    tg /= n
    te = time_calls([st["step"]], max(2, n // 4), 2) / max(2, n // 4)
    del g
    iso = 0.0
    per_shape = {}
    for shp in sorted(set(shapes)):
        idx = [i for i, s in enumerate(shapes) if s == shp]
        N, K = shp
        t = time_rotating(lambda r: fw.fp4w_matmul(st["A"][K], W[idx[r]][0], W[idx[r]][1], st["ws2"], None, 16,
                                                   out=st["out"][shp]), len(idx), 4 * len(idx))
        per_shape[f"N{N}_K{K}"] = {"launches": len(idx), "us": round(t * 1e6, 2)}
        iso += t * len(idx)
    return {"launches": len(shapes), "M": st["M"], "weight_MB_per_step": round(wbytes / 1e6, 1),
            "graph_ms": round(tg * 1e3, 4), "eager_ms": round(te * 1e3, 4),
            "isolated_sum_ms": round(iso * 1e3, 4),
            "weight_GBps_graph": round(wbytes / tg / 1e9, 1),
            "gap_us_per_launch": round((tg - iso) / len(shapes) * 1e6, 3), "per_shape": per_shape}


# ------------------------------------------------------------------ profiling mode

def profile_kernel(which, launches=50):
    """Launch one kernel `launches` times without graphs, for rocprofv3 runs
    (kernel trace or PMC counters).  Weight copies rotate as in the timed runs."""
    if which == "copy":
        n = 256 << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(launches):
            dst.copy_(src)
    elif which == "fp4_gemv":
        # the headline step: M = 1, 2, 4, 8 on rotating weight copies
        w = workloads.WORKLOADS["fp4_gemv_decode"]
        probs = {M: w.make(M=M) for M in w.Ms}
        p0 = probs[w.Ms[0]]
        R = copies_for(p0.B.nbytes + p0.weight_scale.nbytes)
        d = fp4_on_device(p0, copies=R)
        A = {M: dev_bits(probs[M].A, "bf16") for M in w.Ms}
        out = {M: torch.empty(M, w.N, dtype=torch.bfloat16, device="cuda") for M in w.Ms}
        for i in range(launches):
            for M in w.Ms:
                fw.fp4w_matmul(A[M], d["B"][i % R], d["ws"][i % R], d["ws2"], d["bias"], 16, out=out[M])
    elif which == "fp4_gemv_wide":
        w = workloads.WORKLOADS["fp4_gemv_wide"]
        p = w.make(M=4)
        R = copies_for(p.B.nbytes + p.weight_scale.nbytes)
        d = fp4_on_device(p, copies=R)
        out = torch.empty(p.M, w.N, dtype=torch.bfloat16, device="cuda")
        for i in range(launches):
            fw.fp4w_matmul(d["A"], d["B"][i % R], d["ws"][i % R], d["ws2"], d["bias"], 16, out=out)
    elif which == "fp8_gemv":
        p = workloads.WORKLOADS["fp8_gemv"].make(M=4)
        R = copies_for(p.B.nbytes + p.b_scale.nbytes)
        d = fp8_on_device(p, copies=R)
        out = torch.empty(4, p.N, dtype=torch.bfloat16, device="cuda")
        for i in range(launches):
            fw.fp8w_matmul(d["A"], d["B"][i % R], d["bs"][i % R], None, 128, out=out)
    elif which == "fp4_gemm":
        p = workloads.WORKLOADS["fp4_prefill"].make()
        d = fp4_on_device(p)
        out = torch.empty(p.M, p.N, dtype=torch.bfloat16, device="cuda")
        for _ in range(min(launches, 10)):
            fw.fp4w_matmul(d["A"], d["B"][0], d["ws"][0], d["ws2"], None, 16, out=out)
    elif which == "fp8_gemm":
        p = workloads.WORKLOADS["fp8_gemv"].make(M=8192)
        d = fp8_on_device(p)
        out = torch.empty(p.M, p.N, dtype=torch.bfloat16, device="cuda")
        for _ in range(min(launches, 10)):
            fw.fp8w_matmul(d["A"], d["B"][0], d["bs"][0], None, 128, out=out)
    elif which == "w4a4":
        # the W4A4 prefill: NVFP4 activation QDQ + the FP4 GEMM
        p = workloads.WORKLOADS["fp4_prefill"].make()
        d = fp4_on_device(p)
        work = torch.empty_like(d["A"])
        out = torch.empty(p.M, p.N, dtype=torch.bfloat16, device="cuda")
        for _ in range(min(launches, 10)):
            fw.fp4w_matmul_w4a4(d["A"], d["B"][0], d["ws"][0], d["ws2"], None, 16, out=out, workspace=work)
    elif which == "skinny":
        # batched decode, M = 16, 32, 64 at N = 17408, K = 5120 (FP4 then FP8)
        for M in (16, 32, 64):
            p = workloads.make_fp4(M, 17408, 5120, 16, "bf16", seed=M)
            R = copies_for(p.B.nbytes + p.weight_scale.nbytes)
            d = fp4_on_device(p, copies=R)
            out = torch.empty(M, p.N, dtype=torch.bfloat16, device="cuda")
            for i in range(launches):
                fw.fp4w_matmul(d["A"], d["B"][i % R], d["ws"][i % R], d["ws2"], None, 16, out=out)
            del d
            p8 = workloads.make_fp8(M, 17408, 5120, 128, "bf16", seed=M)
            R8 = copies_for(p8.B.nbytes + p8.b_scale.nbytes)
            d8 = fp8_on_device(p8, copies=R8)
            for i in range(launches):
                fw.fp8w_matmul(d8["A"], d8["B"][i % R8], d8["bs"][i % R8], None, 128, out=out)
            del d8
    elif which == "qdq":
        A = torch.randn(8192, 5120, device="cuda").to(torch.bfloat16)
        work = torch.empty_like(A)
        sc = (A.float().abs().max() / 448.0).reshape(1)
        for _ in range(launches):
            fw.fp8w_qdq_activation(A, sc, out=work)
    elif which == "fp8_dequant":
        p = workloads.WORKLOADS["fp8_gemv"].make(M=1)
        d = fp8_on_device(p)
        out = torch.empty(p.N, p.K, dtype=torch.bfloat16, device="cuda")
        for _ in range(launches):
            fw.fp8w_dequant(d["B"][0], d["bs"][0], 128, out=out)
    elif which == "decode_step":
        # the decode-step sequence, replayed from its graph
        st = decode_step_setup()
        g = capture(st["step"])
        for _ in range(max(1, launches // 5)):
            g.replay()
        torch.cuda.synchronize()
        del g
    elif which == "dequant":
        p = workloads.WORKLOADS["fp4_prefill"].make(M=1)
        d = fp4_on_device(p)
        out = torch.empty(p.N, p.K, dtype=torch.bfloat16, device="cuda")
        for _ in range(launches):
            fw.fp4w_dequant(d["B"][0], d["ws"][0], d["ws2"], 16, out=out)
    torch.cuda.synchronize()
    log(f"profiled {launches} launches of {which}")


# ------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--extra", default="", help="comma-separated subset of the extra workloads to run")
    ap.add_argument("--profile-kernel", choices=["fp4_gemv", "fp4_gemv_wide", "fp8_gemv", "fp4_gemm", "fp8_gemm", "w4a4",
                                                 "dequant", "copy", "decode_step", "skinny", "qdq", "fp8_dequant"])
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library runs on a single MI355X and has no "
              "multi-GPU path (--gpus must be 1).", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    fw.load_library()
    if args.profile_kernel:
        profile_kernel(args.profile_kernel)
        return

    torch.cuda.synchronize()
    h = gemv_decode(args.steps, args.warmup)
    log(f"headline: {h['per_step'] * 1e6:.2f} us/step")
    w = h["workload"]
    value = len(h["Ms"]) * h["weight_bytes"] / h["per_step"] / 1e9
    launches_per_step = len(h["Ms"])
    mean_launch = h["per_step"] / launches_per_step
    alg_per_launch = h["alg_bytes_step"] / launches_per_step
    achieved = alg_per_launch / mean_launch / 1e9
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("source_hash") == source_hash(GEMV_SOURCES):
            traffic = tr.get("bytes_per_launch")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "kernel": "fp4_gemv_kernel (MFMA decode GEMV)",
                "alg_bytes_per_launch": round(alg_per_launch), "mean_launch_us": round(mean_launch * 1e6, 3)}

    extra = {"per_M": h["per_m"], "weight_copies": h["R"], "per_replay": h["per_replay"]}
    w8, ww = workloads.WORKLOADS["fp8_gemv"], workloads.WORKLOADS["fp4_gemv_wide"]
    rd = hbm_read({"fp4_gemv_decode": h["weight_bytes"],
                   "fp8_gemv": w8.N * w8.K + w8.N * (w8.K // w8.block_size) * 4,
                   "fp4_gemv_wide": ww.N * ww.K // 2 + ww.N * (ww.K // 16)})
    rd["headline_frac_of_peak"] = round(value / rd["peak_GBps"], 4)
    rd["headline_frac_at_size"] = round(value / rd["at_size"]["fp4_gemv_decode"]["GBps"], 4)
    extra["hbm_read"] = rd
    torch.cuda.empty_cache()
    log(f"hbm_read: {rd}")
    if not args.no_extra:
        for name, fn in (("hbm_copy_GBps", hbm_copy_gbps),
                         ("fp4_gemv_small", lambda: extra_small_gemv(args.steps, args.warmup)),
                         ("fp4_gemv_wide", lambda: extra_wide(args.steps, args.warmup)),
                         ("fp8", lambda: extra_fp8(args.steps, args.warmup)),
                         ("fp8_w8a8", lambda: extra_w8a8(args.steps, args.warmup)),
                         ("fp4_w4a4", lambda: extra_w4a4(args.steps, args.warmup)),
                         ("skinny", lambda: extra_skinny(args.steps, args.warmup)),
                         ("decode_step", lambda: extra_decode_step(args.steps, args.warmup)),
                         ("mid_m", lambda: extra_mid_m(args.steps, args.warmup)),
                         ("mfma_peak", mfma_peak),
                         ("fp4_prefill", extra_prefill_fp4)):
            if args.extra and name not in args.extra.split(","):
                continue
            t0 = time.perf_counter()
            extra[name] = fn()
            torch.cuda.empty_cache()
            log(f"{name}: {extra[name]} ({time.perf_counter() - t0:.1f} s)")

    # the bandwidth-bound GEMV extras against the measured read peak
    peak_rd = rd["peak_GBps"]
    if "fp4_gemv_wide" in extra:
        gb = extra["fp4_gemv_wide"]["weight_GBps"]
        extra["fp4_gemv_wide"]["frac_of_measured_read_peak"] = round(gb / peak_rd, 4)
        extra["fp4_gemv_wide"]["frac_of_read_at_size"] = round(gb / rd["at_size"]["fp4_gemv_wide"]["GBps"], 4)
    # the prefill GEMMs against the MFMA rate measured on random operands
    if "mfma_peak" in extra:
        mp = extra["mfma_peak"]["random_best_TFLOPs"]
        if "fp4_prefill" in extra:
            extra["fp4_prefill"]["fused_frac_of_mfma_probe_random"] = round(extra["fp4_prefill"]["fused_TFLOPs"] / mp, 4)
            extra["fp4_prefill"]["baseline_frac_of_mfma_probe_random"] = round(
                extra["fp4_prefill"]["baseline_TFLOPs"] / mp, 4)
        if "fp8" in extra:
            extra["fp8"]["prefill_frac_of_mfma_probe_random"] = round(extra["fp8"]["prefill_TFLOPs"] / mp, 4)
    if "fp8" in extra:
        gb = extra["fp8"]["gemv_M4_weight_GBps"]
        extra["fp8"]["gemv_M4_frac_of_measured_read_peak"] = round(gb / peak_rd, 4)
        extra["fp8"]["gemv_M4_frac_of_read_at_size"] = round(gb / rd["at_size"]["fp8_gemv"]["GBps"], 4)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline()
        log(f"cpu baseline: {cpu}")

    line = {
        "metric": "FP4 GEMV weight GB/s (M=1..8) & prefill TFLOP/s, % of HBM/MFMA peak",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(h["per_step"] * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; shapes and distributions of the workload)",
        "config": {"workload": "fp4_gemv_decode", "M": list(h["Ms"]), "N": w.N, "K": w.K,
                   "block_size": 16, "activation": "bf16", "bias": True, "weight_copies": h["R"],
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
