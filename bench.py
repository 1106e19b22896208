#!/usr/bin/env python3
"""Benchmark of the block-quantized matmul hot path on one MI355X.

Headline workload (one "step"): the batch-1 decode GEMVs of a Qwen-4B-like
MLP -- Q4_K weights [9728, 2560] and Q6_K weights [2560, 9728], each with its
fp32 activation quantized to Q8_K inside the GEMV (fused quantizer), seeded
synthetic data.  value = algorithmic bytes of the step (compressed weights,
fp32 x and y) / time, in GB/s, with the weights rotated through more buffer
sets than the 256 MB Infinity Cache holds, so every step streams from HBM.

Timing: each timed quantity is a HIP graph of calls over weight copies
rotated past the Infinity Cache (cold), replayed several times, each replay
timed with HIP events; the figure is the median over replays of the per-call
time.

The same line carries:
  roofline     -- the dominant kernel (the Q6_K GEMV) against 8 TB/s HBM,
                  achieved from its median cold launch duration (the mean
                  beside it), and its streaming floor: the same weight bytes
                  in the same launch shape with no compute (vq_stream_probe);
  cpu_baseline -- the CPU oracle running the same decode step on the host's
                  cores (a bounded number of repetitions);
  prefill / q8_0 / grouped / quantizer -- the prefill GEMM (int8 TOPS; also
                  end to end with its activation quantizer), the Q8_0 x Q8_1
                  GEMM and GEMV, the routed-expert grouped GEMM with the
                  weighted expert sum (broadcast arm, and the per-row arm at
                  the down-projection shape), and the standalone quantizer,
                  timed with HIP events in the same run (secondary numbers);
  ceilings     -- measured references beside the spec peaks: the int8 MFMA
                  rate of vq_mfma_probe, a 1 GiB device-to-device copy and a
                  570 MB read-only stream.

Usage: python bench.py [--gpus 1] [--steps 200] [--warmup 20]
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
sys.path.insert(0, ROOT)

METRIC = "decode GEMV GB/s + prefill GEMM int8 TOPS (% of MI355X roofline)"
HBM_PEAK_GBS = 8000.0
INT8_PEAK_TOPS = 5000.0
MALL_BYTES = 256 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


GEMV_SOURCES = ["block_quantized_matmul_fp32_amd/csrc/gemv.hip",
                "block_quantized_matmul_fp32_amd/csrc/vq_device.h"]


def traffic_from_profiles(kernel_key: str, sha: str, launches_bytes: float):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, or None if
    the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    ent = data.get(kernel_key)
    if not ent or ent.get("source_sha") != sha:
        return None
    return ent.get("traffic_bytes_per_launch")


def event_pair():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def time_launches(fn, iters, warmup=3):
    """Average per-launch duration (ms) from HIP events around each launch
    (eager launches; only for kernels much longer than a launch's host cost)."""
    import torch
    for _ in range(warmup):
        fn(0)
    torch.cuda.synchronize()
    pairs = [event_pair() for _ in range(iters)]
    for i in range(iters):
        pairs[i][0].record()
        fn(i)
        pairs[i][1].record()
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in pairs) / iters


def time_graph(fn, per_graph, min_calls, warmup=2, stats=None):
    """Duration (ms) of one call of fn: a HIP graph holds `per_graph`
    back-to-back calls fn(0..per_graph-1) (one per rotation set, so each call
    is cold when the sets outgrow the Infinity Cache); each replay is timed on
    its own with HIP events recorded on the stream the graph replays on, and
    the result is the median over replays of the per-call time.  A host launch
    costs several microseconds, more than the decode kernels run, so eager
    back-to-back launches would time the host; the graph times the GPU.
    Returns (median ms, calls timed); `stats`, if given, receives the mean and
    the spread."""
    import torch
    for i in range(max(warmup, 1)):
        fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            for i in range(per_graph):
                fn(i)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    reps = max(3, math.ceil(min_calls / per_graph))
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    pairs = [event_pair() for _ in range(reps)]
    for a, b in pairs:
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) / per_graph for a, b in pairs)
    med = per[len(per) // 2] if len(per) % 2 else 0.5 * (per[len(per) // 2 - 1] + per[len(per) // 2])
    if stats is not None:
        stats["mean_ms"] = sum(per) / len(per)
        stats["min_ms"] = per[0]
        stats["max_ms"] = per[-1]
        stats["replays"] = reps
    return med, reps * per_graph


def cpu_threads():
    """(threads used, cores in the affinity mask, why): every affinity core,
    unless the environment sets the host's CPU share per GPU in
    OMP_NUM_THREADS, which then caps it."""
    cores = len(os.sched_getaffinity(0))
    share = os.environ.get("OMP_NUM_THREADS", "")
    if share.isdigit() and 0 < int(share) < cores:
        return int(share), cores, "OMP_NUM_THREADS=%s: the host's CPU share for this GPU" % share
    return cores, cores, "every core in the affinity mask"


def run_cpu_fp64_reference(reps_max: int = 20, seconds: float = 5.0):
    """The fp64 dequantize-then-matmul reference (numpy) on the decode step,
    with its BLAS library's own thread count."""
    import numpy as np
    import oracle
    from oracle import ref_fp64
    import synth
    try:
        from threadpoolctl import threadpool_info
        info = [d for d in threadpool_info() if d.get("user_api") == "blas"]
    except Exception:  # threadpoolctl missing: the count stays unknown
        info = []
    blas = {"library": info[0].get("internal_api"), "threads": info[0].get("num_threads")} if info else None
    Qa = oracle.quantize_weights(oracle.Q4_K, synth.tensor("decode_gemv", "Wa"))
    Qb = oracle.quantize_weights(oracle.Q6_K, synth.tensor("decode_gemv", "Wb"))
    aa = oracle.quantize_q8k(synth.tensor("decode_gemv", "xa"))
    ab = oracle.quantize_q8k(synth.tensor("decode_gemv", "xb"))
    reps = 0
    t0 = time.perf_counter()
    while True:
        ref_fp64.gemm_fp64(oracle.Q4_K, Qa, 9728, 2560, aa)
        ref_fp64.gemm_fp64(oracle.Q6_K, Qb, 2560, 9728, ab)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= reps_max:
            break
    return {"ms_per_step": round(1e3 * el / reps, 2), "repetitions": reps, "blas": blas,
            "what": "numpy fp64 dequantize-then-matmul of the decode step (both GEMVs)"}


def run_cpu_baseline(seconds: float):
    """The CPU oracle on the same decode step (both GEMVs and their Q8_K
    quantization), repeated until about `seconds` of work; GB/s on the same
    algorithmic byte count as the GPU step."""
    import numpy as np
    import oracle
    import synth
    threads, cores, why = cpu_threads()
    Wa = synth.tensor("decode_gemv", "Wa")
    Wb = synth.tensor("decode_gemv", "Wb")
    xa = synth.tensor("decode_gemv", "xa")
    xb = synth.tensor("decode_gemv", "xb")
    Qa = oracle.quantize_weights(oracle.Q4_K, Wa)
    Qb = oracle.quantize_weights(oracle.Q6_K, Wb)
    del Wa, Wb
    step_bytes = decode_step_bytes()
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.gemm(oracle.Q4_K, Qa, 9728, 2560, oracle.quantize_q8k(xa), nthreads=threads)
        oracle.gemm(oracle.Q6_K, Qb, 2560, 9728, oracle.quantize_q8k(xb), nthreads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 100000:
            break
    step_ops = 2.0 * (9728 * 2560 + 2560 * 9728)
    return {"value": round(step_bytes * reps / el / 1e9, 4), "unit": "GB/s", "cores": threads,
            "gops": round(step_ops * reps / el / 1e9, 3),
            "affinity_cores": cores, "threads_reason": why,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": "%d repetitions of the full decode step (Q8_K quantization of x plus the Q4_K "
                      "[9728,2560] and Q6_K [2560,9728] GEMVs) in %.1f s with %d threads" % (reps, el, threads),
            "ms_per_step": round(1e3 * el / reps, 3)}


def cpu_model() -> str:
    """The host CPU's model name with its family / model / stepping and clock
    (first processor of /proc/cpuinfo; a virtualised host may show a short
    name), or "unknown"."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if not line.strip():
                    break
                k, _, v = line.partition(":")
                fields[k.strip()] = v.strip()
    except OSError:
        pass
    name = fields.get("model name")
    if not name:
        return "unknown"
    ids = ["%s %s" % (k, fields[k]) for k in ("cpu family", "model", "stepping") if k in fields]
    if "cpu MHz" in fields:
        ids.append("%s MHz" % fields["cpu MHz"].split(".")[0])
    return "%s (%s)" % (name, ", ".join(ids)) if ids else name


def decode_step_bytes():
    qa = 9728 * (2560 // 256) * 144
    qb = 2560 * (9728 // 256) * 210
    return qa + 4 * 2560 + 4 * 9728 + qb + 4 * 9728 + 4 * 2560


def run_decode(args, torch, vq, synth):
    dev = torch.device("cuda:0")
    Wa = torch.from_numpy(synth.tensor("decode_gemv", "Wa")).to(dev)
    Wb = torch.from_numpy(synth.tensor("decode_gemv", "Wb")).to(dev)
    Qa0 = vq.quantize_weights(vq.Q4_K, Wa)
    Qb0 = vq.quantize_weights(vq.Q6_K, Wb)
    del Wa, Wb
    xa = torch.from_numpy(synth.tensor("decode_gemv", "xa")).to(dev)
    xb = torch.from_numpy(synth.tensor("decode_gemv", "xb")).to(dev)
    set_bytes = Qa0.numel() + Qb0.numel()
    R = max(2, math.ceil(args.rotate_mb * (1 << 20) / set_bytes))
    Qa = [Qa0] + [Qa0.clone() for _ in range(R - 1)]
    Qb = [Qb0] + [Qb0.clone() for _ in range(R - 1)]
    ya = [torch.empty(9728, dtype=torch.float32, device=dev) for _ in range(R)]
    yb = [torch.empty(2560, dtype=torch.float32, device=dev) for _ in range(R)]
    def step(i):
        s = i % R
        vq.gemv(vq.Q4_K, Qa[s], 9728, 2560, xa, y=ya[s])
        vq.gemv(vq.Q6_K, Qb[s], 2560, 9728, xb, y=yb[s])

    # The timed steps replay a HIP graph holding one step per rotation set.
    ms, steps_timed = time_graph(step, R, args.steps, warmup=max(2, args.warmup // R))
    # Per-kernel average launch duration: the same, with one kernel per node.
    ka, _ = time_graph(lambda i: vq.gemv(vq.Q4_K, Qa[i % R], 9728, 2560, xa, y=ya[i % R]), R, args.steps)
    kb_stats = {}
    kb, _ = time_graph(lambda i: vq.gemv(vq.Q6_K, Qb[i % R], 2560, 9728, xb, y=yb[i % R]), R, args.steps,
                       stats=kb_stats)
    assert torch.isfinite(ya[0]).all() and torch.isfinite(yb[0]).all()
    # the streaming floor of each GEMV launch: its weight bytes, its launch
    # shape, the same rotation, no compute
    sink = torch.zeros(9728, dtype=torch.int32, device=dev)
    fa, _ = time_graph(lambda i: vq.stream_probe(vq.Q4_K, Qa[i % R], 9728, 2560, sink), R, args.steps)
    fb, _ = time_graph(lambda i: vq.stream_probe(vq.Q6_K, Qb[i % R], 2560, 9728, sink), R, args.steps)
    assert int(sink.abs().sum()) == 0
    return {"ms_per_step": ms, "q4k_ms": ka, "q6k_ms": kb, "q6k_mean_ms": kb_stats["mean_ms"],
            "q4k_floor_ms": fa, "q6k_floor_ms": fb,
            "rotation_sets": R, "steps_timed": steps_timed, "rotation_mb": round(R * set_bytes / (1 << 20), 1)}


def run_prefill(torch, vq, synth, iters):
    dev = torch.device("cuda:0")
    out = {}
    Wg = torch.from_numpy(synth.tensor("prefill_gemm", "Wgate")).to(dev)
    Wd = torch.from_numpy(synth.tensor("prefill_gemm", "Wdown")).to(dev)
    Qg0 = vq.quantize_weights(vq.Q4_K, Wg)
    Qd0 = vq.quantize_weights(vq.Q6_K, Wd)
    del Wg, Wd
    # weight copies rotated past the Infinity Cache: every call reads its
    # weights from HBM
    Rg = max(2, math.ceil(640 * (1 << 20) / Qg0.numel()))
    Rd = max(2, math.ceil(640 * (1 << 20) / Qd0.numel()))
    Qg = [Qg0] + [Qg0.clone() for _ in range(Rg - 1)]
    Qd = [Qd0] + [Qd0.clone() for _ in range(Rd - 1)]
    out["rotation_sets"] = {"q4k": Rg, "q6k": Rd}
    for M in (512, 2048):
        Xh = torch.from_numpy(synth.prefill_activations("Xh", M)).to(dev)
        Xi = torch.from_numpy(synth.prefill_activations("Xi", M)).to(dev)
        qh = vq.quantize_act(vq.Q8_K, Xh)
        qi = vq.quantize_act(vq.Q8_K, Xi)
        Yg = torch.empty((M, 9728), dtype=torch.float32, device=dev)
        Yd = torch.empty((M, 2560), dtype=torch.float32, device=dev)
        tg, _ = time_graph(lambda i: vq.gemm(vq.Q4_K, Qg[i % Rg], 9728, 2560, vq.Q8_K, qh, M, Y=Yg), Rg, 3 * Rg)
        td, _ = time_graph(lambda i: vq.gemm(vq.Q6_K, Qd[i % Rd], 2560, 9728, vq.Q8_K, qi, M, Y=Yd), Rd, 3 * Rd)
        tq, _ = time_graph(lambda i: vq.quantize_act(vq.Q8_K, Xh, Xq=qh), 8, iters)
        # end to end: the quantizer of the fp32 activations, then the GEMM
        tgq, _ = time_graph(lambda i: (vq.quantize_act(vq.Q8_K, Xh, Xq=qh),
                                       vq.gemm(vq.Q4_K, Qg[i % Rg], 9728, 2560, vq.Q8_K, qh, M, Y=Yg)), Rg, 3 * Rg)
        tdq, _ = time_graph(lambda i: (vq.quantize_act(vq.Q8_K, Xi, Xq=qi),
                                       vq.gemm(vq.Q6_K, Qd[i % Rd], 2560, 9728, vq.Q8_K, qi, M, Y=Yd)), Rd, 3 * Rd)
        ops = 2.0 * M * 9728 * 2560
        out["M%d" % M] = {
            "q4k_gate_us": round(tg * 1e3, 2), "q4k_tops": round(ops / (tg * 1e-3) / 1e12, 1),
            "q4k_frac": round(ops / (tg * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
            "q6k_down_us": round(td * 1e3, 2), "q6k_tops": round(ops / (td * 1e-3) / 1e12, 1),
            "q6k_frac": round(ops / (td * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
            "q4k_quant_gemm_us": round(tgq * 1e3, 2), "q6k_quant_gemm_us": round(tdq * 1e3, 2),
            "quantize_q8k_us": round(tq * 1e3, 2),
            "quantize_q8k_gbs": round(M * 2560 * (4 + 1 + 4 / 256 + 2 / 16) / (tq * 1e-3) / 1e9, 1),
        }
    return out


def run_q8_0(torch, vq, synth, iters):
    dev = torch.device("cuda:0")
    W = torch.from_numpy(synth.tensor("q8_0_gemm", "W")).to(dev)
    Q = vq.quantize_weights(vq.Q8_0, W)
    del W
    X = torch.from_numpy(synth.tensor("q8_0_gemm", "X")).to(dev)
    Xq = vq.quantize_act(vq.Q8_1, X)
    Y = torch.empty((2048, 4096), dtype=torch.float32, device=dev)
    R = max(2, math.ceil(640 * (1 << 20) / Q.numel()))
    Qs = [Q] + [Q.clone() for _ in range(R - 1)]
    t, _ = time_graph(lambda i: vq.gemm(vq.Q8_0, Qs[i % R], 4096, 2048, vq.Q8_1, Xq, 2048, Y=Y), R, 3 * R)
    tq, _ = time_graph(lambda i: vq.quantize_act(vq.Q8_1, X, Xq=Xq), 8, iters)
    y = torch.empty(4096, dtype=torch.float32, device=dev)
    tv, _ = time_graph(lambda i: vq.gemv(vq.Q8_0, Qs[i % R], 4096, 2048, X[0], y=y), R, 200)
    sink = torch.zeros(4096, dtype=torch.int32, device=dev)
    tf, _ = time_graph(lambda i: vq.stream_probe(vq.Q8_0, Qs[i % R], 4096, 2048, sink), R, 200)
    ops = 2.0 * 2048 * 4096 * 2048
    gbytes = Q.numel() + 4 * 2048 + 4 * 4096
    return {"gemm_M2048_us": round(t * 1e3, 2), "gemm_tops": round(ops / (t * 1e-3) / 1e12, 1),
            "gemm_frac": round(ops / (t * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
            "gemv_us": round(tv * 1e3, 2), "gemv_gbs": round(gbytes / (tv * 1e-3) / 1e9, 1),
            "gemv_frac": round(gbytes / (tv * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "gemv_stream_floor_us": round(tf * 1e3, 2),
            "quantize_q8_1_us": round(tq * 1e3, 2),
            "quantize_q8_1_gbs": round(2048 * 2048 * (4 + 1 + 4 / 32) / (tq * 1e-3) / 1e9, 1)}


def run_q5k(torch, vq, synth, iters):
    """Q5_K [8192,2560]: the decode GEMV (fused quantizer, weights rotated past
    the Infinity Cache) and the GEMM at M = 2048."""
    dev = torch.device("cuda:0")
    W = torch.from_numpy(synth.tensor("q5k_decode", "W")).to(dev)
    N, K = W.shape
    Q = vq.quantize_weights(vq.Q5_K, W)
    del W
    R = max(2, math.ceil(640 * (1 << 20) / Q.numel()))
    Qs = [Q] + [Q.clone() for _ in range(R - 1)]
    x = torch.from_numpy(synth.tensor("q5k_decode", "x")).to(dev)
    y = torch.empty(N, dtype=torch.float32, device=dev)
    tv, _ = time_graph(lambda i: vq.gemv(vq.Q5_K, Qs[i % R], N, K, x, y=y), R, max(200, 4 * R))
    sink = torch.zeros(N, dtype=torch.int32, device=dev)
    tf, _ = time_graph(lambda i: vq.stream_probe(vq.Q5_K, Qs[i % R], N, K, sink), R, max(200, 4 * R))
    gbytes = Q.numel() + 4 * K + 4 * N
    Y = torch.empty((2048, N), dtype=torch.float32, device=dev)
    X = torch.from_numpy(synth.prefill_activations("Xh", 2048)).to(dev)
    Xq = vq.quantize_act(vq.Q8_K, X)
    tg, _ = time_graph(lambda i: vq.gemm(vq.Q5_K, Qs[i % R], N, K, vq.Q8_K, Xq, 2048, Y=Y), R, 3 * R)
    del Qs
    ops = 2.0 * 2048 * N * K
    return {"gemv_us": round(tv * 1e3, 2), "gemv_gbs": round(gbytes / (tv * 1e-3) / 1e9, 1),
            "gemv_frac": round(gbytes / (tv * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "gemv_stream_floor_us": round(tf * 1e3, 2),
            "gemm_M2048_us": round(tg * 1e3, 2), "gemm_tops": round(ops / (tg * 1e-3) / 1e12, 1),
            "gemm_frac": round(ops / (tg * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4)}


def run_small_batch(torch, vq, synth, iters):
    """vq_gemm at M = 2, 4, 8, 16, 32 on the decode matrices with the default
    crossover ("arm": the GEMV kernel up to the crossover, the MFMA GEMM with
    its split K above), weights rotated past the Infinity Cache; rate = weight
    bytes + activation bytes + output bytes per call."""
    dev = torch.device("cuda:0")
    out = {}
    for name, wt, wn, xn in (("q4k", vq.Q4_K, "Wa", "Xh"), ("q6k", vq.Q6_K, "Wb", "Xi")):
        W = torch.from_numpy(synth.tensor("decode_gemv", wn)).to(dev)
        N, K = W.shape
        Q = vq.quantize_weights(wt, W)
        del W
        R = max(2, math.ceil(640 * (1 << 20) / Q.numel()))
        Qs = [Q] + [Q.clone() for _ in range(R - 1)]
        X = torch.from_numpy(synth.prefill_activations(xn, 32)).to(dev)
        for M in (2, 4, 8, 16, 32):
            Xq = vq.quantize_act(vq.Q8_K, X[:M].contiguous())
            Y = torch.empty((M, N), dtype=torch.float32, device=dev)
            t, _ = time_graph(lambda i: vq.gemm(wt, Qs[i % R], N, K, vq.Q8_K, Xq, M, Y=Y), R, max(iters, 5 * R))
            b = Q.numel() + vq.act_bytes(vq.Q8_K, M, K) + 4 * M * N
            out["%s_M%d" % (name, M)] = {"us": round(t * 1e3, 2), "gbs": round(b / (t * 1e-3) / 1e9, 1),
                                         "frac": round(b / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                         "arm": "gemv" if M <= vq.small_batch_max(wt) else "mfma"}
        del Qs, Q
    return out


def run_producers(torch, vq, synth, iters):
    """RMSNorm -> Q8_K and SiLU-mul -> Q8_K in one launch, decode (M = 1) and
    prefill (M = 2048) rows; bytes = inputs read + Y written + Q8_K written."""
    dev = torch.device("cuda:0")
    out = {}
    for M, K in ((1, 2560), (2048, 2560), (1, 9728), (2048, 9728)):
        X = torch.from_numpy(synth.normal(71, (M, K))).to(dev)
        U = torch.from_numpy(synth.normal(72, (M, K))).to(dev)
        g = torch.from_numpy((1.0 + synth.normal(73, (K,), 0.1)).astype("float32")).to(dev)
        Y = torch.empty((M, K), dtype=torch.float32, device=dev)
        Xq = torch.empty(vq.act_bytes(vq.Q8_K, M, K), dtype=torch.uint8, device=dev)
        n = 16 if M == 1 else 4
        tr, _ = time_graph(lambda i: vq.rmsnorm_quant(vq.Q8_K, X, g, 1e-6, Y=Y, Xq=Xq), n, max(iters, 4 * n))
        ts, _ = time_graph(lambda i: vq.silu_mul_quant(vq.Q8_K, X, U, Y=Y, Xq=Xq), n, max(iters, 4 * n))
        tq, _ = time_graph(lambda i: vq.quantize_act(vq.Q8_K, X, Xq=Xq), n, max(iters, 4 * n))
        qb = vq.act_bytes(vq.Q8_K, M, K)
        br, bs = 4 * M * K + 4 * K + 4 * M * K + qb, 8 * M * K + 4 * M * K + qb
        out["M%d_K%d" % (M, K)] = {
            "rmsnorm_quant_us": round(tr * 1e3, 2), "rmsnorm_quant_gbs": round(br / (tr * 1e-3) / 1e9, 1),
            "silu_mul_quant_us": round(ts * 1e3, 2), "silu_mul_quant_gbs": round(bs / (ts * 1e-3) / 1e9, 1),
            "quantize_only_us": round(tq * 1e3, 2)}
    return out


def run_grouped(torch, vq, synth, iters):
    dev = torch.device("cuda:0")
    cfg = synth.WORKLOADS["grouped_moe"]
    E, N, K, T, top_k = cfg["E"], cfg["N"], cfg["K"], cfg["T"], cfg["top_k"]
    ebytes = vq.weight_bytes(vq.Q4_K, N, K)
    Q0 = torch.empty(E * ebytes, dtype=torch.uint8, device=dev)
    for e in range(E):
        We = torch.from_numpy(synth.expert_weights(e, N, K)).to(dev)
        vq.quantize_weights(vq.Q4_K, We, Wq=Q0[e * ebytes:(e + 1) * ebytes])
    torch.cuda.synchronize()
    X = torch.from_numpy(synth.tensor("grouped_moe", "X")).to(dev)
    ids_np, w_np = synth.routing(T, E, top_k)
    ids = torch.from_numpy(ids_np).to(dev)
    rw = torch.from_numpy(w_np).to(dev)
    Xq = vq.quantize_act(vq.Q8_K, X)
    Y = torch.empty((T, top_k, N), dtype=torch.float32, device=dev)
    S = torch.empty((T, N), dtype=torch.float32, device=dev)
    ws = torch.empty(vq.grouped_workspace_bytes(E, T, top_k), dtype=torch.uint8, device=dev)
    R = max(2, math.ceil(640 * (1 << 20) / Q0.numel()))
    Qs = [Q0] + [Q0.clone() for _ in range(R - 1)]

    def call(i, sets):
        vq.gemm_grouped(vq.Q4_K, sets[i % len(sets)], E, N, K, vq.Q8_K, Xq, T, ids, top_k, route_w=rw,
                        Y=Y, Ysum=S, ws=ws)

    t_cold, _ = time_graph(lambda i: call(i, Qs), R, max(iters, 3 * R))
    t_warm, _ = time_graph(lambda i: call(i, [Q0]), 4, iters)
    ops = 2.0 * T * top_k * N * K
    alg = Q0.numel() + Xq.numel() + Y.numel() * 4 + S.numel() * 4 + T * top_k * 8
    out = {"route_gemm_sum_us_cold": round(t_cold * 1e3, 2),
           "tops_cold": round(ops / (t_cold * 1e-3) / 1e12, 1),
           "mfma_frac_cold": round(ops / (t_cold * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
           "hbm_frac_cold": round(alg / (t_cold * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "route_gemm_sum_us_warm": round(t_warm * 1e3, 2),
           "tops_warm": round(ops / (t_warm * 1e-3) / 1e12, 1),
           "mfma_frac_warm": round(ops / (t_warm * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
           "rotation_sets_cold": R, "algorithmic_bytes": int(alg),
           "rows_per_expert": T * top_k / E, "tile_rows": tile_rows(T * top_k / E)}
    # 512 tokens (16 rows per expert): the first tokens of the same X and
    # routing, the same expert weights
    T2 = 512
    Xq2 = vq.quantize_act(vq.Q8_K, X[:T2].contiguous())
    ids2, rw2 = ids[:T2].contiguous(), rw[:T2].contiguous()
    Y2 = torch.empty((T2, top_k, N), dtype=torch.float32, device=dev)
    S2 = torch.empty((T2, N), dtype=torch.float32, device=dev)
    ws2 = torch.empty(vq.grouped_workspace_bytes(E, T2, top_k), dtype=torch.uint8, device=dev)
    t2, _ = time_graph(lambda i: vq.gemm_grouped(vq.Q4_K, Qs[i % R], E, N, K, vq.Q8_K, Xq2, T2, ids2, top_k,
                                                 route_w=rw2, Y=Y2, Ysum=S2, ws=ws2), R, max(iters, 3 * R))
    ops2 = 2.0 * T2 * top_k * N * K
    alg2 = Q0.numel() + Xq2.numel() + Y2.numel() * 4 + S2.numel() * 4 + T2 * top_k * 8
    out["n512"] = {"route_gemm_sum_us_cold": round(t2 * 1e3, 2),
                   "tops_cold": round(ops2 / (t2 * 1e-3) / 1e12, 1),
                   "mfma_frac_cold": round(ops2 / (t2 * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
                   "hbm_frac_cold": round(alg2 / (t2 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                   "algorithmic_bytes": int(alg2), "rows_per_expert": T2 * top_k / E,
                   "tile_rows": tile_rows(T2 * top_k / E)}
    return out


def tile_rows(r):
    """The routed tile height the library picks at r rows per expert (for the
    record: the smallest of 32, 64, 96 rows holding r + 3 sqrt(r), else 96)."""
    return 32 * min(3, max(1, math.ceil((r + 3.0 * math.sqrt(r)) / 32.0)))


def run_grouped_down(torch, vq, synth, iters):
    """The per-row arm at the MoE down-projection shape: 256 experts of Q4_K
    [2048, 512], one activation row per (token, slot) pair, top-8 routing."""
    dev = torch.device("cuda:0")
    cfg = synth.WORKLOADS["grouped_moe_down"]
    E, N, K, T, top_k = cfg["E"], cfg["N"], cfg["K"], cfg["T"], cfg["top_k"]
    ebytes = vq.weight_bytes(vq.Q4_K, N, K)
    Q0 = torch.empty(E * ebytes, dtype=torch.uint8, device=dev)
    for e in range(E):
        We = torch.from_numpy(synth.expert_weights(e, N, K, seed=cfg["W_seed"])).to(dev)
        vq.quantize_weights(vq.Q4_K, We, Wq=Q0[e * ebytes:(e + 1) * ebytes])
    torch.cuda.synchronize()
    X = torch.from_numpy(synth.tensor("grouped_moe_down", "X")).to(dev)
    ids_np, w_np = synth.routing(T, E, top_k)
    ids = torch.from_numpy(ids_np).to(dev)
    rw = torch.from_numpy(w_np).to(dev)
    Xq = vq.quantize_act(vq.Q8_K, X)
    Y = torch.empty((T, top_k, N), dtype=torch.float32, device=dev)
    S = torch.empty((T, N), dtype=torch.float32, device=dev)
    ws = torch.empty(vq.grouped_workspace_bytes(E, T, top_k), dtype=torch.uint8, device=dev)
    R = max(2, math.ceil(640 * (1 << 20) / Q0.numel()))
    Qs = [Q0] + [Q0.clone() for _ in range(R - 1)]

    def call(i, sets):
        vq.gemm_grouped(vq.Q4_K, sets[i % len(sets)], E, N, K, vq.Q8_K, Xq, T, ids, top_k, route_w=rw,
                        Y=Y, Ysum=S, ws=ws, per_row=True)

    t_cold, _ = time_graph(lambda i: call(i, Qs), R, max(iters, 3 * R))
    ops = 2.0 * T * top_k * N * K
    alg = Q0.numel() + Xq.numel() + Y.numel() * 4 + S.numel() * 4 + T * top_k * 8
    return {"shape": "E=256 x Q4_K [2048,512], per-row Q8_K input [16384,512], top-8",
            "route_gemm_sum_us_cold": round(t_cold * 1e3, 2),
            "tops_cold": round(ops / (t_cold * 1e-3) / 1e12, 1),
            "mfma_frac_cold": round(ops / (t_cold * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
            "hbm_frac_cold": round(alg / (t_cold * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "rotation_sets_cold": R, "algorithmic_bytes": int(alg)}


def run_ceilings(torch, vq):
    """Measured ceilings beside the spec peaks: the int8 MFMA rate of
    vq_mfma_probe (register operands, nothing else, 2 workgroups per CU), a
    1 GiB device-to-device copy (read + write bytes) by torch, and a 570 MB
    read-only stream (vq_stream_probe)."""
    dev = torch.device("cuda:0")
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    iters = 4096
    for _ in range(5):  # about 5 ms of the same load first: the clocks settle under it
        vq.mfma_probe(iters, sink)
    torch.cuda.synchronize()
    times = []
    for _ in range(9):
        a, b = event_pair()
        a.record()
        ops = vq.mfma_probe(iters, sink)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    ms = sorted(times)[len(times) // 2]
    tops = ops / (ms * 1e-3) / 1e12
    n = 1 << 28  # 1 GiB of fp32
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ct = []
    for _ in range(5):
        a, b = event_pair()
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        ct.append(a.elapsed_time(b))
    cms = sorted(ct)[len(ct) // 2]
    gbs = 2 * 4 * n / (cms * 1e-3) / 1e9
    del src, dst
    # read-only: the streaming probe over a 570 MB Q8_0 buffer (262144 rows of
    # 2048), each workgroup reading its rows once
    Nr, Kr = 262144, 2048
    Wr = torch.zeros(vq.weight_bytes(vq.Q8_0, Nr, Kr), dtype=torch.uint8, device=dev)
    rsink = torch.zeros(Nr, dtype=torch.int32, device=dev)
    vq.stream_probe(vq.Q8_0, Wr, Nr, Kr, rsink)
    torch.cuda.synchronize()
    rt = []
    for _ in range(5):
        a, b = event_pair()
        a.record()
        vq.stream_probe(vq.Q8_0, Wr, Nr, Kr, rsink)
        b.record()
        torch.cuda.synchronize()
        rt.append(a.elapsed_time(b))
    rms = sorted(rt)[len(rt) // 2]
    rgbs = Wr.numel() / (rms * 1e-3) / 1e9
    del Wr, rsink
    return {"int8_mfma_tops": round(tops, 1), "int8_mfma_frac_of_spec": round(tops / INT8_PEAK_TOPS, 4),
            "int8_mfma_probe": "vq_mfma_probe: %d rounds of 8 v_mfma_i32_32x32x32_i8 chains per wave, "
                               "2 workgroups of 4 waves per CU, %.1f us" % (iters, ms * 1e3),
            "hbm_copy_gbs": round(gbs, 1), "hbm_copy_frac_of_spec": round(gbs / HBM_PEAK_GBS, 4),
            "hbm_copy": "1 GiB device-to-device copy (torch), read + write bytes, %.1f us" % (cms * 1e3),
            "hbm_read_gbs": round(rgbs, 1), "hbm_read_frac_of_spec": round(rgbs / HBM_PEAK_GBS, 4),
            "hbm_read": "vq_stream_probe over a 570 MB buffer (Q8_0 [262144, 2048]), %.1f us" % (rms * 1e3)}


def calibrate_copy(torch, nbytes):
    """A plain device copy of known size, for scaling rocprofv3 FETCH_SIZE and
    WRITE_SIZE (run under rocprofv3 --pmc)."""
    dev = torch.device("cuda:0")
    a = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "launches": 5}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rotate-mb", type=int, default=640,
                    help="total size of the rotated weight sets (> the 256 MB Infinity Cache)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--secondary-iters", type=int, default=20)
    ap.add_argument("--sections", default="prefill,q8_0,q5k,small_batch,producers,grouped,grouped_down_per_row,ceilings",
                    help="comma-separated secondary sections to run (all by default)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes (rocprofv3 counter scaling)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path; run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X (no GPU visible)", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy(torch, args.calibrate_copy)
        return

    import block_quantized_matmul_fp32_amd as vq
    import synth
    vq.lib()  # fails loudly if the HIP library is missing

    log("[bench] decode step: warmup %d, steps %d" % (args.warmup, args.steps))
    dec = run_decode(args, torch, vq, synth)
    step_bytes = decode_step_bytes()
    value = step_bytes / (dec["ms_per_step"] * 1e-3) / 1e9
    b6 = 2560 * (9728 // 256) * 210 + 4 * 9728 + 4 * 2560
    ach6 = b6 / (dec["q6k_ms"] * 1e-3) / 1e9
    b4 = 9728 * (2560 // 256) * 144 + 4 * 2560 + 4 * 9728
    ach4 = b4 / (dec["q4k_ms"] * 1e-3) / 1e9
    sha = source_sha(GEMV_SOURCES)
    roofline = {"bound": "hbm", "kernel": "gemv_kernel<1, 1> (Q6_K [2560,9728] x fused Q8_K)",
                "achieved": round(ach6, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach6 / HBM_PEAK_GBS, 4),
                "traffic": traffic_from_profiles("gemv_q6k_decode", sha, b6),
                "algorithmic_bytes_per_launch": b6,
                "median_launch_us": round(dec["q6k_ms"] * 1e3, 3),
                "avg_launch_us": round(dec["q6k_mean_ms"] * 1e3, 3),
                "stream_floor_us": round(dec["q6k_floor_ms"] * 1e3, 3),
                "source_sha": sha}
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": dec["steps_timed"], "warmup": args.warmup, "ms_per_step": round(dec["ms_per_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "decode GEMV, M=1: Q4_K [9728,2560] + Q6_K [2560,9728], "
                               "Q8_K activation quantizer fused, seeded N(0,1) x and N(0,0.02) weights",
                   "global_batch": 1, "parallelism": "none (1 GPU)",
                   "launch": "timed steps replay a HIP graph (one step per rotation set)",
                   "rotation_sets": dec["rotation_sets"], "rotation_mb": dec["rotation_mb"],
                   "bytes_per_step": step_bytes},
        "roofline": roofline,
        "decode_kernels": {"q4k_us": round(dec["q4k_ms"] * 1e3, 3), "q4k_gbs": round(ach4, 1),
                           "q4k_frac": round(ach4 / HBM_PEAK_GBS, 4),
                           "q4k_stream_floor_us": round(dec["q4k_floor_ms"] * 1e3, 3),
                           "q6k_us": round(dec["q6k_ms"] * 1e3, 3), "q6k_gbs": round(ach6, 1),
                           "q6k_frac": round(ach6 / HBM_PEAK_GBS, 4),
                           "q6k_stream_floor_us": round(dec["q6k_floor_ms"] * 1e3, 3),
                           "timing": "median over graph replays of rotated (cold) launches",
                           "stream_floor": "vq_stream_probe: the GEMV's weight bytes and launch shape, no compute"},
    }
    wanted = set(x for x in args.sections.split(",") if x)
    if not args.no_secondary:
        it = args.secondary_iters
        sections = [
            ("prefill", "prefill GEMM", lambda: run_prefill(torch, vq, synth, it)),
            ("q8_0", "Q8_0 GEMM, GEMV and quantizer", lambda: run_q8_0(torch, vq, synth, it)),
            ("q5k", "Q5_K GEMV and GEMM", lambda: run_q5k(torch, vq, synth, it)),
            ("small_batch", "small batches", lambda: run_small_batch(torch, vq, synth, it)),
            ("producers", "producers with the quantizer epilogue", lambda: run_producers(torch, vq, synth, it)),
            ("grouped", "grouped MUL_MAT_ID", lambda: run_grouped(torch, vq, synth, max(5, it // 2))),
            ("grouped_down_per_row", "grouped per-row arm (MoE down projection)",
             lambda: run_grouped_down(torch, vq, synth, max(5, it // 2))),
        ]
        unknown = wanted - set(k for k, _, _ in sections) - {"ceilings"}
        if unknown:
            sys.exit("unknown --sections entries: %s" % ", ".join(sorted(unknown)))
        for key, what, fn in sections:
            if key in wanted:
                log("[bench] " + what)
                line[key] = fn()
    if not args.no_secondary and "ceilings" in wanted:
        log("[bench] measured ceilings (int8 MFMA probe, 1 GiB copy)")
        line["ceilings"] = run_ceilings(torch, vq)
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline (%.0f s)" % args.cpu_seconds)
        line["cpu_baseline"] = run_cpu_baseline(args.cpu_seconds)
        line["cpu_baseline"]["gpu_speedup"] = round(line["cpu_baseline"]["ms_per_step"] / dec["ms_per_step"], 1)
        log("[bench] fp64 reference (numpy)")
        line["cpu_baseline"]["fp64_reference"] = run_cpu_fp64_reference()
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
