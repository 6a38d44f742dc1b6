#!/usr/bin/env python3
"""Throughput of the W4A8 block-quantized GEMV path on one MI355X.

One step = one batch-1 Llama-3.1-8B decode pass over the Llama-shaped
matrices of the hot path, stream-ordered on one HIP stream with no host
round trip:
    quantize(x) + gate|up Q4_K 28672 x 4096 + SiLU(gate)*up + requantize
                           (one launch)
    -> down Q6_K 4096 x 14336
    quantize(x') + lm_head Q6_K 128256 x 4096 (one launch)
(--separate-quant quantizes x and x' in launches of their own; --unfused also
splits gate|up from SiLU*up + requantize.)
All inputs are seeded synthetic data (synth module) resident in HBM before the
timed region; weights are rotated over --copies copies so consecutive steps do
not read the same bytes (one copy is already 545 MB, twice the 256 MB
Infinity Cache).

Prints ONE JSON line on stdout (diagnostics go to stderr):
  value      weight GB/s of the whole step (logical weight bytes / step time)
  roofline   the dominant kernel (the lm_head Q6_K GEMV): algorithmic bytes
             per launch / its average duration from HIP events recorded
             around each of its launches inside the timed region
  cpu_baseline  the CPU oracle timed on this host over whole steps
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
SMALL_M_LIST = (1, 2, 4, 8, 16, 24, 32, 48, 64)
METRIC = "quantized GEMV weight GB/s and % of HBM peak at Llama-3-8B shapes, 1 GPU"
WORKLOAD = ("llama3.1-8b decode step, batch 1: ffn gate|up q4_k 28672x4096 with fused "
            "silu*up requant -> down q6_k 4096x14336, then lm_head q6_k 128256x4096 "
            "(activation quantization inside the gate|up and lm_head launches; "
            "q6_k repacked at load into aligned 8-super-block tiles, same bytes)")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_q6k_lm_head.json")
# the sources the lm_head kernel is built from (its unit code, quantiser,
# kernel template and launcher); a stored traffic profile applies only while
# they are unchanged
KERNEL_SOURCES = ["qgemv_device.h", "qgemv_quant.h", "k_gemv.h", "k_gemv.hip",
                  "k_gemv_q6_k_r8.hip"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipTimer:
    """Two pairs of HIP events created without the system-scope fence
    (hipEventDisableSystemFence): the default fence writes back and
    invalidates the caches at every record, which opens a gap of several
    microseconds in the queue.  Pair 0 brackets a launch on its stream (it
    also takes in the queue gap before the kernel); pair 1 is handed to
    qgemv_time_next_launch, so that the kernel itself records it at its start
    and end."""
    FLAGS = 0x20000000  # hipEventDisableSystemFence

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.c_void_p, ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.c_void_p, ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(4):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreateWithFlags(ctypes.byref(e), self.FLAGS) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.ev.append(e)

    def record(self, k, stream_handle):
        if self.hip.hipEventRecord(self.ev[k], stream_handle) != 0:
            raise RuntimeError("hipEventRecord failed")

    def kernel_events(self):
        return self.ev[2], self.ev[3]

    def elapsed_ms(self, pair=0):
        a, b = self.ev[2 * pair], self.ev[2 * pair + 1]
        ms = self.ct.c_float()
        self.hip.hipEventSynchronize(b)
        if self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        for e in getattr(self, "ev", []):
            self.hip.hipEventDestroy(e)


def workload_name(args) -> str:
    w = WORKLOAD
    if args.unfused or args.separate_quant:
        w = w.replace("activation quantization inside the gate|up and lm_head launches; ",
                      "activation quantization in launches of its own; ")
    if args.unfused:
        w = w.replace("with fused", "then a separate")
    if args.native_q6k:
        w = w.replace("(q6_k repacked at load into aligned 8-super-block tiles, same bytes)",
                      "(q6_k in the on-disk layout)")
    return w


def kernel_fingerprint() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "block_quantized_gemv_w4a8_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=1000,
                    help="untimed steps first (0.1 s: the clocks settle; 30 steps read ~1 us "
                         "per step slower)")
    ap.add_argument("--copies", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the per-kernel/config extras")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--event-every", type=int, default=30,
                    help="bracket every n-th lm_head launch of the timed steps with HIP events "
                         "(each pair costs ~20 us of step time, so they are sampled)")
    ap.add_argument("--roofline-steps", type=int, default=30,
                    help="after the timed steps, this many more steps (same rotation) in which "
                         "every lm_head launch records its own start/end events; the roofline's "
                         "duration is their average")
    ap.add_argument("--small-m-profile", action="store_true",
                    help="only run the small-M products (Q4_K 14336x4096, Q6_K 4096x14336; "
                         "both variants at every M of SMALL_M_LIST), 20 calls each, for "
                         "counter collection")
    ap.add_argument("--native-q6k", action="store_true",
                    help="run the Q6_K GEMVs on the on-disk layout instead of the repacked one")
    ap.add_argument("--unfused", action="store_true",
                    help="gate|up GEMV and SiLU*up requant as two launches, and the activation "
                         "quantizations as launches of their own (comparison)")
    ap.add_argument("--separate-quant", action="store_true",
                    help="quantize x and x' in launches of their own (comparison)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (for counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the "
              "multi-GPU sharding of this path is a design note, not a measured mode.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_quantized_gemv_w4a8_amd as qg
    import synth

    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.small_m_profile:
        small_m_profile(qg, torch, np, synth, dev)
        return
    t0 = time.time()
    c2 = synth.config2()
    c3 = synth.config3()
    log(f"[bench] inputs generated in {time.time() - t0:.1f}s")
    Ngu, Kgu, Nd, Kd = c2["N_gu"], c2["K_gu"], c2["N_down"], c2["K_down"]
    Nh, Kh = c3["N"], c3["K"]
    R = max(1, args.copies)
    w_gu = [torch.from_numpy(c2["w_gu"]).to(dev)]
    w_dn = [torch.from_numpy(c2["w_down"]).to(dev)]
    w_hd = [torch.from_numpy(c3["w"]).to(dev)]
    for _ in range(R - 1):
        w_gu.append(w_gu[0].clone())
        w_dn.append(w_dn[0].clone())
        w_hd.append(w_hd[0].clone())
    # load-time repack of the Q6_K weights (outside the timed region; the
    # repacked rows hold the same bytes, only moved into aligned tiles)
    gemv_q6 = qg.qgemv_q6_k
    fmt_q6 = qg.QGEMV_FMT_Q6_K
    if not args.native_q6k:
        def repack(wt, N, K):
            wr = torch.empty((N, qg.q6_k_r8_row_bytes(K)), dtype=torch.uint8, device=dev)
            qg.qgemv_q6_k_repack(wt, N, K, wr)
            return wr
        w_dn = [repack(wt, Nd, Kd) for wt in w_dn]
        w_hd = [repack(wt, Nh, Kh) for wt in w_hd]
        torch.cuda.synchronize()
        gemv_q6 = qg.qgemv_q6_k_r8
        fmt_q6 = qg.QGEMV_FMT_Q6_K_R8
    x_ffn = torch.from_numpy(c2["x"]).to(dev)
    x_head = torch.from_numpy(c3["x"]).to(dev)
    q1, d1, s1 = qg.act_buffers(1, Kgu, dev)
    gu = torch.empty(Ngu, dtype=torch.float32, device=dev)
    q2, d2, s2 = qg.act_buffers(1, Kd, dev)
    y_ffn = torch.empty(Nd, dtype=torch.float32, device=dev)
    q3, d3, s3 = qg.act_buffers(1, Kh, dev)
    logits = torch.empty(Nh, dtype=torch.float32, device=dev)

    wbytes = {
        "gate_up": synth.logical_bytes("q4_k", Ngu, Kgu),
        "down": synth.logical_bytes("q6_k", Nd, Kd),
        "lm_head": synth.logical_bytes("q6_k", Nh, Kh),
    }
    step_wbytes = sum(wbytes.values())
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    sep_quant = args.unfused or args.separate_quant

    def step(i, ev=None):
        c = i % R
        if sep_quant:
            qg.qgemv_quantize_act(x_ffn, 1, Kgu, Kgu, q1, d1, s1, stream=sh)
        if args.unfused:
            qg.qgemv_q4_k(w_gu[c], Ngu, Kgu, q1, d1, s1, gu, stream=sh)
            qg.qgemv_silu_mul_quantize(gu, Kd, q2, d2, s2, None, stream=sh)
        elif sep_quant:
            qg.qgemv_q4_k_swiglu_quantize(w_gu[c], Kd, Kgu, q1, d1, s1, q2, d2, s2, None, None,
                                          stream=sh)
        else:
            qg.qgemv_quantize_q4_k_swiglu(w_gu[c], Kd, Kgu, x_ffn, q1, d1, s1, q2, d2, s2,
                                          None, None, stream=sh)
        gemv_q6(w_dn[c], Nd, Kd, q2, d2, s2, y_ffn, stream=sh)
        if sep_quant:
            qg.qgemv_quantize_act(x_head, 1, Kh, Kh, q3, d3, s3, stream=sh)
        if ev is not None:
            ev.record(0, sh)
            qg.qgemv_time_next_launch(*ev.kernel_events())
        if sep_quant:
            gemv_q6(w_hd[c], Nh, Kh, q3, d3, s3, logits, stream=sh)
        else:
            qg.qgemv_quantize_gemv(fmt_q6, w_hd[c], Nh, Kh, x_head, q3, d3, s3, logits,
                                   stream=sh)
        if ev is not None:
            ev.record(1, sh)

    # the achievable read rate is measured right before the warm-up steps: its
    # ~30 streaming reads of 1 GiB also bring the GPU out of the idle it sat
    # in while the host generated the inputs, so a short warm-up (the
    # driver's 5 steps) starts the timed steps on a busy device
    read = read_kernel_rate(qg, torch, np, dev)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    K = max(1, args.steps)
    # every P-th step's lm_head is bracketed by events (at least one when
    # fewer than P steps are timed)
    P = max(1, min(args.event_every, K))
    evs = [HipTimer() if i % P == P - 1 else None for i in range(K)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    start.record(stream)
    for i in range(K):
        step(i, evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    w1 = time.perf_counter()
    gpu_ms = start.elapsed_time(end)
    wall_ms = (w1 - w0) * 1e3
    ms_per_step = max(gpu_ms, wall_ms) / K
    value = step_wbytes / (ms_per_step * 1e-3) / 1e9
    # the lm_head kernel's own start/end events (qgemv_time_next_launch), and
    # the bracket recorded on the stream around the same launch: sampled
    # inside the timed steps ...
    loop_us = [e.elapsed_ms(1) * 1e3 for e in evs if e is not None]
    # ... and on every lm_head launch of a window of further steps (the same
    # rotation continued), which the roofline's duration is read from
    RW = max(5, args.roofline_steps)
    evw = [HipTimer() for _ in range(RW)]
    for i in range(RW):
        step(K + i, evw[i])
    torch.cuda.synchronize()
    head_us = [e.elapsed_ms(1) * 1e3 for e in evw]
    bracket_us = [e.elapsed_ms(0) * 1e3 for e in evw]
    head_avg_us = float(np.mean(head_us))
    bracket_avg_us = float(np.mean(bracket_us))
    log(f"[bench] step {ms_per_step * 1e3:.1f} us (events {gpu_ms / K * 1e3:.1f}, wall "
        f"{wall_ms / K * 1e3:.1f}); lm_head kernel avg {head_avg_us:.2f} us over "
        f"{len(head_us)} event-timed launches after the timed steps (stream bracket "
        f"{bracket_avg_us:.2f} us; {float(np.mean(loop_us)):.2f} us over {len(loop_us)} "
        f"launches sampled inside them)")

    # dominant kernel roofline: algorithmic bytes per launch of the lm_head GEMV
    # = N rows x (row weight bytes + 4 B output) + one activation row (codes,
    # scales, sums) + (quantization in the launch) the fp32 input row
    act_bytes = Kh + 2 * (Kh // 32) + 4 * (Kh // 32)
    head_alg = Nh * (synth.row_bytes("q6_k", Kh) + 4) + act_bytes + (0 if sep_quant else 4 * Kh)
    achieved = head_alg / (head_avg_us * 1e-6) / 1e9
    traffic, traffic_src = None, None
    if os.path.exists(TRAFFIC_FILE):
        tr = json.load(open(TRAFFIC_FILE))
        fp = kernel_fingerprint()
        if tr.get("kernel_fingerprint") == fp:
            traffic = tr.get("bytes_per_launch")
            traffic_src = (f"stored profile profiles/{os.path.basename(TRAFFIC_FILE)} "
                           f"(rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE passes of an earlier "
                           f"run, scaled by a 1 GiB copy; kernel source fingerprint {fp}), "
                           f"not measured in this run")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "kernel": (("qgemv_q6_k lm_head 128256x4096" if args.native_q6k else
                            "qgemv_q6_k_r8 lm_head 128256x4096 (repacked Q6_K)") +
                           ("" if sep_quant else ", activation quantized in the launch "
                            "(qgemv_quantize_gemv)")),
                "traffic_source": traffic_src,
                "avg_us": round(head_avg_us, 2),
                "timed_launches": len(head_us),
                "timing": ("kernel start/end events (qgemv_time_next_launch) on every lm_head "
                           "launch of %d steps run right after the timed steps" % len(head_us)),
                "in_loop_sampled_avg_us": round(float(np.mean(loop_us)), 2),
                "in_loop_sampled_launches": len(loop_us),
                "stream_bracket_avg_us": round(bracket_avg_us, 2),
                "alg_bytes_per_launch": head_alg,
                "achievable_read_GBps": read["GBps"],
                "frac_of_achievable_read": round(achieved / read["GBps"], 4)}

    extra = {}
    if not args.no_extra:
        extra = extras(qg, torch, np, synth, dev, R, c2, c3, args)

    if args.calib_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(np, synth, c2, c3, args.cpu_seconds, step_wbytes)

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded; shapes and value distributions of the five workloads)",
        "config": {"workload": workload_name(args), "batch": 1,
                   "weight_bytes_per_step": step_wbytes, "weight_copies_rotated": R,
                   "steps_per_s": round(1e3 / ms_per_step, 1)},
        "hbm_peak_frac": round(value / HBM_PEAK_GBPS, 4),
        "read_kernel": read,
        "read_kernel_frac": round(value / read["GBps"], 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if extra:
        out["extra"] = extra
    print(json.dumps(out), flush=True)


def read_kernel_rate(qg, torch, np, dev, gib=1, reps=5):
    """The achievable HBM read rate on this device: qgemv_stream_read (plain
    16-byte streaming loads, non-temporal and ordinary, 2 or 4 workgroups per
    compute unit) over `gib` GiB, timed with events around each read after
    two warm-up reads; the best configuration's median."""
    nbytes = gib << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.random_(0, 256)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    res = {}
    for nt in (1, 0):
        for wpc in (2, 4):
            for _ in range(2):
                qg.qgemv_stream_read(buf, nbytes, nt, sink, wpc)
            per = []
            for _ in range(reps):
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record()
                qg.qgemv_stream_read(buf, nbytes, nt, sink, wpc)
                b.record()
                torch.cuda.synchronize()
                per.append(a.elapsed_time(b) * 1e-3)
            res[(nt, wpc)] = nbytes / float(np.median(per)) / 1e9
    del buf
    best = max(res, key=res.get)
    out = {"GBps": round(res[best], 1), "bytes": nbytes,
           "config": {"nontemporal": bool(best[0]), "wg_per_cu": best[1]},
           "all_GBps": {f"{'nt' if k[0] else 'plain'}_wg{k[1]}": round(v, 1)
                        for k, v in res.items()},
           "kernel": "qgemv_stream_read: 16-byte loads, 8 per thread in flight, grid-stride"}
    log(f"[bench] read kernel {out['GBps']} GB/s ({out['all_GBps']})")
    return out


def small_m_profile(qg, torch, np, synth, dev):
    """The small-M products alone (both variants, every M of SMALL_M_LIST,
    20 calls each, in this order), for rocprofv3 counter passes."""
    g = np.random.default_rng(4)
    for fmt, N, K in (("q4_k", 14336, 4096), ("q6_k", 4096, 14336)):
        w = torch.from_numpy(synth.weights(fmt, g, N, K)).to(dev)
        x64, _ = synth.activation(g, 64, K)
        for M in SMALL_M_LIST:
            q, d, s = qg.act_buffers(M, K, dev)
            qg.qgemv_quantize_act(torch.from_numpy(np.ascontiguousarray(x64[:M])).to(dev), M, K, K,
                                  q, d, s)
            y = torch.empty((M, N), dtype=torch.float32, device=dev)
            for v in (qg.QGEMV_VARIANT_DOT4, qg.QGEMV_VARIANT_MFMA):
                for _ in range(20):
                    qg.SMALL_M[fmt](w, N, K, M, q, d, s, y, v)
                torch.cuda.synchronize()
            log(f"[small-m-profile] {fmt} {N}x{K} M={M} done")


def kernel_stats(torch, fn, iters, R, windows=5):
    """Microseconds per launch of fn(i) over `windows` windows of `iters`
    back-to-back launches (events around each window), after `iters` warm-up
    launches: median, min and max of the windows.  A kernel shorter than the
    host's cost of one call reads as that cost here; its own duration is in
    the kernel trace."""
    for i in range(iters):
        fn(i % R)
    torch.cuda.synchronize()
    per = []
    for _ in range(windows):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(iters):
            fn(i % R)
        b.record()
        torch.cuda.synchronize()
        per.append(a.elapsed_time(b) * 1e3 / iters)
    per.sort()
    return {"us": round(per[len(per) // 2], 2), "us_min": round(per[0], 2),
            "us_max": round(per[-1], 2)}


def time_kernel(torch, fn, iters, R):
    """The median of kernel_stats (microseconds per launch)."""
    return kernel_stats(torch, fn, iters, R)["us"]


def graph_time(torch, calls, reps=20):
    """Capture `calls` (each launches on the current stream) into one graph;
    returns microseconds per replay."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for f in calls:
            f()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in calls:
            f()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return g, a.elapsed_time(b) * 1e3 / reps


def graph_config0_fused(qg, torch, np, dev, c0, copies):
    """Config 0 with the activation quantised in each GEMV's own launch
    (qgemv_quantize_gemv), one graph of `copies` launches; a replay's output
    must equal the eager call's bit for bit."""
    ws = [torch.from_numpy(c0["w"]).to(dev)]
    for _ in range(copies - 1):
        ws.append(ws[0].clone())
    x = torch.from_numpy(c0["x"]).to(dev)
    q, d, s = qg.act_buffers(1, 896, dev)
    ys = torch.empty((copies, 896), dtype=torch.float32, device=dev)
    F = qg.QGEMV_FMT_Q4_0
    calls = [lambda c=c: qg.qgemv_quantize_gemv(F, ws[c], 896, 896, x, q, d, s, ys[c])
             for c in range(copies)]
    eager = torch.empty(896, dtype=torch.float32, device=dev)
    qg.qgemv_quantize_gemv(F, ws[0], 896, 896, x, q, d, s, eager)
    g, us = graph_time(torch, calls)
    ys.fill_(float("nan"))
    g.replay()
    torch.cuda.synchronize()
    same = bool(torch.equal(ys[0].view(torch.int32), eager.view(torch.int32)) and
                torch.equal(ys[-1].view(torch.int32), eager.view(torch.int32)))
    per = us / copies
    del ws, g
    return {"us_per_quantize_gemv": round(per, 3), "weight_GBps": round(451584 / per / 1e3, 1),
            "calls_per_s": round(1e6 / per), "replay_equals_eager": same}


def graph_config0(qg, torch, np, dev, c0, copies):
    """Config 0 (Q4_0 896x896) as one graph of `copies` GEMVs over rotated
    weight copies; a replay's output must equal the eager call's bit for bit."""
    ws = [torch.from_numpy(c0["w"]).to(dev)]
    for _ in range(copies - 1):
        ws.append(ws[0].clone())
    q, d, s = qg.act_buffers(1, 896, dev)
    qg.qgemv_quantize_act(torch.from_numpy(c0["x"]).to(dev), 1, 896, 896, q, d, s)
    ys = torch.empty((copies, 896), dtype=torch.float32, device=dev)
    calls = [lambda c=c: qg.qgemv_q4_0(ws[c], 896, 896, q, d, s, ys[c]) for c in range(copies)]
    eager = torch.empty(896, dtype=torch.float32, device=dev)
    qg.qgemv_q4_0(ws[0], 896, 896, q, d, s, eager)
    g, us = graph_time(torch, calls)
    ys.fill_(float("nan"))
    g.replay()
    torch.cuda.synchronize()
    same = bool(torch.equal(ys[0].view(torch.int32), eager.view(torch.int32)) and
                torch.equal(ys[-1].view(torch.int32), eager.view(torch.int32)))
    per = us / copies
    del ws, g
    return {"us_per_gemv": round(per, 3), "weight_GBps": round(451584 / per / 1e3, 1),
            "calls_per_s": round(1e6 / per), "replay_equals_eager": same}


def graph_config1(qg, torch, np, dev, c1, layers, fused=False, grouped=False):
    """One config-1 layer per rotated weight copy, `layers` layers in one
    graph: 3 activation quantisations + 7 Q4_K GEMVs; with `fused`, 7 GEMVs
    that quantise their own input; with `grouped`, 4 launches in the order a
    decode layer's dependencies allow -- q|k|v, o, gate|up (qgemv_quantize_multi
    where matrices share an input), down."""
    mats = c1["mats"]
    wl = {n: [torch.from_numpy(m["w"]).to(dev)] for n, m in mats.items()}
    for n in wl:
        for _ in range(layers - 1):
            wl[n].append(wl[n][0].clone())
    # activations: q/k/v/gate/up share one 896-vector, o and down have their own
    xs = {}
    for n, m in mats.items():
        key = m["x"].tobytes()
        if key not in xs:
            xs[key] = (torch.from_numpy(m["x"]).to(dev), m["K"], qg.act_buffers(1, m["K"], dev))
    ys = {n: torch.empty(m["N"], dtype=torch.float32, device=dev) for n, m in mats.items()}

    def layer(c):
        if grouped:
            calls = []
            for names in (("q", "k", "v"), ("o",), ("gate", "up"), ("down",)):
                m0 = mats[names[0]]
                x, _, a = xs[m0["x"].tobytes()]
                calls.append(lambda names=names, m0=m0, x=x, a=a: qg.qgemv_quantize_multi(
                    qg.QGEMV_FMT_Q4_K, [wl[n][c] for n in names], [mats[n]["N"] for n in names],
                    m0["K"], x, *a, [ys[n] for n in names]))
            return calls
        if fused:
            calls = []
            for n, m in mats.items():
                x, _, a = xs[m["x"].tobytes()]
                calls.append(lambda n=n, m=m, x=x, a=a: qg.qgemv_quantize_gemv(
                    qg.QGEMV_FMT_Q4_K, wl[n][c], m["N"], m["K"], x, *a, ys[n]))
            return calls
        calls = [lambda x=x, K=K, a=a: qg.qgemv_quantize_act(x, 1, K, K, *a)
                 for x, K, a in xs.values()]
        for n, m in mats.items():
            a = xs[m["x"].tobytes()][2]
            calls.append(lambda n=n, m=m, a=a: qg.qgemv_q4_k(wl[n][c], m["N"], m["K"], *a, ys[n]))
        return calls

    calls = []
    for c in range(layers):
        calls += layer(c)
    for f in layer(0):
        f()
    torch.cuda.synchronize()
    eager = {n: y.clone() for n, y in ys.items()}
    g, us = graph_time(torch, calls)
    for y in ys.values():
        y.fill_(float("nan"))
    g.replay()
    torch.cuda.synchronize()
    same = all(torch.equal(ys[n].view(torch.int32), eager[n].view(torch.int32)) for n in ys)
    per = us / layers
    del wl, g
    return {"us_per_layer": round(per, 2), "weight_GBps": round(8386560 / per / 1e3, 1),
            "layers_per_s": round(1e6 / per), "replay_equals_eager": same}


def extras(qg, torch, np, synth, dev, R, c2, c3, args):
    """Per-kernel timings of the step's GEMVs and the other workloads."""
    ex = {}
    Ngu, Kgu, Nd, Kd = c2["N_gu"], c2["K_gu"], c2["N_down"], c2["K_down"]
    Nh, Kh = c3["N"], c3["K"]

    def gemv_case(fmt, w_host, N, K, x, copies):
        ws = [torch.from_numpy(w_host).to(dev)]
        if fmt == "q6_k_r8":
            wr = torch.empty((N, qg.q6_k_r8_row_bytes(K)), dtype=torch.uint8, device=dev)
            qg.qgemv_q6_k_repack(ws[0], N, K, wr)
            ws = [wr]
        for _ in range(copies - 1):
            ws.append(ws[0].clone())
        q, d, s = qg.act_buffers(1, K, dev)
        qg.qgemv_quantize_act(torch.from_numpy(x).to(dev), 1, K, K, q, d, s)
        y = torch.empty(N, dtype=torch.float32, device=dev)
        f = qg.GEMV[fmt]
        st = kernel_stats(torch, lambda c: f(ws[c], N, K, q, d, s, y), 100, copies)
        us = st["us"]
        wb = synth.logical_bytes(fmt.replace("_r8", ""), N, K)
        del ws
        return {**st, "weight_GBps": round(wb / us / 1e3, 1),
                "hbm_frac": round(wb / us / 1e3 / HBM_PEAK_GBPS, 4), "calls_per_s": round(1e6 / us),
                "weight_copies_rotated": copies}

    ex["gate_up_q4_k_28672x4096"] = gemv_case("q4_k", c2["w_gu"], Ngu, Kgu, c2["x"], 8)
    # the same product with SiLU*up and the requantisation fused in (one launch)
    wsw = [torch.from_numpy(c2["w_gu"]).to(dev)]
    for _ in range(7):
        wsw.append(wsw[0].clone())
    qa, da, sa = qg.act_buffers(1, Kgu, dev)
    qg.qgemv_quantize_act(torch.from_numpy(c2["x"]).to(dev), 1, Kgu, Kgu, qa, da, sa)
    qo, do, so = qg.act_buffers(1, Kd, dev)
    us = time_kernel(torch, lambda c: qg.qgemv_q4_k_swiglu_quantize(
        wsw[c], Kd, Kgu, qa, da, sa, qo, do, so, None, None), 100, 8)
    wb = synth.logical_bytes("q4_k", Ngu, Kgu)
    ex["gate_up_swiglu_fused_q4_k_28672x4096"] = {
        "us": round(us, 2), "weight_GBps": round(wb / us / 1e3, 1),
        "hbm_frac": round(wb / us / 1e3 / HBM_PEAK_GBPS, 4), "calls_per_s": round(1e6 / us)}
    # ... and with the quantisation of x in the same launch
    xg = torch.from_numpy(c2["x"]).to(dev)
    us = time_kernel(torch, lambda c: qg.qgemv_quantize_q4_k_swiglu(
        wsw[c], Kd, Kgu, xg, qa, da, sa, qo, do, so, None, None), 100, 8)
    ex["quantize_gate_up_swiglu_fused_q4_k_28672x4096"] = {
        "us": round(us, 2), "weight_GBps": round(wb / us / 1e3, 1),
        "hbm_frac": round(wb / us / 1e3 / HBM_PEAK_GBPS, 4), "calls_per_s": round(1e6 / us)}
    del wsw
    hx = np.random.default_rng(0).standard_normal((1, Kd)).astype(np.float32)
    ex["down_q6_k_4096x14336"] = gemv_case("q6_k", c2["w_down"], Nd, Kd, hx, 11)
    ex["lm_head_q6_k_128256x4096"] = gemv_case("q6_k", c3["w"], Nh, Kh, c3["x"], 2)
    ex["lm_head_q6_k_r8_128256x4096"] = gemv_case("q6_k_r8", c3["w"], Nh, Kh, c3["x"], 2)
    ex["down_q6_k_r8_4096x14336"] = gemv_case("q6_k_r8", c2["w_down"], Nd, Kd, hx, 11)
    # lm_head (repacked) with the quantisation of x in the same launch
    wh = torch.from_numpy(c3["w"]).to(dev)
    whr = [torch.empty((Nh, qg.q6_k_r8_row_bytes(Kh)), dtype=torch.uint8, device=dev)]
    qg.qgemv_q6_k_repack(wh, Nh, Kh, whr[0])
    del wh
    whr.append(whr[0].clone())
    xh = torch.from_numpy(c3["x"]).to(dev)
    qh, dh, sh_ = qg.act_buffers(1, Kh, dev)
    yh = torch.empty(Nh, dtype=torch.float32, device=dev)
    us = time_kernel(torch, lambda c: qg.qgemv_quantize_gemv(
        qg.QGEMV_FMT_Q6_K_R8, whr[c], Nh, Kh, xh, qh, dh, sh_, yh), 100, 2)
    wb = synth.logical_bytes("q6_k", Nh, Kh)
    ex["lm_head_quantize_gemv_q6_k_r8_128256x4096"] = {
        "us": round(us, 2), "weight_GBps": round(wb / us / 1e3, 1),
        "hbm_frac": round(wb / us / 1e3 / HBM_PEAK_GBPS, 4), "calls_per_s": round(1e6 / us)}
    del whr
    # cache-resident (single 48 MB copy of down, read again and again)
    one = gemv_case("q6_k", c2["w_down"], Nd, Kd, hx, 1)
    ex["down_q6_k_cache_resident_single_copy"] = one

    # quantize and glue kernels
    q, d, s = qg.act_buffers(1, Kgu, dev)
    x = torch.from_numpy(c2["x"]).to(dev)
    # host cost of one call through the Python binding (submission only)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(2000):
        qg.qgemv_quantize_act(x, 1, Kgu, Kgu, q, d, s)
    ex["host_us_per_call_python_binding"] = round((time.perf_counter() - t0) / 2000 * 1e6, 2)
    torch.cuda.synchronize()
    # the same C-ABI call refused at its argument checks (NULL x: nothing is
    # launched): the binding's and the library's own host cost; the rest of
    # a call is the HIP runtime's kernel submission
    ptr_args = (q.data_ptr(), d.data_ptr(), s.data_ptr())
    t0 = time.perf_counter()
    for _ in range(2000):
        qg._lib.qgemv_quantize_act(None, 1, Kgu, Kgu, *ptr_args, None)
    ex["host_us_per_call_refused_before_launch"] = round(
        (time.perf_counter() - t0) / 2000 * 1e6, 2)
    ex["quantize_act_4096"] = kernel_stats(
        torch, lambda c: qg.qgemv_quantize_act(x, 1, Kgu, Kgu, q, d, s), 200, 1)
    gu = torch.randn(Ngu, device=dev)
    q2, d2, s2 = qg.act_buffers(1, Kd, dev)
    ex["silu_mul_quantize_14336"] = kernel_stats(
        torch, lambda c: qg.qgemv_silu_mul_quantize(gu, Kd, q2, d2, s2, None), 200, 1)

    # config 0 / config 1: launch-bound small GEMVs (weights rotated over 1200
    # and 64 copies), launched one by one and as one captured graph
    c0 = synth.config0()
    ex["config0_q4_0_896x896"] = gemv_case("q4_0", c0["w"], 896, 896, c0["x"], 1200)
    ex["config0_q4_0_896x896"]["graph"] = graph_config0(qg, torch, np, dev, c0, 1200)
    ex["config0_q4_0_896x896"]["graph_quantize_in_launch"] = graph_config0_fused(
        qg, torch, np, dev, c0, 1200)
    c1 = synth.config1()
    layer_us = 0.0
    per = {}
    for name, m in c1["mats"].items():
        r = gemv_case("q4_k", m["w"], m["N"], m["K"], m["x"], 64)
        per[name] = r["us"]
        layer_us += r["us"]
    ex["config1_q4_k_layer"] = {"per_matrix_us": per, "sum_us": round(layer_us, 2),
                                "weight_GBps": round(8386560 / layer_us / 1e3, 1),
                                "graph": graph_config1(qg, torch, np, dev, c1, 64),
                                "graph_quantize_in_launch": graph_config1(qg, torch, np, dev, c1, 64,
                                                                          fused=True),
                                "graph_grouped_4_launches": graph_config1(qg, torch, np, dev, c1, 64,
                                                                          grouped=True)}

    # config 4: small-M Q4_K 14336 x 4096
    c4 = synth.config4()
    N4, K4 = c4["N"], c4["K"]
    w4 = [torch.from_numpy(c4["w"]).to(dev)]
    for _ in range(15):
        w4.append(w4[0].clone())
    sm = {}
    for M in SMALL_M_LIST:
        xm = torch.from_numpy(np.ascontiguousarray(c4["x64"][:M])).to(dev)
        qm, dm, smm = qg.act_buffers(M, K4, dev)
        qg.qgemv_quantize_act(xm, M, K4, K4, qm, dm, smm)
        ym = torch.empty((M, N4), dtype=torch.float32, device=dev)
        for vname, v in (("dot4", qg.QGEMV_VARIANT_DOT4), ("mfma", qg.QGEMV_VARIANT_MFMA)):
            us = time_kernel(torch, lambda c: qg.qgemm_q4_k_small_m(
                w4[c], N4, K4, M, qm, dm, smm, ym, v), 50, 16)
            sm[f"M{M}_{vname}_us"] = round(us, 2)
    for M in (1, 2):
        xm = torch.from_numpy(np.ascontiguousarray(c4["x64"][:M])).to(dev)
        qm, dm, smm = qg.act_buffers(M, K4, dev)
        qg.qgemv_quantize_act(xm, M, K4, K4, qm, dm, smm)
        ym = torch.empty((M, N4), dtype=torch.float32, device=dev)
        sm[f"M{M}_auto_us"] = round(time_kernel(torch, lambda c: qg.qgemm_q4_k_small_m(
            w4[c], N4, K4, M, qm, dm, smm, ym, qg.QGEMV_VARIANT_AUTO), 50, 16), 2)
    for M in (8, 64):
        best = min(sm[f"M{M}_dot4_us"], sm[f"M{M}_mfma_us"])
        sm[f"M{M}_weight_GBps"] = round(33030144 / best / 1e3, 1)
        # int8 MACs of the product over the measured time, against the dense int8 peak
        sm[f"M{M}_mfma_int8_TOPS"] = round(2 * M * N4 * K4 / sm[f"M{M}_mfma_us"] / 1e6, 1)
    sm["crossover_M_mfma_faster_from"] = next(
        (M for M in SMALL_M_LIST if sm[f"M{M}_mfma_us"] < sm[f"M{M}_dot4_us"]), None)
    # one weight copy read again and again (33 MB stays in the Infinity Cache):
    # the cache-resident figure, labelled as such
    for M in (8, 64):
        xm = torch.from_numpy(np.ascontiguousarray(c4["x64"][:M])).to(dev)
        qm, dm, smm = qg.act_buffers(M, K4, dev)
        qg.qgemv_quantize_act(xm, M, K4, K4, qm, dm, smm)
        ym = torch.empty((M, N4), dtype=torch.float32, device=dev)
        sm[f"M{M}_mfma_cache_resident_single_copy_us"] = round(time_kernel(
            torch, lambda c: qg.qgemm_q4_k_small_m(w4[0], N4, K4, M, qm, dm, smm, ym,
                                                   qg.QGEMV_VARIANT_MFMA), 50, 1), 2)
    ex["config4_small_m_q4_k_14336x4096"] = sm
    del w4

    # the other weight formats at the gate/up shape (Q8_0 and Q4_0 GEMVs)
    gf = np.random.default_rng(13)
    xf, _ = synth.activation(gf, 1, 4096)
    ex["q8_0_14336x4096"] = gemv_case("q8_0", synth.q8_0_weights(gf, 14336, 4096), 14336,
                                      4096, xf, 8)
    ex["q4_0_14336x4096"] = gemv_case("q4_0", synth.q4_0_weights(gf, 14336, 4096), 14336,
                                      4096, xf, 16)

    # the one-time load repack of the lm_head weights (Q6_K -> Q6_K_R8)
    wh = torch.from_numpy(c3["w"]).to(dev)
    whr = torch.empty((Nh, qg.q6_k_r8_row_bytes(Kh)), dtype=torch.uint8, device=dev)
    us = time_kernel(torch, lambda c: qg.qgemv_q6_k_repack(wh, Nh, Kh, whr), 5, 1)
    wb = synth.logical_bytes("q6_k", Nh, Kh)
    ex["q6_k_repack_128256x4096"] = {"us": round(us, 2),
                                     "read_plus_write_GBps": round(2 * wb / us / 1e3, 1)}
    del wh, whr

    ex["shard8_step"] = shard_step(qg, torch, np, synth, dev, c2, c3)

    # the prefill chunk through the down projection: Q6_K 4096 x 14336
    g6 = np.random.default_rng(11)
    N6, K6 = 4096, 14336
    w6h = synth.q6_k_weights(g6, N6, K6)
    w6 = [torch.from_numpy(w6h).to(dev)]
    for _ in range(10):
        w6.append(w6[0].clone())
    x6, _ = synth.activation(g6, 64, K6)
    sm6 = {}
    for M in SMALL_M_LIST:
        xm = torch.from_numpy(np.ascontiguousarray(x6[:M])).to(dev)
        qm, dm, smm = qg.act_buffers(M, K6, dev)
        qg.qgemv_quantize_act(xm, M, K6, K6, qm, dm, smm)
        ym = torch.empty((M, N6), dtype=torch.float32, device=dev)
        for vname, v in (("dot4", qg.QGEMV_VARIANT_DOT4), ("mfma", qg.QGEMV_VARIANT_MFMA),
                         ("auto", qg.QGEMV_VARIANT_AUTO)):
            us = time_kernel(torch, lambda c: qg.qgemm_q6_k_small_m(
                w6[c], N6, K6, M, qm, dm, smm, ym, v), 50, 11)
            sm6[f"M{M}_{vname}_us"] = round(us, 2)
    wb6 = synth.logical_bytes("q6_k", N6, K6)
    for M in (8, 64):
        sm6[f"M{M}_mfma_weight_GBps"] = round(wb6 / sm6[f"M{M}_mfma_us"] / 1e3, 1)
        sm6[f"M{M}_mfma_int8_TOPS"] = round(2 * M * N6 * K6 / sm6[f"M{M}_mfma_us"] / 1e6, 1)
    sm6["crossover_M_mfma_faster_from"] = next(
        (M for M in SMALL_M_LIST if sm6[f"M{M}_mfma_us"] < sm6[f"M{M}_dot4_us"]), None)
    ex["small_m_q6_k_4096x14336"] = sm6
    del w6

    # a prefill chunk through the lm_head: Q6_K 128256 x 4096 (a wide matrix)
    wl = [torch.from_numpy(c3["w"]).to(dev)]
    wl.append(wl[0].clone())
    Nl, Kl = c3["N"], c3["K"]
    xl, _ = synth.activation(np.random.default_rng(12), 64, Kl)
    sml = {}
    for M in (8, 64):
        xm = torch.from_numpy(np.ascontiguousarray(xl[:M])).to(dev)
        qm, dm, smm = qg.act_buffers(M, Kl, dev)
        qg.qgemv_quantize_act(xm, M, Kl, Kl, qm, dm, smm)
        ym = torch.empty((M, Nl), dtype=torch.float32, device=dev)
        us = time_kernel(torch, lambda c: qg.qgemm_q6_k_small_m(
            wl[c], Nl, Kl, M, qm, dm, smm, ym, qg.QGEMV_VARIANT_MFMA), 10, 2)
        wbl = synth.logical_bytes("q6_k", Nl, Kl)
        sml[f"M{M}_mfma_us"] = round(us, 2)
        sml[f"M{M}_mfma_weight_GBps"] = round(wbl / us / 1e3, 1)
        sml[f"M{M}_mfma_int8_TOPS"] = round(2 * M * Nl * Kl / us / 1e6, 1)
        del ym
    ex["small_m_q6_k_lm_head_128256x4096"] = sml
    del wl

    # plain device copy: the achievable HBM figure beside the datasheet peak
    a = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    us = time_kernel(torch, lambda c: b.copy_(a), 10, 1)
    ex["device_copy_1GiB_GBps_read_plus_write"] = round(2 * (1 << 30) / us / 1e3, 1)
    return ex


def shard_step(qg, torch, np, synth, dev, c2, c3, G=8, steps=200):
    """One GPU's share of the decode step split over G GPUs, kernels only:
    gate|up by rows (N/G gate and N/G up rows, SwiGLU and the requantisation
    local), down by K at super-block boundaries (a K/G slice, giving a partial
    y to be all-reduced), lm_head by rows.  The collectives are not run."""
    Kgu, Kd, Nd = c2["K_gu"], c2["K_down"], c2["N_down"]
    Nh, Kh = c3["N"], c3["K"]
    nh, Kd8, Nh8 = Kd // G, Kd // G, Nh // G
    g = np.random.default_rng(17)
    fmt_r8 = qg.QGEMV_FMT_Q6_K_R8

    def copies(w_host, N, K, n, r8):
        w0 = torch.from_numpy(w_host).to(dev)
        if r8:
            wr = torch.empty((N, qg.q6_k_r8_row_bytes(K)), dtype=torch.uint8, device=dev)
            qg.qgemv_q6_k_repack(w0, N, K, wr)
            w0 = wr
        return [w0] + [w0.clone() for _ in range(n - 1)]

    # copies so that each rotation covers at least ~512 MB
    wgu = copies(synth.q4_k_weights(g, 2 * nh, Kgu), 2 * nh, Kgu, 64, False)
    wdn = copies(synth.q6_k_weights(g, Nd, Kd8), Nd, Kd8, 80, True)
    whd = copies(synth.q6_k_weights(g, Nh8, Kh), Nh8, Kh, 10, True)
    x_ffn = torch.from_numpy(np.ascontiguousarray(c2["x"].reshape(-1))).to(dev)
    x_head = torch.from_numpy(np.ascontiguousarray(c3["x"].reshape(-1))).to(dev)
    q1, d1, s1 = qg.act_buffers(1, Kgu, dev)
    q2, d2, s2 = qg.act_buffers(1, Kd8, dev)
    q3, d3, s3 = qg.act_buffers(1, Kh, dev)
    y = torch.empty(Nd, dtype=torch.float32, device=dev)
    logits = torch.empty(Nh8, dtype=torch.float32, device=dev)

    def step(i):
        qg.qgemv_quantize_q4_k_swiglu(wgu[i % len(wgu)], nh, Kgu, x_ffn, q1, d1, s1,
                                      q2, d2, s2, None, None)
        qg.qgemv_q6_k_r8(wdn[i % len(wdn)], Nd, Kd8, q2, d2, s2, y)
        qg.qgemv_quantize_gemv(fmt_r8, whd[i % len(whd)], Nh8, Kh, x_head, q3, d3, s3,
                               logits)

    for i in range(20):
        step(i)
    res = []
    for _ in range(5):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for i in range(steps):
            step(i)
        b.record()
        torch.cuda.synchronize()
        res.append(a.elapsed_time(b) * 1e3 / steps)
    out = {"gate_up_swiglu": kernel_stats(torch, lambda c: qg.qgemv_quantize_q4_k_swiglu(
               wgu[c], nh, Kgu, x_ffn, q1, d1, s1, q2, d2, s2, None, None), 100, len(wgu)),
           "down_r8": kernel_stats(torch, lambda c: qg.qgemv_q6_k_r8(
               wdn[c], Nd, Kd8, q2, d2, s2, y), 100, len(wdn)),
           "lm_head_r8": kernel_stats(torch, lambda c: qg.qgemv_quantize_gemv(
               fmt_r8, whd[c], Nh8, Kh, x_head, q3, d3, s3, logits), 100, len(whd))}
    us = float(np.median(res))
    wb = (synth.logical_bytes("q4_k", 2 * nh, Kgu) + synth.logical_bytes("q6_k", Nd, Kd8) +
          synth.logical_bytes("q6_k", Nh8, Kh))
    del wgu, wdn, whd
    return {"gpus": G, "shapes": {"gate_up": [2 * nh, Kgu], "down": [Nd, Kd8],
                                  "lm_head": [Nh8, Kh]},
            "per_kernel": out,
            "step_us": round(us, 2), "weight_bytes": wb,
            "weight_GBps": round(wb / us / 1e3, 1),
            "hbm_frac": round(wb / us / 1e3 / HBM_PEAK_GBPS, 4),
            "not_timed": "the 16 KB all-reduce of down's partial y and the logits gather"}


def cpu_baseline(np, synth, c2, c3, seconds, step_wbytes):
    """The oracle (single-threaded plain C) over whole steps of the same
    workload, repeated until `seconds` of CPU time have passed (at least once)."""
    import oracle
    Ngu, Kgu, Nd, Kd = c2["N_gu"], c2["K_gu"], c2["N_down"], c2["K_down"]
    Nh, Kh = c3["N"], c3["K"]
    times = []
    t_all = time.perf_counter()
    while True:
        t = time.perf_counter()
        q, d, s = oracle.quantize_act(c2["x"])
        gu, _ = oracle.gemv("q4_k", c2["w_gu"], Ngu, Kgu, q, d, s)
        h = oracle.silu_mul(gu.astype(np.float32))
        q2, d2, s2 = oracle.quantize_act(h.astype(np.float32)[None])
        oracle.gemv("q6_k", c2["w_down"], Nd, Kd, q2, d2, s2)
        q3, d3, s3 = oracle.quantize_act(c3["x"])
        oracle.gemv("q6_k", c3["w"], Nh, Kh, q3, d3, s3)
        times.append(time.perf_counter() - t)
        if time.perf_counter() - t_all >= seconds:
            break
    per = float(np.median(times))
    return {"value": round(step_wbytes / per / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "ms_per_step": round(per * 1e3, 1),
            "sample": f"{len(times)} whole steps of the same workload, single thread, "
                      f"median step time",
            "parallel": oracle_parallel(np, c2, c3, step_wbytes),
            "per_kernel": oracle_rates(np, synth, c2, c3)}


def oracle_parallel(np, c2, c3, step_wbytes, seconds=3.0):
    """The same whole steps with each GEMV's rows split into equal ranges
    over host threads (rows are independent; the oracle's C code releases
    the interpreter lock while it runs), at most 16 threads."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    # at most 16 threads: the host CPU share that goes with one GPU on the
    # machines this runs on, whatever the affinity mask shows
    T = max(1, min(16, avail))
    Ngu, Kgu, Nd, Kd = c2["N_gu"], c2["K_gu"], c2["N_down"], c2["K_down"]
    Nh, Kh = c3["N"], c3["K"]

    def gemv(pool, fmt, w, N, K, q, d, s):
        b = np.linspace(0, N, T + 1).astype(np.int64)
        futs = [pool.submit(oracle.gemv, fmt, w, N, K, q, d, s, (int(b[i]), int(b[i + 1] - b[i])))
                for i in range(T)]
        return np.concatenate([f.result()[0] for f in futs])

    times = []
    with ThreadPoolExecutor(T) as pool:
        t_all = time.perf_counter()
        while True:
            t = time.perf_counter()
            q, d, s = oracle.quantize_act(c2["x"])
            gu = gemv(pool, "q4_k", c2["w_gu"], Ngu, Kgu, q, d, s)
            h = oracle.silu_mul(gu.astype(np.float32))
            q2, d2, s2 = oracle.quantize_act(h.astype(np.float32)[None])
            gemv(pool, "q6_k", c2["w_down"], Nd, Kd, q2, d2, s2)
            q3, d3, s3 = oracle.quantize_act(c3["x"])
            gemv(pool, "q6_k", c3["w"], Nh, Kh, q3, d3, s3)
            times.append(time.perf_counter() - t)
            if time.perf_counter() - t_all >= seconds:
                break
    per = float(np.median(times))
    return {"value": round(step_wbytes / per / 1e9, 4), "unit": "GB/s", "cores": T,
            "cores_in_affinity_mask": avail,
            "ms_per_step": round(per * 1e3, 1),
            "sample": f"{len(times)} whole steps, each GEMV's rows split over {T} threads "
                      f"(capped at 16, the host CPU share of one GPU; {avail} in the affinity "
                      f"mask), median step time"}


def oracle_rates(np, synth, c2, c3, seconds=0.3):
    """The oracle beside each per-kernel GPU figure of `extra`: the same
    shapes, on a bounded sample of weight rows (the first 512, or 64 for the
    small-M products), each repeated for at least `seconds`; single thread."""
    import oracle
    g = np.random.default_rng(23)
    out = {}

    def per_call(fn):
        n, t0 = 0, time.perf_counter()
        while True:
            fn()
            n += 1
            t = time.perf_counter() - t0
            if t >= seconds:
                return t / n

    def gemv_rate(name, fmt, w, N, K, x, S=512):
        q, d, s = oracle.quantize_act(x)
        t = per_call(lambda: oracle.gemv(fmt, w, N, K, q, d, s, rows=(0, S)))
        out[name] = {"weight_GBps": round(synth.logical_bytes(fmt, S, K) / t / 1e9, 4),
                     "sample_rows": S}

    def gemm_rate(name, fmt, w, N, K, x, S=64):
        q, d, s = oracle.quantize_act(x)
        t = per_call(lambda: oracle.gemm(fmt, w, N, K, q, d, s, rows=(0, S)))
        M = x.shape[0]
        out[name] = {"weight_GBps": round(synth.logical_bytes(fmt, S, K) / t / 1e9, 4),
                     "int8_GOPS": round(2 * M * S * K / t / 1e9, 4), "sample_rows": S}

    hx = np.random.default_rng(0).standard_normal((1, c2["K_down"])).astype(np.float32)
    gemv_rate("gate_up_q4_k_28672x4096", "q4_k", c2["w_gu"], c2["N_gu"], c2["K_gu"], c2["x"])
    gemv_rate("down_q6_k_4096x14336", "q6_k", c2["w_down"], c2["N_down"], c2["K_down"], hx)
    gemv_rate("lm_head_q6_k_128256x4096", "q6_k", c3["w"], c3["N"], c3["K"], c3["x"])
    x4k, _ = synth.activation(g, 1, 4096)
    gemv_rate("q8_0_14336x4096", "q8_0", synth.q8_0_weights(g, 512, 4096), 512, 4096, x4k)
    gemv_rate("q4_0_14336x4096", "q4_0", synth.q4_0_weights(g, 512, 4096), 512, 4096, x4k)
    out["quantize_act_4096_us"] = round(per_call(lambda: oracle.quantize_act(c2["x"])) * 1e6, 1)
    gu = g.standard_normal(2 * c2["K_down"]).astype(np.float32)
    out["silu_mul_quantize_14336_us"] = round(per_call(lambda: oracle.quantize_act(
        oracle.silu_mul(gu).astype(np.float32)[None])) * 1e6, 1)
    w4 = synth.q4_k_weights(g, 64, 4096)
    x64, _ = synth.activation(g, 64, 4096)
    w6 = synth.q6_k_weights(g, 64, 14336)
    x64b, _ = synth.activation(g, 64, 14336)
    for M in (8, 64):
        gemm_rate(f"small_m_q4_k_14336x4096_M{M}", "q4_k", w4, 64, 4096,
                  np.ascontiguousarray(x64[:M]))
        gemm_rate(f"small_m_q6_k_4096x14336_M{M}", "q6_k", w6, 64, 14336,
                  np.ascontiguousarray(x64b[:M]))
    return out


if __name__ == "__main__":
    main()
