#!/usr/bin/env python3
"""Benchmark of the FP8 delayed-scaling Linear on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input,
the fwd+bwd Linear at 4096 hidden with M = 16384 tokens (X, W, dY bf16; HYBRID
recipe: E4M3 forward, E5M2 gradients; amax history 16, window max, margin 0):

  cast X (fused amax)  ->  cast W (+ transposed bytes)  ->  Y = Xq Wq  ->
  cast dY  ->  dX = dYq Wq^T  ->  dW = Xq^T dYq  ->  scale update of 3 histories

`value` is the step's GEMM work (3 x 2 M N K flop) over the measured time of the
whole step (casts and scale update included), in TFLOP/s, timed with events at
the step boundaries only.  Inputs are resident in HBM before timing; four input
sets are rotated so that the 256 MB Infinity Cache cannot hold a step's working
set.  Per-kernel times (the roofline figures) come from HIP events on the
stream the library launches on around K back-to-back launches of each call of
the step (inputs rotated over the sets), run just before the timed region.

The forward GEMM runs on gfx950's FP8 matrix instructions, the dX and dW GEMMs
on the exact F16-widened datapath (DelayedScalingLinear's defaults).  The line
also carries context figures that are not `value`: each GEMM on the other
datapath (`other_datapath_tflops`), the 2^30-element stress
casts (`cast_stress`), per-token / per-channel / current scaling of the same
Linear's forward (`finer_scaling`), the fused AdamW step on the 4096 x 4096
weight that also writes the next forward's FP8 weights (`optimizer`, against
the unfused update plus weight cast), and `configs`, the throughput of the other workloads
(forward-only 4096 Linear at M = 8192, the decoder-layer projections at
M = 8192, 512 small Linears).

Prints one JSON line.  `--gpus N` with N > 1 is refused: the benchmark measures
one GPU.  `--copy-calib` only runs device copies of known size (the reference
for the HBM byte counters, see profiles/).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

M_TOK, K_IN, N_OUT = 16384, 4096, 4096
HIST_LEN = 16
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 MFMA
PEAK_F16_TFLOPS = 2500.0   # MI355X dense F16 MFMA (the instruction of the exact datapath)
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E
N_SETS = 4
CPU_SAMPLE_ROWS = 8192
CPU_CAST_SAMPLE = 1 << 24   # elements of the 2^30 stress tensor cast by the oracle
CPU_GEMM_ROWS = 512         # rows of the forward 4096 Linear's GEMM computed by the oracle
KERNEL_SOURCES = ["delayed_scaling_gemm_amd/csrc/gemm_kernel.h",
                  "delayed_scaling_gemm_amd/csrc/device_common.h"]
TRAFFIC_FILE = "profiles/gemm_linear_4096_m16384_traffic.txt"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stress", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-configuration throughput report")
    ap.add_argument("--no-optimizer", action="store_true",
                    help="skip the fused AdamW + weight-cast measurement")
    ap.add_argument("--no-finer", action="store_true",
                    help="skip the per-token / per-channel / current scaling measurement")
    ap.add_argument("--no-fp8-path", action="store_true",
                    help="skip the context timing of the FP8-MFMA datapath")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MIB",
                    help="only run 5 device-to-device copies of MIB MiB and exit")
    return ap.parse_args()


def _code_only(src: str) -> str:
    """C++ source without its comments, blank lines and trailing blanks (the GEMM
    sources hold no string literal that contains a comment marker)."""
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return "\n".join(line.rstrip() for line in src.splitlines() if line.strip())


def kernel_source_hash() -> str:
    """Hash of the GEMM kernel's code: a change to its comments alone keeps the
    counter figures taken on it."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None
    when there is none or it was taken on another version of the kernel source."""
    path = os.path.join(ROOT, TRAFFIC_FILE)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    key = f"{kernel}_hbm_bytes_per_launch"
    return float(fields[key]) if key in fields else None


def cpu_baseline(xb, wb, dyb, rows=CPU_SAMPLE_ROWS):
    """The oracle's training step on a row sample of the same workload (CPU)."""
    from oracle import bf16 as obf16
    from oracle import fp8 as ofp8
    from oracle import linear as olinear
    from oracle.scaling import ScalingState

    states = {"x": ScalingState(ofp8.E4M3, HIST_LEN), "w": ScalingState(ofp8.E4M3, HIST_LEN),
              "dy": ScalingState(ofp8.E5M2, HIST_LEN)}
    x = obf16.widen(xb[:rows])
    w = obf16.widen(wb)
    dy = obf16.widen(dyb[:rows])
    t0 = time.perf_counter()
    olinear.train_step(x, w, dy, states, 0, 0)
    dt = time.perf_counter() - t0
    flops = 3 * 2 * rows * K_IN * N_OUT
    try:
        import threadpoolctl
        blas = max((p.get("num_threads", 0) for p in threadpoolctl.threadpool_info()), default=0)
    except Exception:  # threadpoolctl is optional
        blas = 0
    cores = len(os.sched_getaffinity(0))
    return {
        "value": round(flops / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": max(blas, 1) if blas else cores,
        "kind": "oracle",
        "sample": f"one oracle fwd+bwd step on the first {rows} of {M_TOK} token rows: casts of "
                  f"X[{rows}x{K_IN}], W[{K_IN}x{N_OUT}], dY[{rows}x{N_OUT}] (numpy, one thread) "
                  f"and the three exact fp64 GEMMs of that sample (BLAS threads: {blas or 'n/a'}, "
                  f"usable cores {cores}); {dt:.2f} s",
        "seconds": round(dt, 3),
    }


def cpu_other(workloads, cast_sample):
    """The oracle on bounded samples of two more workloads (CPU, one thread for
    the numpy casts, BLAS threads for the fp64 GEMM): the amax + E4M3 cast of the
    first 2^24 elements of the 2^30-element stress tensor (3 algorithmic bytes
    per element), and the exact GEMM of the first 512 token rows of the forward
    4096 Linear (8192 x 4096 x 4096, E4M3 both; the rows cast by the oracle)."""
    from oracle import amax as oamax
    from oracle import bf16 as obf16
    from oracle import fp8 as ofp8
    from oracle import gemm as ogemm

    out = {}
    if cast_sample is not None:
        x = obf16.widen(cast_sample)
        t0 = time.perf_counter()
        oamax.amax(x)
        ofp8.cast(x, np.float32(1.0), ofp8.E4M3)
        dt = time.perf_counter() - t0
        out["amax_cast_2e30_stress"] = {
            "sample": f"first {cast_sample.size} elements, amax + cast to E4M3 at scale 1",
            "seconds": round(dt, 3), "GB/s": round(3.0 * cast_sample.size / dt / 1e9, 3)}
    xb, wb = workloads.forward_4096()
    x = obf16.widen(xb[:CPU_GEMM_ROWS])
    w = obf16.widen(wb)
    xs, ws = np.float32(448.0) / oamax.amax(x), np.float32(448.0) / oamax.amax(w)
    cx, _ = ofp8.cast(x, xs, ofp8.E4M3)
    cw, _ = ofp8.cast(w, ws, ofp8.E4M3)
    t0 = time.perf_counter()
    acc, _ = ogemm.gemm_exact(cx, ofp8.E4M3, ogemm.OP_N, cw, ofp8.E4M3, ogemm.OP_N)
    ogemm.dequant_to_bf16(acc, xs, ws)
    dt = time.perf_counter() - t0
    flop = 2.0 * CPU_GEMM_ROWS * w.shape[0] * w.shape[1]
    out["gemm_forward_4096"] = {
        "sample": f"{CPU_GEMM_ROWS} of 8192 rows, exact fp64 GEMM (with sum|ab|) and BF16 dequant",
        "seconds": round(dt, 3), "TFLOP/s": round(flop / dt / 1e12, 6)}
    return out


def copy_calibration(torch, mib: int):
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calib_bytes": n, "copies": 5}), flush=True)


def time_launches(torch, stream, fn, iters, dsg=None):
    """Average time of `iters` back-to-back calls of `fn`.  With `dsg`, the
    library calls `fn` makes are prepared once (dsg.prepare) and replayed, so
    that the binding's per-call checks do not pace launches shorter than them."""
    if dsg is not None:
        fn = dsg.prepare(fn)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(iters):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def stress_cast(torch, dsg, workloads, dev, iters=10):
    """Standalone amax+cast of 2^30 bf16 elements to E4M3 and E5M2 (3 B/element),
    the E4M3 cast with its health counts, and the amax alone."""
    n = 1 << 30
    print("[bench] stress cast 2^30", file=sys.stderr, flush=True)
    bits = workloads.big_cast_input(n)
    x = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
    sample = bits[:CPU_CAST_SAMPLE].copy()  # for the oracle's timing on the CPU
    del bits
    q = torch.empty(n, dtype=torch.uint8, device=dev)
    s = torch.ones(1, dtype=torch.float32, device=dev)
    am = torch.zeros(1, dtype=torch.float32, device=dev)
    sat = torch.zeros(1, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream()
    out = {}
    for fmt, name in ((dsg.E4M3, "e4m3"), (dsg.E5M2, "e5m2")):
        # timed: the accumulating call (the cast kernel alone; the amax and the
        # count combine over the repeats); reported counts: one resetting call
        dsg.fp8ds_cast_acc(x, fmt, s, q, None, None, am, sat)
        ms = time_launches(torch, stream,
                           lambda: dsg.fp8ds_cast_acc(x, fmt, s, q, None, None, am, sat), iters, dsg)
        dsg.fp8ds_cast(x, fmt, s, q, None, None, am, sat)
        gbps = 3.0 * n / (ms * 1e-3) / 1e9
        out[name] = {"ms": round(ms, 4), "GB/s": round(gbps, 1),
                     "frac_hbm": round(gbps / PEAK_HBM_GBPS, 4), "saturated": int(sat.item())}
    counts = torch.zeros(dsg.HEALTH_COUNTS, dtype=torch.int64, device=dev)
    dsg.fp8ds_cast_health(x, dsg.E4M3, s, q, counts, amax=am)
    ms = time_launches(torch, stream,
                       lambda: dsg.fp8ds_cast_health(x, dsg.E4M3, s, q, counts, amax=am), iters, dsg)
    gbps = 3.0 * n / (ms * 1e-3) / 1e9
    out["e4m3_health"] = {"ms": round(ms, 4), "GB/s": round(gbps, 1),
                          "frac_hbm": round(gbps / PEAK_HBM_GBPS, 4),
                          "counts": dict(zip(dsg.HEALTH_NAMES, counts.cpu().tolist()))}
    ms = time_launches(torch, stream, lambda: dsg.fp8ds_amax(x, am), iters, dsg)
    out["amax"] = {"ms": round(ms, 4), "GB/s": round(2.0 * n / (ms * 1e-3) / 1e9, 1),
                   "frac_hbm": round(2.0 * n / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}
    del x, q
    torch.cuda.empty_cache()
    return out, sample


def optimizer_report(torch, dsg, workloads, dev, rows=4096, cols=4096, iters=10):
    """The fused AdamW step on the benchmarked Linear's [4096 x 4096] fp32 master
    weights with its BF16 dW, writing Wq and Wq^T for the next forward (28
    algorithmic bytes per element: read w, m, v, g = 14; write w, m, v, q, q_t =
    14), against the unfused pair: the update alone (26 B) and the transposing
    cast of the fp32 weights (6 B)."""
    print("[bench] fused AdamW 4096x4096", file=sys.stderr, flush=True)
    w, m, v, gbits = workloads.adamw_state(rows, cols)
    n = rows * cols
    wd, md, vd = (torch.from_numpy(a).to(dev) for a in (w, m, v))
    g = torch.from_numpy(gbits.view(np.int16)).to(dev).view(torch.bfloat16)
    q = torch.empty(n, dtype=torch.uint8, device=dev)
    qt = torch.empty(n, dtype=torch.uint8, device=dev)
    s = torch.tensor([448.0 / 0.1], device=dev)
    su = torch.zeros(1, device=dev)
    am = torch.zeros(1, device=dev)
    sat = torch.zeros(1, dtype=torch.int64, device=dev)
    ga = torch.tensor([float(np.abs((gbits.astype(np.uint32) << 16).view(np.float32)).max())],
                      device=dev)
    stream = torch.cuda.current_stream()
    hp = (1e-4, 0.9, 0.999, 1e-8, 0.01)

    def fused():
        dsg.fp8ds_adamw(wd, g, md, vd, *hp, 10, grad_amax=ga, fmt=dsg.E4M3, scale=s, q=q, q_t=qt,
                        scale_used=su, amax=am, sat_count=sat)

    def update_only():
        dsg.fp8ds_adamw(wd, g, md, vd, *hp, 10, grad_amax=ga)

    def cast_w():
        dsg.fp8ds_cast(wd, dsg.E4M3, s, q, qt, su, am, sat)

    out = {"shape": [rows, cols], "grad": "bf16", "fmt": "e4m3"}
    t = {}
    for name, fn in (("fused", fused), ("update_only", update_only), ("cast_w_t_fp32", cast_w)):
        fn()
        t[name] = time_launches(torch, stream, fn, iters, dsg)
    alg = {"fused": 28.0, "update_only": 26.0, "cast_w_t_fp32": 6.0}
    for name, ms in t.items():
        gbps = alg[name] * n / (ms * 1e-3) / 1e9
        out[name] = {"ms": round(ms, 4), "GB/s": round(gbps, 1),
                     "frac_hbm": round(gbps / PEAK_HBM_GBPS, 4)}
    unfused = t["update_only"] + t["cast_w_t_fp32"]
    out["unfused_ms"] = round(unfused, 4)
    out["fused_speedup"] = round(unfused / t["fused"], 3)
    del wd, md, vd, g, q, qt
    torch.cuda.empty_cache()
    return out


def finer_report(torch, dsg, x, w, dy=None, iters=10):
    """Finer-grained scaling on the benchmarked Linear's forward operands: the
    per-token cast of X [M x K] (a scale per row; 3 B/element, read once), the
    per-channel cast of W^T [N x K] (a scale per output channel), the per-tensor
    current cast of X (amax pass, then the cast: 5 B/element), the forward
    GEMM with per-row x per-column dequant factors (2 M N K flop), and MXFP8:
    the block casts of X and W^T, the MX forward GEMM and a whole MX training
    step."""
    print("[bench] finer scaling: per-token / per-channel / current", file=sys.stderr, flush=True)
    dev = x.device
    M, K = x.shape
    N = w.shape[1]
    wt = w.t().contiguous()  # [N x K]: one row per output channel
    xq = torch.empty(M, K, dtype=torch.uint8, device=dev)
    wq = torch.empty(N, K, dtype=torch.uint8, device=dev)
    sx, ix, ax = (torch.empty(M, dtype=torch.float32, device=dev) for _ in range(3))
    sw, iw, aw = (torch.empty(N, dtype=torch.float32, device=dev) for _ in range(3))
    s1, i1, a1 = (torch.empty(1, dtype=torch.float32, device=dev) for _ in range(3))
    y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    amax_y = torch.zeros(1, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    calls = {
        "per_token_cast_x": (lambda: dsg.fp8ds_cast_rowwise(x, dsg.E4M3, 0, xq, sx, ix, ax),
                             3.0 * M * K),
        "per_channel_cast_wt": (lambda: dsg.fp8ds_cast_rowwise(wt, dsg.E4M3, 0, wq, sw, iw, aw),
                                3.0 * N * K),
        "current_cast_x": (lambda: dsg.fp8ds_cast_current(x, dsg.E4M3, 0, xq, s1, a1,
                                                          scale_inv=i1), 5.0 * M * K),
    }
    out = {"shape": [M, K, N], "fmt": "e4m3"}
    for name, (fn, nbytes) in calls.items():
        fn()
        ms = time_launches(torch, stream, fn, iters, dsg)
        gbps = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"ms": round(ms, 4), "GB/s": round(gbps, 1),
                     "frac_hbm": round(gbps / PEAK_HBM_GBPS, 4)}
    dsg.fp8ds_cast_rowwise(x, dsg.E4M3, 0, xq, sx, ix, ax)

    def gemm():
        dsg.fp8ds_gemm_rowcol(dsg.OP_N, dsg.OP_T, M, N, K, xq, dsg.E4M3, K, ix, wq, dsg.E4M3, K,
                              iw, y, N, amax_y)

    gemm()
    ms = time_launches(torch, stream, gemm, iters, dsg)
    tflops = 2.0 * M * N * K / (ms * 1e-3) / 1e12
    out["rowcol_gemm_fwd_nt"] = {"ms": round(ms, 4), "TFLOP/s": round(tflops, 1),
                                 "frac_fp8_peak": round(tflops / PEAK_FP8_TFLOPS, 4)}
    # MXFP8: blocks of 32 along K with E8M0 scales (3 + 1/32 B per element cast)
    xs = torch.empty(M, K // 32, dtype=torch.uint8, device=dev)
    ws = torch.empty(N, K // 32, dtype=torch.uint8, device=dev)
    for name, (fn, nbytes) in {
            "mx_cast_x": (lambda: dsg.fp8ds_cast_mx(x, dsg.E4M3, xq, xs), (3 + 1 / 32) * M * K),
            "mx_cast_wt": (lambda: dsg.fp8ds_cast_mx(wt, dsg.E4M3, wq, ws), (3 + 1 / 32) * N * K),
    }.items():
        fn()
        ms = time_launches(torch, stream, fn, iters, dsg)
        gbps = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"ms": round(ms, 4), "GB/s": round(gbps, 1),
                     "frac_hbm": round(gbps / PEAK_HBM_GBPS, 4)}

    def mx_gemm():
        dsg.fp8ds_gemm_mx(M, N, K, xq, dsg.E4M3, K, xs, K // 32, wq, dsg.E4M3, K, ws, K // 32, y, N,
                          amax_y)

    mx_gemm()
    ms = time_launches(torch, stream, mx_gemm, iters, dsg)
    tflops = 2.0 * M * N * K / (ms * 1e-3) / 1e12
    out["mx_gemm_fwd_nt"] = {"ms": round(ms, 4), "TFLOP/s": round(tflops, 1),
                             "frac_fp8_peak": round(tflops / PEAK_FP8_TFLOPS, 4)}

    def mx_gemm_fp8():  # context: gfx950's block-scaled FP8 MFMA (not the exact datapath)
        dsg.fp8ds_gemm_mx(M, N, K, xq, dsg.E4M3, K, xs, K // 32, wq, dsg.E4M3, K, ws, K // 32, y, N,
                          amax_y, mma=dsg.MMA_FP8)

    mx_gemm_fp8()
    ms = time_launches(torch, stream, mx_gemm_fp8, iters, dsg)
    tflops = 2.0 * M * N * K / (ms * 1e-3) / 1e12
    out["mx_gemm_fwd_nt_fp8_mma"] = {"ms": round(ms, 4), "TFLOP/s": round(tflops, 1),
                                     "frac_fp8_peak": round(tflops / PEAK_FP8_TFLOPS, 4)}
    del wt, xq, wq, y, xs, ws
    if dy is not None:
        out["mx_training_step"] = mx_step_report(torch, dsg, x, w, dy, iters)
    return out


def mx_step_report(torch, dsg, x, w, dy, iters):
    """A whole MXFP8 training step of the Linear (MXLinear): one cast per tensor
    with its transposed copy (X, W E4M3; dY E5M2), then Y = X W, dX = dY W^T and
    dW = X^T dY, all as NT MX GEMMs (blocks along K)."""
    from delayed_scaling_gemm_amd.linear import MXLinear

    M, K = x.shape
    lin = MXLinear(device=x.device)
    stream = torch.cuda.current_stream()
    lin.step(x, w, dy)
    ms = time_launches(torch, stream, lambda: lin.step(x, w, dy), iters)
    cast_ms = time_launches(torch, stream, lambda: lin._cast(0, "x", x, None), iters, dsg)
    res = {"ms": round(ms, 4), "TFLOP/s": round(6.0 * M * w.shape[1] * K / (ms * 1e-3) / 1e12, 1),
           "cast_x_with_transpose_ms": round(cast_ms, 4),
           "cast_x_with_transpose_GB/s": round(4.0625 * M * K / (cast_ms * 1e-3) / 1e9, 1)}
    del lin
    torch.cuda.empty_cache()
    return res


def configs_report(torch, dsg, workloads, dev, iters=5):
    """Throughput of the other workloads, one Linear at a time: the forward-only
    4096 Linear (M=8192, history 1024), the decoder-layer projections (M=8192,
    fwd+bwd; v and o share the k and q shapes, up shares gate's) and the batch of
    512 small Linears.  Step times include every launch of the step (casts, GEMMs,
    scale update); per-GEMM rates time each GEMM call alone on the step's operands.
    The launches are prepared once (dsg.prepare): on these shorter steps the
    binding's per-call argument checks would otherwise take longer than the
    kernels.  A Linear alternates its accumulator sets by step parity, so its steps
    are recorded in pairs."""
    from delayed_scaling_gemm_amd import E4M3, E5M2, OP_N, OP_T, fp8ds_gemm
    from delayed_scaling_gemm_amd.linear import BatchedDelayedScalingLinear, DelayedScalingLinear

    stream = torch.cuda.current_stream()

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(
            torch.bfloat16)

    def tf(flop, ms):
        return round(flop / (ms * 1e-3) / 1e12, 1)

    def step_ms_of(fn, reps):
        pair = dsg.prepare(lambda: (fn(), fn()))
        return time_launches(torch, stream, pair, reps) / 2

    def call_ms(fn, reps):
        return time_launches(torch, stream, dsg.prepare(fn), reps)

    reps = max(iters, 20)
    out = {}
    print("[bench] configs: forward 4096", file=sys.stderr, flush=True)
    xb, wb = workloads.forward_4096()
    x, w = to_dev(xb), to_dev(wb)
    M, K = x.shape
    N = w.shape[1]
    lin = DelayedScalingLinear(hist_len=1024, device=dev)
    lin.step(x, w)
    step_ms = step_ms_of(lambda: lin.step(x, w), reps)
    b, su = lin._bufs, lin.scale_used
    g_ms = call_ms(lambda: fp8ds_gemm(
        OP_N, OP_T, M, N, K, b["xq"], E4M3, K, su[0:1], b["wqt"], E4M3, K, su[1:2], b["y"], N,
        lin.amax_y, mma=lin.fwd_datapath(K)), reps)
    out["forward_4096_m8192"] = {"step_ms": round(step_ms, 4), "gemm_ms": round(g_ms, 4),
                                 "gemm_tflops": tf(2 * M * N * K, g_ms),
                                 "gemm_frac_fp8_peak": round(tf(2 * M * N * K, g_ms) /
                                                             PEAK_FP8_TFLOPS, 4)}
    del x, w, lin, b
    proj = {}
    for name in ("q_proj", "k_proj", "gate_proj", "down_proj"):
        print(f"[bench] configs: {name}", file=sys.stderr, flush=True)
        xb, wb, dyb = workloads.llama_tensors(name, 0)
        x, w, dy = to_dev(xb), to_dev(wb), to_dev(dyb)
        M, K = x.shape
        N = w.shape[1]
        lin = DelayedScalingLinear(hist_len=16, device=dev)
        lin.step(x, w, dy)
        step_ms = step_ms_of(lambda: lin.step(x, w, dy), reps)
        b, su = lin._bufs, lin.scale_used
        calls = {
            "fwd_nt": lambda: fp8ds_gemm(OP_N, OP_T, M, N, K, b["xq"], E4M3, K, su[0:1], b["wqt"],
                                         E4M3, K, su[1:2], b["y"], N, lin.amax_y,
                                         mma=lin.fwd_datapath(K)),
            "dgrad_nt": lambda: fp8ds_gemm(OP_N, OP_T, M, K, N, b["dyq"], E5M2, N, su[2:3],
                                           b["wq"], E4M3, N, su[1:2], b["dx"], K),
            "wgrad_tn": lambda: fp8ds_gemm(OP_T, OP_N, K, N, M, b["xq"], E4M3, K, su[0:1],
                                           b["dyq"], E5M2, N, su[2:3], b["dw"], N),
        }
        gem = {n: tf(2 * M * N * K, call_ms(fn, reps)) for n, fn in calls.items()}
        proj[name] = {"M": M, "in": K, "out": N, "step_ms": round(step_ms, 4),
                      "step_tflops": tf(6 * M * N * K, step_ms), "gemm_tflops": gem,
                      "step_frac_fp8_peak": round(tf(6 * M * N * K, step_ms) / PEAK_FP8_TFLOPS, 4)}
        del x, w, dy, lin, b
    out["decoder_projections_m8192"] = proj
    print("[bench] configs: 512 small Linears", file=sys.stderr, flush=True)
    xb, wb = workloads.small_batch()
    x, w = to_dev(xb), to_dev(wb)
    B, M, K = x.shape
    N = w.shape[2]
    blin = BatchedDelayedScalingLinear(B, hist_len=16, device=dev)
    split = BatchedDelayedScalingLinear(B, hist_len=16, device=dev, fused=False)
    blin.step(x, w)
    split.step(x, w)
    # the steps' launches prepared once (argument checks done at preparation):
    # the binding's per-call checks take about as long as the one-launch step
    step_fused = dsg.prepare(lambda: blin.step(x, w))
    step_split = dsg.prepare(lambda: split.step(x, w))
    reps = max(iters, 50)  # the steps are short: average over more repeats
    ms = time_launches(torch, stream, step_fused, reps)
    ms_split = time_launches(torch, stream, step_split, reps)
    ms_py = time_launches(torch, stream, lambda: blin.step(x, w), reps)
    # bytes of the step as four launches: casts read bf16 X, W (2 B) and write FP8
    # (1 B); the GEMM reads the FP8 operands and writes bf16 Y.  The one-launch step
    # moves less (the FP8 operands stay on chip): its own bytes are reported too.
    nbytes = B * (3 * (M * K + K * N) + (M * K + K * N) + 2 * M * N)
    nbytes_fused = B * (3 * (M * K + K * N) + 2 * M * N)
    gbps = nbytes / (ms * 1e-3) / 1e9
    out["small_batch_512x256"] = {
        "launches": 1 if blin.takes_fused(x, w) else 4,
        "step_ms": round(ms, 4), "tflops": tf(2 * B * M * N * K, ms),
        "GB/s": round(gbps, 1), "frac_hbm": round(gbps / PEAK_HBM_GBPS, 4),
        "moved_GB/s": round(nbytes_fused / (ms * 1e-3) / 1e9, 1),
        "four_launch_step_ms": round(ms_split, 4),
        "step_ms_with_binding_checks": round(ms_py, 4)}
    del x, w, blin, split
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: the library and this benchmark "
              "run on one GPU only (sharding the Linear over several GPUs is not implemented)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calib:
        copy_calibration(torch, args.copy_calib)
        return

    import delayed_scaling_gemm_amd as dsg
    import workloads
    from delayed_scaling_gemm_amd import (E4M3, E5M2, MMA_FP8, OP_N, OP_T, fp8ds_cast_acc,
                                          fp8ds_gemm, fp8ds_gemm_acc, fp8ds_scale_update_clear)
    from delayed_scaling_gemm_amd.linear import DelayedScalingLinear

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating inputs M={M_TOK} K={K_IN} N={N_OUT}", file=sys.stderr, flush=True)
    xb, wb, dyb = workloads.fwd_bwd_4096(M_TOK, K_IN, N_OUT)

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)

    base = [to_dev(xb), to_dev(wb), to_dev(dyb)]
    sets = [base] + [[t.clone() for t in base] for _ in range(N_SETS - 1)]
    torch.cuda.synchronize()

    lin = DelayedScalingLinear(hist_len=HIST_LEN, algo=dsg.ALGO_MAX, margin=0, device=dev)
    stream = torch.cuda.current_stream()
    M, K, N = M_TOK, K_IN, N_OUT

    names = ["cast_x", "cast_w_t", "gemm_fwd_nt", "cast_dy", "gemm_dgrad_nt", "gemm_wgrad_tn",
             "scale_update"]

    def launches(x, w, dy):
        """The launches of DelayedScalingLinear.step, one closure each, in order
        (for the per-kernel figures; they combine into one accumulator set)."""
        b = lin._bufs
        xq, wq, wqt, y, dyq, dx, dw = (b[k] for k in ("xq", "wq", "wqt", "y", "dyq", "dx", "dw"))
        slot = lin._slot
        s, su = lin.scale, lin.scale_used
        am, sat = lin._amax_of(slot), lin._sat_of(slot)
        amy = lin._acc[slot, 3:4].view(torch.float32)
        amdw = lin._acc[slot, 4:5].view(torch.float32)
        return [
            lambda: fp8ds_cast_acc(x, E4M3, s[0:1], xq, None, su[0:1], am[0:1], sat[0:1]),
            lambda: fp8ds_cast_acc(w, E4M3, s[1:2], wq, wqt, su[1:2], am[1:2], sat[1:2]),
            lambda: fp8ds_gemm_acc(OP_N, OP_T, M, N, K, xq, E4M3, K, su[0:1], wqt, E4M3, K, su[1:2],
                                   y, N, amy, mma=lin.fwd_datapath(K)),
            lambda: fp8ds_cast_acc(dy, E5M2, s[2:3], dyq, None, su[2:3], am[2:3], sat[2:3]),
            lambda: fp8ds_gemm(OP_N, OP_T, M, K, N, dyq, E5M2, N, su[2:3], wq, E4M3, N, su[1:2],
                               dx, K, mma=lin.mma_bwd),
            lambda: fp8ds_gemm_acc(OP_T, OP_N, K, N, M, xq, E4M3, K, su[0:1], dyq, E5M2, N,
                                   su[2:3], dw, N, amdw, mma=lin.mma_bwd),
            lambda: fp8ds_scale_update_clear(lin.history, lin.cursor, am, lin.fmts, lin.algo,
                                             lin.margin, s, lin._acc[slot ^ 1]),
        ]

    def step(x, w, dy):
        lin.step(x, w, dy)

    for i in range(max(args.warmup, 1)):
        x, w, dy = sets[i % N_SETS]
        lin.step(x, w, dy)  # also allocates the output buffers
    torch.cuda.synchronize()

    # Per-kernel durations, before the timed region: each launch of the step K
    # times back to back between two events on the library's stream, the inputs
    # rotated over the input sets (events between launches would add several
    # microseconds to every interval).  The launches are prepared (dsg.prepare):
    # called through the binding's checks, the short ones (casts, scale update)
    # were paced by the host rather than the GPU.  These are the casts' and the
    # scale update's figures; the GEMMs' (the roofline) are taken again inside
    # the step below.  The scaling state is restored afterwards.
    print(f"[bench] per-kernel timing, {args.steps} launches each", file=sys.stderr, flush=True)
    saved = [t.clone() for t in (lin.history, lin.cursor, lin.scale, lin._acc)]
    per = {}
    for j, name in enumerate(names):
        fns = [dsg.prepare(launches(*sets[i])[j]) for i in range(N_SETS)]
        fns[0]()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for r in range(args.steps):
            fns[r % N_SETS]()
        e1.record(stream)
        torch.cuda.synchronize()
        per[name] = e0.elapsed_time(e1) / args.steps
    # The GEMMs again, in the step: K full steps of the launches with events
    # around the one GEMM being timed.  Back to back, the same GEMM runs several
    # percent longer than between the step's memory-bound casts (measured in the
    # kernel trace: ~410 against ~390 us for the dX GEMM; the matrix cores alone
    # draw more power), so these are the figures of the step; each interval also
    # holds the event pair's own ~1-2 us.
    per_b2b = {}
    for name in ("gemm_fwd_nt", "gemm_dgrad_nt", "gemm_wgrad_tn"):
        j = names.index(name)
        pairs = []
        for r in range(args.steps):
            for jj, f in enumerate(launches(*sets[r % N_SETS])):
                if jj == j:
                    a = torch.cuda.Event(enable_timing=True)
                    b = torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    f()
                    b.record(stream)
                    pairs.append((a, b))
                else:
                    f()
        torch.cuda.synchronize()
        per_b2b[name] = per[name]
        per[name] = sum(a.elapsed_time(b) for a, b in pairs) / len(pairs)
    for t, v in zip((lin.history, lin.cursor, lin.scale, lin._acc), saved):
        t.copy_(v)
    torch.cuda.synchronize()

    # The timed region: K steps with events only at its two ends.
    e_start = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    e_start.record(stream)
    for i in range(args.steps):
        x, w, dy = sets[i % N_SETS]
        step(x, w, dy)
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall0
    ms_per_step = e_start.elapsed_time(e_end) / args.steps

    # Step-time distribution: a separate pass of at least 50 steps with an event
    # at every step boundary (each event adds a few microseconds to its step, so
    # `value` comes from the region above, timed at its ends only).
    n_dist = max(50, args.steps)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_dist + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(n_dist):
        x, w, dy = sets[i % N_SETS]
        step(x, w, dy)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    dist = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(n_dist)])
    step_dist = {"steps": n_dist, "median_ms": round(float(np.median(dist)), 4),
                 "p10_ms": round(float(np.percentile(dist, 10)), 4),
                 "p90_ms": round(float(np.percentile(dist, 90)), 4)}

    flop_gemm = 2.0 * M * K * N
    value = 3 * flop_gemm / (ms_per_step * 1e-3) / 1e12
    avg = {n: float(per[n]) for n in names}
    gemms = ("gemm_fwd_nt", "gemm_dgrad_nt", "gemm_wgrad_tn")
    gemm_tflops = {n: round(flop_gemm / (avg[n] * 1e-3) / 1e12, 1) for n in gemms}
    # algorithmic bytes of the casts: read the input (2 B), write the FP8 bytes (1 B)
    cast_bytes = {"cast_x": M * K * 3, "cast_w_t": K * N * 4, "cast_dy": M * N * 3}
    cast_gbps = {n: round(b / (avg[n] * 1e-3) / 1e9, 1) for n, b in cast_bytes.items()}
    dom = max(gemms, key=lambda n: avg[n])
    achieved = flop_gemm / (avg[dom] * 1e-3) / 1e12
    traffic = measured_traffic(dom)

    result = {
        "metric": "FP8 scaled-GEMM TFLOP/s (% FP8 MFMA peak); amax+cast GB/s (% HBM peak)",
        "value": round(value, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic (seeded; X ~ N(0,1), W ~ N(0,0.02^2), heavy-tailed dY), bf16 inputs",
        "config": {
            "workload": "fwd+bwd FP8 delayed-scaling Linear, 4096 hidden, M=16384 tokens "
                        "(X, W, dY bf16; HYBRID E4M3/E5M2; history 16, max, margin 0; "
                        "forward GEMM on FP8 MFMA, dX and dW GEMMs on the exact "
                        "F16-widened datapath)",
            "M": M, "K": K, "N": N, "hist_len": HIST_LEN,
        },
        "roofline": {
            "kernel": dom,
            "bound": "mfma",
            "achieved": round(achieved, 1),
            "peak": PEAK_FP8_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_FP8_TFLOPS, 4),
            "traffic": traffic,
            "peak_f16_mfma": PEAK_F16_TFLOPS,
            "frac_f16_mfma": round(achieved / PEAK_F16_TFLOPS, 4),
        },
        # the Linear's X cast: one fp8ds_cast_acc call (the cast kernel alone)
        "cast_roofline_linear": {
            "kernel": "cast_x",
            "bound": "hbm",
            "achieved": cast_gbps["cast_x"],
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(cast_gbps["cast_x"] / PEAK_HBM_GBPS, 4),
        },
        "gemm_tflops": gemm_tflops,
        "cast_gbps": cast_gbps,
        "kernel_ms": {n: round(v, 4) for n, v in avg.items()},
        "gemm_ms_back_to_back": {n: round(v, 4) for n, v in per_b2b.items()},
        "step_ms_distribution": step_dist,
        "wall_ms_per_step": round(wall / args.steps * 1e3, 4),
        "sum_of_kernel_ms": round(sum(avg.values()), 4),
    }

    if not args.no_fp8_path:
        # context only: each GEMM of the step on the other datapath -- the forward
        # on the exact F16-widened path, the backward products on the FP8 matrix
        # instructions (whose summation misses the tolerance on heavy-tailed
        # gradients, see fp8ds_mma)
        b = lin._bufs
        su = lin.scale_used
        other = {0: 1, 1: 0}
        calls = {
            "gemm_fwd_nt": lambda: fp8ds_gemm(OP_N, OP_T, M, N, K, b["xq"], E4M3, K, su[0:1],
                                              b["wqt"], E4M3, K, su[1:2], b["y"], N, None,
                                              mma=other[lin.fwd_datapath(K)]),
            "gemm_dgrad_nt": lambda: fp8ds_gemm(OP_N, OP_T, M, K, N, b["dyq"], E5M2, N, su[2:3],
                                                b["wq"], E4M3, N, su[1:2], b["dx"], K, None,
                                                mma=other[lin.mma_bwd]),
            "gemm_wgrad_tn": lambda: fp8ds_gemm(OP_T, OP_N, K, N, M, b["xq"], E4M3, K, su[0:1],
                                                b["dyq"], E5M2, N, su[2:3], b["dw"], N, None,
                                                mma=other[lin.mma_bwd]),
        }
        alt = {}
        for n, fn in calls.items():
            fn()
            ms = time_launches(torch, stream, fn, 10)
            alt[n] = round(flop_gemm / (ms * 1e-3) / 1e12, 1)
        result["other_datapath_tflops"] = {
            "datapaths": {"gemm_fwd_nt": "exact" if lin.fwd_datapath(K) == MMA_FP8 else "fp8",
                          "gemm_dgrad_nt": "exact" if lin.mma_bwd == MMA_FP8 else "fp8",
                          "gemm_wgrad_tn": "exact" if lin.mma_bwd == MMA_FP8 else "fp8"},
            **alt}

    if not args.no_finer:
        x0, w0, dy0 = sets[0]
        result["finer_scaling"] = finer_report(torch, dsg, x0, w0, dy0)
    if not args.no_stress:
        result["cast_stress"], cast_sample = stress_cast(torch, dsg, workloads, dev)
        # the metric's amax+cast figure: the 2^30-element bandwidth workload
        st = result["cast_stress"]["e4m3"]
        result["cast_roofline"] = {
            "kernel": "cast_kernel: amax + cast of 2^30 bf16 elements to E4M3 (3 B/element)",
            "bound": "hbm", "achieved": st["GB/s"], "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": st["frac_hbm"]}
    if not args.no_optimizer:
        result["optimizer"] = optimizer_report(torch, dsg, workloads, dev)
    if not args.no_configs:
        del sets, base
        torch.cuda.empty_cache()
        result["configs"] = configs_report(torch, dsg, workloads, dev)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(xb, wb, dyb)
        result["cpu_baseline"]["other_workloads"] = cpu_other(
            workloads, cast_sample if not args.no_stress else None)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
