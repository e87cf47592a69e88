#!/usr/bin/env python3
"""Throughput of the windowed-attention forward hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
the log-CPB table for the window size (swin_cpb_table) and the fused window
attention over the grid, partition, shift mask and reverse map included
(swin_window_attn_fwd).  Inputs are resident in HBM before timing starts.

Timing: W untimed warm-up steps, then exactly K timed steps between two
torch.cuda.synchronize() calls.  The defaults (200 warm-up, 500 timed)
measure the steady state: the GPU's clocks settle over the first hundred or
so launches of the path, and the first 50 steps after 10 run about 10%
slower than the same steps later.  Cold cache by default: the steps rotate
through enough distinct input/output sets (> 512 MB in all) that the 256 MB
Infinity Cache cannot hold one set between its uses; --warm reuses one set.
The attention kernel's own duration is taken from HIP events recorded on the
launch stream around every timed launch; the events are created with
hipEventDisableSystemFence (timing only), so recording them adds no cache
writeback or invalidation to the interval.

Prints ONE JSON line.  `value` is tokens/s over the whole job.

Other modes (same protocol, their own JSON line): --backward times the
backward step; --branch times the attention branch of a block (input
projection, table, attention, output projection with the residual post-norm;
--fused takes the input projection inside the attention kernel);
--linmapper times LinMapper's in-window linear mapping.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "window-attn fwd tokens/s + TFLOP/s (% bf16 MFMA peak), SwinV2-T M=16 256px"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 vector, TFLOP/s
MALL_BYTES = 256 * 2 ** 20
KERNEL_SOURCE = {"attn_small_kernel": "attn_small.hip", "attn_large_kernel": "attn_large.hip",
                 "attn_mfma_kernel": "attn_mfma.hip", "attn_valu_kernel": "attn_valu.hip",
                 "attn_video_mfma_kernel": "attn_video_mfma.hip"}


# headers a kernel's file includes beyond the shared ones
KERNEL_HEADERS = {"attn_small_kernel": ("small_core.hpp",)}


def kernel_sha(kernel: str) -> str:
    """Hash of the sources that define `kernel` (its file and the headers it includes)."""
    h = hashlib.sha256()
    for f in (KERNEL_SOURCE[kernel], *KERNEL_HEADERS.get(kernel, ()), "common.hpp", "launch.hpp", "tile_io.hpp",
              "lanes.hpp"):
        with open(os.path.join(ROOT, "vision_transformer_windowed_partition_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(wl_name: str, kernel: str):
    """HBM bytes per launch from committed rocprofv3 --pmc counts, if they
    were taken on the current sources of `kernel`; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{wl_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel") != kernel or t.get("kernel_sha") != kernel_sha(kernel):
        return None
    return round(t.get("hbm_bytes_per_launch"))


class HipTimer:
    """Pairs of HIP events on one stream, created with
    hipEventDisableSystemFence.  Uses the HIP runtime the process already
    loaded (torch's), found by its soname."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n: int, stream_handle: int):
        hip = ctypes.CDLL("libamdhip64.so.7")
        hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip, self.stream = hip, ctypes.c_void_p(stream_handle)
        self.ev = []
        for _ in range(2 * n):
            e = ctypes.c_void_p()
            self._ok(hip.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE), "create")
            self.ev.append(e)

    def _ok(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"hipEvent{what} failed: {rc}")

    def record(self, i: int, end: bool):
        self._ok(self.hip.hipEventRecord(self.ev[2 * i + int(end)], self.stream), "Record")

    def elapsed_ms(self) -> list[float]:
        out = []
        for i in range(len(self.ev) // 2):
            self._ok(self.hip.hipEventSynchronize(self.ev[2 * i + 1]), "Synchronize")
            ms = ctypes.c_float()
            self._ok(self.hip.hipEventElapsedTime(ctypes.byref(ms), self.ev[2 * i], self.ev[2 * i + 1]),
                     "ElapsedTime")
            out.append(ms.value)
        return out

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)
        self.ev = []


def cpu_baseline(wl, x, budget_s: float):
    """The fp64 oracle on a bounded sample of the same workload, on the host's
    cores, in tokens/s: evenly spaced windows sized to about budget_s of wall
    time, the whole sample repeated while it takes less than half of it."""
    import numpy as np
    import torch

    import oracle

    f64 = lambda t: t.to(torch.float64).numpy()
    q, k, v = f64(x["q"]), f64(x["k"]), f64(x["v"])
    nwin = wl.n_windows
    t0 = time.perf_counter()
    table = None
    if wl.pos == "table":
        table = oracle.cpb_table(wl.M, f64(x["w1"]), f64(x["b1"]), f64(x["w2"]), f64(x["b2"]))
    t_table = time.perf_counter() - t0
    kw = dict(heads=wl.heads, M=wl.M, shift=wl.shift, partition=wl.partition, sim=wl.sim, pos=wl.pos,
              tau=f64(x["tau"]), table=table, rope_base=wl.rope_base)
    # probe on a few windows, then size the sample to the budget
    probe = np.linspace(0, nwin - 1, num=min(nwin, 8), dtype=np.int64)
    t0 = time.perf_counter()
    oracle.window_attn(q, k, v, windows=probe, **kw)
    per_win = (time.perf_counter() - t0) / len(probe)
    n = int(min(nwin, max(len(probe), budget_s / max(per_win, 1e-9))))
    wins = np.unique(np.linspace(0, nwin - 1, num=n, dtype=np.int64))
    reps, dt = 0, t_table
    while reps == 0 or dt < 0.5 * budget_s:
        t0 = time.perf_counter()
        oracle.window_attn(q, k, v, windows=wins, **kw)
        dt += time.perf_counter() - t0
        reps += 1
    tokens = reps * len(wins) * wl.N
    sample = (f"all {nwin} windows" if len(wins) == nwin else
              f"{len(wins)} of {nwin} windows, evenly spaced over the batch") + \
             (f", {reps} passes" if reps > 1 else "") + \
             f" ({tokens} tokens, {dt:.1f} s incl. one CPB table)"
    return {"value": tokens / dt, "unit": "tokens/s", "cores": oracle.max_threads(), "kind": "oracle",
            "sample": sample, "cpu": oracle.cpu_model()}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", type=int, default=1, help="index into synth.WORKLOADS (1 = headline)")
    ap.add_argument("--warm", action="store_true", help="reuse one input set (cache-warm)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle wall time")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward step instead: swin_window_attn_bwd (dq, dk, dv, dtau, dtable) "
                         "and swin_cpb_table_bwd, from one forward's output")
    ap.add_argument("--own-lse", action="store_true",
                    help="with --backward: the backward recomputes the softmax statistics instead of "
                         "taking the forward's log-sum-exp")
    ap.add_argument("--branch", action="store_true",
                    help="time the whole attention branch instead: swin_qkv_proj, the CPB table, "
                         "swin_window_attn_fwd and swin_proj_post_norm (residual post-norm)")
    ap.add_argument("--fused", action="store_true",
                    help="with --branch: the input layer fused into the attention (swin_qkv_window_attn_fwd) "
                         "instead of swin_qkv_proj then swin_window_attn_fwd")
    ap.add_argument("--linmapper", action="store_true",
                    help="time LinMapper's in-window linear mapping (swin_window_linear) on the "
                         "workload's values instead of the attention")
    ap.add_argument("--video", type=int, nargs="?", const=0, default=None, metavar="IDX",
                    help="time video (3D) window attention instead: swin_window_attn3d_fwd on "
                         "synth.VIDEO_WORKLOADS[IDX] (0: 256^2 x 8 frames, 16^2 x 8 windows; 1: 320^2 x 8 "
                         "frames, 20^2 x 8 windows), its table from swin_cpb_table3d")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run copies of known size for HBM-counter calibration: y = -x over "
                         "2^28 fp32 (whole lines), then an interleaved window gather and its "
                         "scatter of a 16x512x512x32 bf16 grid (64-byte pieces), 3 launches each")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py: this library runs on one GPU; --gpus {args.gpus} is not supported "
              "(windows, heads and batch shard with no exchange; see the design notes)", file=sys.stderr)
        return 2

    import torch

    from vision_transformer_windowed_partition_amd import binding, synth

    if args.video is not None:
        return bench_video(args)
    wl = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    x = synth.make_inputs(wl)

    set_bytes = 4 * wl.tokens * wl.C * wl.elem_size
    nsets = 1 if args.warm else max(2, math.ceil(2 * MALL_BYTES / set_bytes) + 1)
    sets = []
    for i in range(nsets):
        if i == 0:
            q, k, v = (x[n].to(dev) for n in "qkv")
        else:   # distinct buffers with the same contents (a permuted batch would change nothing timed)
            q, k, v = (sets[0][j].clone() for j in range(3))
        sets.append((q, k, v, torch.empty_like(q)))
    par = {n: x[n].to(dev) for n in ("tau", "w1", "b1", "w2", "b2")}
    table = torch.empty(((2 * wl.M - 1) ** 2, wl.heads), dtype=torch.float32, device=dev)
    desc = binding.make_desc(B=wl.B, H=wl.H, W=wl.W, C=wl.C, heads=wl.heads, M=wl.M, shift=wl.shift,
                             partition=wl.partition, sim=wl.sim, pos=wl.pos, dtype=q.dtype,
                             rope_base=wl.rope_base)
    stream = torch.cuda.current_stream(dev)
    kernel = binding.swin_window_attn_kernel(desc)
    if args.backward:
        return bench_backward(args, wl, x, sets, nsets, par, table, desc, stream)
    if args.branch:
        del sets
        return bench_branch(args, wl, par, table, desc, stream)
    if args.linmapper:
        return bench_linmapper(args, wl, sets, nsets, stream)

    def step(i, timed=None):
        q, k, v, o = sets[i % nsets]
        tab = None
        if wl.pos == "table":
            tab = binding.swin_cpb_table(wl.M, par["w1"], par["b1"], par["w2"], par["b2"], out=table,
                                         stream=stream)
        if timed is not None:
            timer.record(timed, False)
        binding.swin_window_attn_fwd(q, k, v, heads=wl.heads, M=wl.M, desc=desc, tau=par["tau"],
                                     table=tab, out=o, stream=stream)
        if timed is not None:
            timer.record(timed, True)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    timer = HipTimer(args.steps, stream.cuda_stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = timer.elapsed_ms()
    timer.close()
    kern_avg = sum(kern_ms) / len(kern_ms)

    if args.calib_copy:
        run_calib_copies(dev)

    ms_per_step = wall * 1e3 / args.steps
    tokens_s = wl.tokens / (wall / args.steps)
    alg_bytes = wl.bytes
    kern_s = kern_avg * 1e-3
    gbs = alg_bytes / kern_s / 1e9
    tflops = wl.flops / kern_s / 1e12
    peak_tf = BF16_PEAK_TFLOPS if wl.dtype == "bf16" else FP32_PEAK_TFLOPS
    ai = wl.flops / alg_bytes
    ridge = peak_tf * 1e12 / (HBM_PEAK_GBS * 1e9)
    if ai < ridge:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": peak_tf, "unit": "TFLOP/s",
                "frac": round(tflops / peak_tf, 4)}
    roof["traffic"] = load_traffic(wl.name, kernel)
    roof["kernel"] = kernel
    roof["kernel_ms"] = round(kern_avg, 5)
    roof["kernel_ms_median"] = round(sorted(kern_ms)[len(kern_ms) // 2], 5)
    roof["kernel_ms_min"] = round(min(kern_ms), 5)
    roof["alg_bytes_per_launch"] = alg_bytes
    roof["alg_flops_per_launch"] = wl.flops

    out = {
        "metric": METRIC,
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) q/k/v, random-init log-CPB MLP)",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "W": wl.W, "C": wl.C, "heads": wl.heads,
                   "M": wl.M, "shift": wl.shift, "partition": wl.partition, "sim": wl.sim,
                   "pos": wl.pos, "cache": "warm" if args.warm else f"cold ({nsets} rotating sets)",
                   "parallelism": "none (1 GPU)"},
        "tflops": round(tflops, 2),
        "mfma_frac": round(tflops / BF16_PEAK_TFLOPS, 4) if wl.dtype == "bf16" else None,
        "hbm_gbs": round(gbs, 1),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, x, args.cpu_budget)
    print(json.dumps(out))
    return 0


def bench_backward(args, wl, x, sets, nsets, par, table, desc, stream) -> int:
    """Backward step: dq, dk, dv, dtau, dtable from (q, k, v, out, dout), then
    the meta network's parameter gradients from dtable.  Algorithmic work per
    (window, head): the five N x N x d contractions of the backward (scores
    recomputed, dP, dV, dQ, dK: 10 N^2 d flops) and 8 N d elements moved
    (read q, k, v, out, dout; write dq, dk, dv), plus N fp32 statistics
    read when the forward's log-sum-exp is given (the default; --own-lse
    recomputes them)."""
    import torch

    from vision_transformer_windowed_partition_amd import binding, synth

    tab = None
    if wl.pos == "table":
        tab = binding.swin_cpb_table(wl.M, par["w1"], par["b1"], par["w2"], par["b2"], out=table)
    dout = synth.make_dout(wl).to(sets[0][0].device)
    use_lse = not args.own_lse
    lses = []
    for q, k, v, o in sets:
        if use_lse:
            lses.append(binding.swin_window_attn_fwd_lse(q, k, v, heads=wl.heads, M=wl.M, desc=desc, tau=par["tau"],
                                                         table=tab, out=o)[1])
        else:
            binding.swin_window_attn_fwd(q, k, v, heads=wl.heads, M=wl.M, desc=desc, tau=par["tau"], table=tab,
                                         out=o)
    torch.cuda.synchronize()
    kw = dict(heads=wl.heads, M=wl.M, shift=wl.shift, partition=wl.partition, sim=wl.sim, pos=wl.pos,
              tau=par["tau"], table=tab, rope_base=wl.rope_base, desc=desc, stream=stream)

    def step(i, timed=None):
        q, k, v, o = sets[i % nsets]
        if timed is not None:
            timer.record(timed, False)
        g = binding.swin_window_attn_bwd(q, k, v, o, dout, lse=lses[i % nsets] if use_lse else None, **kw)
        if timed is not None:
            timer.record(timed, True)
        if wl.pos == "table":
            binding.swin_cpb_table_bwd(wl.M, par["w1"], par["b1"], par["w2"], tab, g["dtable"], stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    timer = HipTimer(args.steps, stream.cuda_stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = timer.elapsed_ms()
    timer.close()
    kern_avg = sum(kern_ms) / len(kern_ms)
    flops = int(2.5 * wl.flops)
    alg_bytes = 2 * wl.bytes + (wl.tokens * wl.heads * 4 if use_lse else 0)
    kern_s = kern_avg * 1e-3
    tflops = flops / kern_s / 1e12
    kernel = binding.swin_window_attn_bwd_kernel(desc)
    if kernel == "attn_bwd_kernel":      # fp32 vector ALUs
        compute, peak_tf = "alu", FP32_PEAK_TFLOPS
    else:                                # bf16 matrix cores
        compute, peak_tf = "mfma", BF16_PEAK_TFLOPS
    # the ceiling is whichever of HBM and the compute peak takes longer
    if flops / alg_bytes < peak_tf * 1e12 / (HBM_PEAK_GBS * 1e9):
        gbs = alg_bytes / kern_s / 1e9
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": compute, "achieved": round(tflops, 2), "peak": peak_tf, "unit": "TFLOP/s",
                "frac": round(tflops / peak_tf, 4)}
    roof.update({"traffic": None, "kernel": kernel, "kernel_ms": round(kern_avg, 5),
                 "kernel_ms_median": round(sorted(kern_ms)[len(kern_ms) // 2], 5),
                 "kernel_ms_min": round(min(kern_ms), 5), "alg_bytes_per_launch": alg_bytes,
                 "alg_flops_per_launch": flops})
    out = {
        "metric": "window-attn bwd tokens/s (dq, dk, dv, dtau, dtable + CPB meta-network gradients)",
        "value": round(wl.tokens / (wall / args.steps), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) q/k/v/dout, random-init log-CPB MLP)",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "W": wl.W, "C": wl.C, "heads": wl.heads,
                   "M": wl.M, "shift": wl.shift, "partition": wl.partition, "sim": wl.sim,
                   "pos": wl.pos, "pass": "backward",
                   "softmax_stats": "forward's log-sum-exp" if use_lse else "recomputed",
                   "cache": "warm" if args.warm else f"cold ({nsets} rotating sets)",
                   "parallelism": "none (1 GPU)"},
        "tflops": round(tflops, 2),
        "hbm_gbs": round(alg_bytes / kern_s / 1e9, 1),
        "roofline": roof,
    }
    print(json.dumps(out))
    return 0


def _roof(flops: float, alg_bytes: float, ms: float, peak_tf: float, compute: str) -> dict:
    """Roofline entry of one kernel: HBM if its arithmetic intensity is below
    the ridge of its compute unit, else that unit."""
    s = ms * 1e-3
    if flops / alg_bytes < peak_tf * 1e12 / (HBM_PEAK_GBS * 1e9):
        gbs = alg_bytes / s / 1e9
        return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4)}
    tf = flops / s / 1e12
    return {"bound": compute, "achieved": round(tf, 2), "peak": peak_tf, "unit": "TFLOP/s",
            "frac": round(tf / peak_tf, 4)}


def bench_branch(args, wl, par, table, desc, stream) -> int:
    """Attention branch step of a Swin V2 block: q, k, v = split(x W_qkv^T +
    b), the CPB table, the window attention, y = x + norm_1(o W_proj^T + b);
    for interleaved windows (Iwin) the depthwise 3x3 convolution of v is added
    to o before the output layer.  Algorithmic work: QKV 6 T C^2 flops and
    4 T C es bytes (read x, write q, k, v); attention as the forward;
    convolution 18 T C flops and 3 T C es bytes (read v and o, write o);
    output layer 2 T C^2 flops and 3 T C es bytes (read o and x, write y);
    weights counted once."""
    import torch

    from vision_transformer_windowed_partition_amd import binding, synth

    dev = torch.device("cuda:0")
    p = synth.make_branch_params(wl)
    w = {n: p[n].to(dev) for n in ("w_qkv", "b_qkv", "w_proj", "b_proj", "gamma", "beta", "w_dw", "b_dw")}
    iwin = wl.partition == "interleaved"          # Iwin couples its attention with the convolution branch
    T, C, es = wl.tokens, wl.C, wl.elem_size
    set_bytes = 6 * T * C * es
    nsets = 1 if args.warm else max(2, math.ceil(2 * MALL_BYTES / set_bytes) + 1)
    x0 = p["x"].to(dev).reshape(wl.B, wl.H, wl.W, C)
    sets = []
    for i in range(nsets):
        xs = x0 if i == 0 else x0.clone()
        sets.append(dict(x=xs, q=torch.empty_like(xs), k=torch.empty_like(xs), v=torch.empty_like(xs),
                         o=torch.empty_like(xs), y=torch.empty_like(xs)))
    fused = args.fused
    if fused and iwin:
        raise SystemExit("bench.py: --fused covers the attention branch without the convolution of v")
    first = ("qkv_attn",) if fused else ("qkv", "attn")
    names = first + (("dwconv", "norm") if iwin else ("norm",))

    def step(i, timed=None):
        st = sets[i % nsets]
        rec = (lambda n, end: timers[n].record(timed, end)) if timed is not None else (lambda n, end: None)
        tab = None
        if wl.pos == "table":
            tab = binding.swin_cpb_table(wl.M, par["w1"], par["b1"], par["w2"], par["b2"], out=table,
                                         stream=stream)
        if fused:
            rec("qkv_attn", False)
            binding.swin_qkv_window_attn_fwd(st["x"], w["w_qkv"], w["b_qkv"], heads=wl.heads, M=wl.M,
                                             shift=wl.shift, partition=wl.partition, sim=wl.sim, pos=wl.pos,
                                             tau=par["tau"], table=tab, out=st["o"], stream=stream)
            rec("qkv_attn", True)
        else:
            rec("qkv", False)
            binding.swin_qkv_proj(st["x"], w["w_qkv"], w["b_qkv"], out=(st["q"], st["k"], st["v"]),
                                  stream=stream)
            rec("qkv", True)
            rec("attn", False)
            binding.swin_window_attn_fwd(st["q"], st["k"], st["v"], heads=wl.heads, M=wl.M, desc=desc,
                                         tau=par["tau"], table=tab, out=st["o"], stream=stream)
            rec("attn", True)
        if iwin:
            rec("dwconv", False)
            binding.swin_dwconv_add(st["v"], w["w_dw"], w["b_dw"], st["o"], stream=stream)
            rec("dwconv", True)
        rec("norm", False)
        binding.swin_proj_post_norm(st["o"], w["w_proj"], w["b_proj"], st["x"], w["gamma"], w["beta"], eps=1e-5,
                                    out=st["y"], stream=stream)
        rec("norm", True)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    timers = {n: HipTimer(args.steps, stream.cuda_stream) for n in names}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = {}
    for n in names:
        e = timers[n].elapsed_ms()
        timers[n].close()
        ms[n] = sum(e) / len(e)
    peak_tf = BF16_PEAK_TFLOPS if wl.dtype == "bf16" else FP32_PEAK_TFLOPS
    compute = "mfma" if wl.dtype == "bf16" else "alu"
    work = {"qkv": (6.0 * T * C * C, 4.0 * T * C * es),
            "attn": (float(wl.flops), float(wl.bytes)),
            "qkv_attn": (6.0 * T * C * C + float(wl.flops), 2.0 * T * C * es),
            "norm": (2.0 * T * C * C, 3.0 * T * C * es),
            "dwconv": (18.0 * T * C, 3.0 * T * C * es)}
    kname = {"qkv": "qkv_kernel" if wl.dtype == "bf16" else "qkv_f32_kernel",
             "attn": binding.swin_window_attn_kernel(desc),
             "qkv_attn": "attn_fused_kernel",
             "norm": "norm_kernel" if wl.dtype == "bf16" else "norm_f32_kernel",
             "dwconv": "dwconv_add_kernel"}
    kernels = {}
    for n in names:
        r = _roof(work[n][0], work[n][1], ms[n], peak_tf, compute)
        r.update({"kernel": kname[n], "kernel_ms": round(ms[n], 5), "alg_flops_per_launch": work[n][0],
                  "alg_bytes_per_launch": work[n][1], "traffic": None})
        kernels[n] = r
    dominant = max(names, key=lambda n: ms[n])
    out = {
        "metric": "attention branch tokens/s (QKV projection, CPB table, window attention, "
                  if not fused else
                  "attention branch tokens/s (CPB table, window attention with the QKV projection fused in, "
                  + ("depthwise 3x3 convolution of v, " if iwin else "")
                  + "output projection + residual post-norm)",
        "value": round(T / (wall / args.steps), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) features, randn/sqrt(C) weights, random-init log-CPB MLP)",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "W": wl.W, "C": wl.C, "heads": wl.heads,
                   "M": wl.M, "shift": wl.shift, "partition": wl.partition, "sim": wl.sim, "pos": wl.pos,
                   "pass": "attention branch" + (" (fused input layer)" if fused else ""),
                   "cache": "warm" if args.warm else f"cold ({nsets} rotating sets)",
                   "parallelism": "none (1 GPU)"},
        "roofline": kernels[dominant],
        "kernels": kernels,
    }
    print(json.dumps(out))
    return 0


def bench_linmapper(args, wl, sets, nsets, stream) -> int:
    """LinMapper's aggregation in place of the attention: per window and head
    out = A_h v (+ bias), A_h an N x N matrix shared by all windows.
    Algorithmic work per (window, head): 2 N^2 d flops, 2 N d es bytes (read v,
    write out; the matrices, heads N^2 es bytes, counted once per launch)."""
    import torch

    from vision_transformer_windowed_partition_amd import binding

    dev = torch.device("cuda:0")
    N = wl.M * wl.M
    gen = torch.Generator().manual_seed(3000)
    A = (torch.randn((wl.heads, N, N), generator=gen) / math.sqrt(N)).to(sets[0][0].dtype).to(dev)
    bias = (0.1 * torch.randn((wl.heads, N), generator=gen)).to(dev)

    def step(i, timed=None):
        q, k, v, o = sets[i % nsets]
        if timed is not None:
            timer.record(timed, False)
        binding.swin_window_linear(v, A, bias, heads=wl.heads, M=wl.M, shift=wl.shift, partition=wl.partition,
                                   out=o, stream=stream)
        if timed is not None:
            timer.record(timed, True)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    timer = HipTimer(args.steps, stream.cuda_stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = timer.elapsed_ms()
    timer.close()
    kern_avg = sum(kern_ms) / len(kern_ms)
    es = wl.elem_size
    flops = 2.0 * wl.tokens * N * wl.C
    alg_bytes = 2.0 * wl.tokens * wl.C * es + wl.heads * N * N * es
    peak_tf = BF16_PEAK_TFLOPS if wl.dtype == "bf16" else FP32_PEAK_TFLOPS
    roof = _roof(flops, alg_bytes, kern_avg, peak_tf, "mfma" if wl.dtype == "bf16" else "alu")
    fast = wl.dtype == "bf16" and wl.M in (8, 16)
    kname = ("wlin16_kernel" if wl.M == 16 else "wlin_kernel") if fast else "wlin_valu_kernel"
    roof.update({"kernel": kname, "kernel_ms": round(kern_avg, 5),
                 "alg_flops_per_launch": flops, "alg_bytes_per_launch": alg_bytes, "traffic": None})
    out = {
        "metric": "LinMapper in-window linear mapping tokens/s",
        "value": round(wl.tokens / (wall / args.steps), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) values, randn/sqrt(N) window matrices)",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "W": wl.W, "C": wl.C, "heads": wl.heads,
                   "M": wl.M, "shift": wl.shift, "partition": wl.partition, "pass": "linmapper",
                   "cache": "warm" if args.warm else f"cold ({nsets} rotating sets)",
                   "parallelism": "none (1 GPU)"},
        "roofline": roof,
    }
    print(json.dumps(out))
    return 0


def run_calib_copies(dev) -> None:
    """Copies of known size for HBM-counter calibration (see --calib-copy)."""
    import torch

    from vision_transformer_windowed_partition_amd import binding

    a = torch.zeros(2 ** 28, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        torch.neg(a, out=b)
    del a, b
    # each token's 64 bytes sits 4 KiB from the next token of its window
    g = torch.zeros((16, 512, 512, 32), dtype=torch.bfloat16, device=dev)
    w = binding.swin_window_partition(g, 8, 0, "interleaved")
    for _ in range(3):
        binding.swin_window_partition(g, 8, 0, "interleaved", out=w)
    for _ in range(3):
        binding.swin_window_reverse(w, 16, 512, 512, 8, 0, "interleaved", out=g)
    torch.cuda.synchronize()


def bench_video(args) -> int:
    """Video (3D) window attention: swin_window_attn3d_fwd with the table from
    swin_cpb_table3d in each step.  Algorithmic work as for 2D windows: 4 N C
    flops per token (N = Mt M^2) and q, k, v read and o written once."""
    import torch

    from vision_transformer_windowed_partition_amd import binding, synth

    wl = synth.VIDEO_WORKLOADS[args.video]
    dev = torch.device("cuda:0")
    x = synth.make_video_inputs(wl)
    set_bytes = wl.bytes
    nsets = 1 if args.warm else max(2, math.ceil(2 * MALL_BYTES / set_bytes) + 1)
    sets = []
    for i in range(nsets):
        qkv = tuple(x[n].to(dev) for n in "qkv") if i == 0 else tuple(t.clone() for t in sets[0][:3])
        sets.append(qkv + (torch.empty_like(qkv[0]),))
    par = {n: x[n].to(dev) for n in ("tau", "w1", "b1", "w2", "b2")}
    table = torch.empty(((2 * wl.Mt - 1) * (2 * wl.M - 1) ** 2, wl.heads), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(i, timed=None):
        q, k, v, o = sets[i % nsets]
        tab = binding.swin_cpb_table3d(wl.Mt, wl.M, par["w1"], par["b1"], par["w2"], par["b2"], out=table,
                                       stream=stream)
        if timed is not None:
            timer.record(timed, False)
        binding.swin_window_attn3d_fwd(q, k, v, heads=wl.heads, Mt=wl.Mt, M=wl.M, shift_t=wl.shift_t,
                                       shift=wl.shift, partition=wl.partition, sim=wl.sim, pos=wl.pos,
                                       tau=par["tau"], table=tab, out=o, stream=stream)
        if timed is not None:
            timer.record(timed, True)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    timer = HipTimer(args.steps, stream.cuda_stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = timer.elapsed_ms()
    timer.close()
    kern_avg = sum(kern_ms) / len(kern_ms)
    if args.calib_copy:
        run_calib_copies(dev)
    desc = binding.make_desc(B=wl.B, H=wl.H, W=wl.W, C=wl.C, heads=wl.heads, M=wl.M, shift=wl.shift,
                             partition=wl.partition, sim=wl.sim, pos=wl.pos, dtype=sets[0][0].dtype)
    kernel = binding.swin_window_attn3d_kernel(desc, wl.T, wl.Mt)
    mfma = kernel == "attn_video_mfma_kernel"
    roof = _roof(wl.flops, wl.bytes, kern_avg, BF16_PEAK_TFLOPS if mfma else FP32_PEAK_TFLOPS,
                 "mfma" if mfma else "alu")
    roof.update({"kernel": kernel, "kernel_ms": round(kern_avg, 5),
                 "alg_flops_per_launch": wl.flops, "alg_bytes_per_launch": wl.bytes,
                 "traffic": load_traffic(wl.name, kernel) if kernel in KERNEL_SOURCE else None})
    out = {
        "metric": "video window-attn fwd tokens/s",
        "value": round(wl.tokens / (wall / args.steps), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) q/k/v, random-init 3-input log-CPB MLP)",
        "config": {"workload": wl.name, "B": wl.B, "T": wl.T, "H": wl.H, "W": wl.W, "C": wl.C,
                   "heads": wl.heads, "Mt": wl.Mt, "M": wl.M, "shift_t": wl.shift_t, "shift": wl.shift,
                   "partition": wl.partition, "sim": wl.sim, "pos": wl.pos, "pass": "video",
                   "cache": "warm" if args.warm else f"cold ({nsets} rotating sets)",
                   "parallelism": "none (1 GPU)"},
        "roofline": roof,
    }
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
