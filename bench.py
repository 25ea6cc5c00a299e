#!/usr/bin/env python3
"""Benchmark of the causal FFT long convolution on one MI355X.

A step is one fftconv_forward over the whole batch (the full hot path:
load + pack, forward Monarch stages, spectrum product, inverse stages,
unpack + store).  The kernel spectrum is computed once before timing, as the
method precomputes it per channel.  Default workload: the Hyena-shaped
B=64, H=768, N=1024 bf16 convolution.

Prints one JSON line: throughput in outputs/s (B*H*N per step), the
roofline of the dominant kernel, and the fp64 CPU oracle timed on the host
as a baseline.

--gated times the gated form y = v * ((u * w) conv k) instead (one
fftconv_forward_gated per step; the gates are seeded N(0,1) tensors of the
shape of u, resident in HBM like u).  --circular times the non-causal
(circular) convolution on the plan at FFT size N (fftconv_plan_circular),
and beside it, under "compare", the causal call and the circular operator
through the causal plan's 2N-point transform; --backward one
fftconv_backward (du and dk of the causal convolution for a seeded N(0,1)
dy).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import tempfile
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("FFT-conv B*H*N outputs/sec and % of HBM/MFMA roofline, "
          "N=1K..4M, 1 GPU")
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "f32": 157.3}
ROTATE_BYTES = 1 << 30          # > 4x the 256 MB Infinity Cache
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_hash() -> str:
    """sha1 over the library sources; measured traffic is only reported
    while the kernels are the ones the counters were taken on."""
    import hashlib
    d = os.path.join(ROOT, "fft_long_convolution_amd", "csrc")
    h = hashlib.sha1()
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".cpp", ".h")):
            h.update(f.encode())
            with open(os.path.join(d, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha1") != kernel_source_hash():
        return None
    return rec.get("traffic_bytes")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # default (flag not given): sized from a short estimate so that warmup
    # covers >= 0.3 s of work (clocks settle) and the timed region ~1 s
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="hyena_bf16_n1k")
    ap.add_argument("--gated", action="store_true",
                    help="time the gated convolution v * ((u * w) conv k)")
    ap.add_argument("--circular", action="store_true",
                    help="time the non-causal (circular) convolution")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (du and dk)")
    ap.add_argument("--lowpass", type=int, default=None, metavar="F",
                    help="time the frequency-sparse convolution whose kernel "
                         "spectrum keeps frequencies within F of zero")
    ap.add_argument("--blocksparse", default=None, metavar="A,D",
                    help="time the frequency-sparse convolution with zero "
                         "blocks along the transform's digits (a middle values "
                         "of the top digit, d outer classes)")
    ap.add_argument("--no-cpu", action="store_true",
                    help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only the library's streaming copy of the "
                         "workload's input size (reference for HBM byte "
                         "counters)")
    ap.add_argument("--no-extra", action="store_true",
                    help="time only the selected workload (no 'workloads' key)")
    ap.add_argument("--profile", action="store_true",
                    help="profile the selected workload and operator under "
                         "rocprofv3 (kernel trace, HBM byte and instruction "
                         "counters) and write its summary to profiles/")
    ap.add_argument("--profile-dir", default=os.path.join(tempfile.gettempdir(), "fftconv_prof"),
                    help="where rocprofv3 writes its raw output")
    ap.add_argument("--profile-out", default=os.path.join(ROOT, "profiles"),
                    help="where the summary and traffic.json are written")
    return ap.parse_args()


def kf_min_bytes(info: dict, H: int) -> int:
    """The kernel spectrum at its information content: a real kernel's
    spectrum of length L = 2M is Hermitian, so M + 1 complex bins per
    channel carry it (f16 complex for 16-bit plans, fp32 complex for fp32
    plans).  The plans store 8 (16) B per bin, twice that, as per-bin
    coefficients; the roofline counts the minimum."""
    return H * (info["M"] + 1) * (8 if info["dtype"] == "f32" else 4)


def to_torch(a, dtype, torch):
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a))


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: measures one GPU only; %d GPUs were requested (rows "
              "would shard by channel with no communication, each GPU "
              "running this path on its channels)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.profile:
        # drives rocprofv3 runs of this script as child processes; touches
        # no GPU itself
        return profile(args)
    import torch
    from fft_long_convolution_amd import inputs
    from fft_long_convolution_amd.fftconv import FFTConv

    w = inputs.WORKLOADS[args.workload]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        # the library's streaming copy (16-byte non-temporal loads and
        # stores, the access pattern of the kernels) over the workload's
        # input size: the reference of the HBM byte counters
        from fft_long_convolution_amd.fftconv import stream_copy
        esz = 4 if w.dtype == "f32" else 2
        a = torch.ones(w.rows * w.N * esz // 4, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(args.steps or 100):
            stream_copy(a, b)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_each_way": a.numel() * 4,
                          "copies": args.steps or 100}))
        return
    if (args.gated + args.circular + args.backward + (args.lowpass is not None)
            + (args.blocksparse is not None)) > 1:
        print("bench.py: choose one of --gated, --circular, --backward, "
              "--lowpass, --blocksparse", file=sys.stderr)
        sys.exit(2)
    op = ("gated" if args.gated else "circular" if args.circular
          else "backward" if args.backward
          else "lowpass" if args.lowpass is not None
          else "blocksparse" if args.blocksparse is not None else "plain")
    bs_a, bs_d = ((int(x) for x in args.blocksparse.split(","))
                  if args.blocksparse is not None else (0, 0))
    # the circular operator runs on the plan at FFT size N
    conv = FFTConv(w.N, dtype=w.dtype, circular=(op == "circular"))
    info = conv.info

    # ---- inputs (seeded, synthetic) resident in HBM before timing
    t0 = time.time()
    u_np = inputs.input_rows(w)
    k_np = inputs.kernel_rows(w)
    if op == "gated":
        g_np = [inputs.gate_rows(w, "w"), inputs.gate_rows(w, "v")]
    elif op == "backward":
        g_np = [inputs.dy_rows(w)]
    else:
        g_np = []
    gen_s = time.time() - t0
    u0 = to_torch(u_np, w.dtype, torch).view(w.B, w.H, w.N).to(dev)
    g0 = [to_torch(a, w.dtype, torch).view(w.B, w.H, w.N).to(dev) for a in g_np]
    k = torch.from_numpy(k_np).to(dev)
    kind = {"circular": "circular", "backward": "causal_adjoint"}.get(op, "causal")
    if op == "lowpass":
        kf = conv.kernel_spectrum_lowpass(k, args.lowpass)
    elif op == "blocksparse":
        kf = conv.kernel_spectrum_blocksparse(k, bs_a, bs_d)
    else:
        kf = conv.kernel_spectrum(k, kind=kind)
    esz = 4 if w.dtype == "f32" else 2
    # [B][H][N] streams per step: u and y, + the two gates (gated), or u, dy
    # and du (backward, which also writes the fp32 [H][N] dk)
    nstream = {"gated": 4, "backward": 3}.get(op, 2)
    set_bytes = nstream * w.rows * w.N * esz
    nsets = max(1, min(8, -(-ROTATE_BYTES // set_bytes)))
    us = [u0] + [u0.clone() for _ in range(nsets - 1)]
    gs = [g0] + [[g.clone() for g in g0] for _ in range(nsets - 1)]
    ys = [torch.empty_like(u0) for _ in range(nsets)]
    dks = ([torch.empty(w.H, w.N, dtype=torch.float32, device=dev)
            for _ in range(nsets)] if op == "backward" else [])
    wsb = (conv.backward_workspace_bytes(w.B, w.H) if op == "backward"
           else conv.workspace_bytes(w.B, w.H))
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step(i):
        j = i % nsets
        if op == "gated":
            conv.forward_gated(us[j], gs[j][0], gs[j][1], kf, out=ys[j],
                               workspace=ws)
        elif op == "backward":
            conv.backward(us[j], gs[j][0], kf, workspace=ws, out_du=ys[j],
                          out_dk=dks[j])
        elif op == "lowpass":
            conv.forward_lowpass(us[j], kf, args.lowpass, out=ys[j], workspace=ws)
        elif op == "blocksparse":
            conv.forward_blocksparse(us[j], kf, bs_a, bs_d, out=ys[j], workspace=ws)
        else:
            conv.forward(us[j], kf, out=ys[j], workspace=ws)

    # ---- warmup, then K timed steps between two HIP events recorded on the
    # stream the kernels are launched on (launches back to back)
    stream = torch.cuda.current_stream()
    if args.steps is None or args.warmup is None:
        # estimate the step time (these calls are untimed warmup too)
        for i in range(3):
            step(i)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(10):
            step(i)
        e1.record(stream)
        torch.cuda.synchronize()
        est = max(e0.elapsed_time(e1) / 10, 1e-3)
        if args.warmup is None:
            args.warmup = max(20, int(math.ceil(300.0 / est)))
        if args.steps is None:
            args.steps = max(100, int(math.ceil(1000.0 / est)))
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    # per-step spread from individually bracketed launches
    per = []
    for i in range(min(args.steps, 20)):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step(i)
        b.record(stream)
        per.append((a, b))
    torch.cuda.synchronize()
    ms_med = float(np.median([a.elapsed_time(b) for a, b in per]))
    outputs = w.rows * w.N
    value = outputs / (ms_step * 1e-3)

    # ---- roofline of the dominant kernel: algorithmic bytes and flops per
    # forward call over its average duration in the timed region (HIP events
    # on the launch stream around K back-to-back calls; a kernel trace's
    # average agrees up to the gaps between launches).  Individually
    # bracketed launches (ms_median_single_launch) also carry the events' own
    # overhead.
    kf_bytes = kf_min_bytes(info, w.H)
    alg_bytes = nstream * w.rows * w.N * esz + kf_bytes
    if op == "backward":
        alg_bytes += w.H * w.N * 4
    ms_kernel = ms_step
    achieved_gbs = alg_bytes / (ms_kernel * 1e-3) / 1e9
    # matrix-core flops: one forward call's; the backward counts two (du is
    # one forward call, dk two forward transforms per row)
    flops = info["mfma_flops_per_row"] * w.rows * (2 if op == "backward" else 1)
    achieved_tf = flops / (ms_kernel * 1e-3) / 1e12
    t_hbm = alg_bytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (MFMA_PEAK_TFLOPS[w.dtype] * 1e12)
    bound = "hbm" if t_hbm >= t_mfma else "mfma"
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": round(achieved_gbs, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved_gbs / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(achieved_tf, 2),
                "peak": MFMA_PEAK_TFLOPS[w.dtype], "unit": "TFLOP/s",
                "frac": round(achieved_tf / MFMA_PEAK_TFLOPS[w.dtype], 4)}
    roof["traffic"] = measured_traffic(w.name + ("" if op == "plain" else "_" + op))
    roof["kernel"] = info["kernel"] + ("+kgrad" if op == "backward" else "")
    roof["algorithmic_bytes"] = int(alg_bytes)
    roof["kf_stored_bytes"] = int(conv.spectrum_bytes(w.H))
    roof["mfma_flops"] = float(flops)
    roof["mfma_frac"] = round(achieved_tf / MFMA_PEAK_TFLOPS[w.dtype], 4)
    roof["launch_ms"] = round(ms_kernel, 5)
    # the practical roof: the library's streaming copy (read + write) on
    # this GPU, measured in the same run
    copy_gbs = stream_copy_rate(torch, dev)
    roof["copy_gbs"] = round(copy_gbs, 1)
    roof["frac_of_copy"] = round(achieved_gbs / copy_gbs, 4) if bound == "hbm" else None

    # ---- sampled correctness of the timed output against the oracle
    import oracle
    y_last = ys[(args.steps - 1) % nsets].view(w.rows, w.N)
    rng = np.random.default_rng(7)
    rows = rng.integers(0, w.rows, 48)
    ts = rng.integers(0, w.N, 48)
    ts[:4] = [0, w.N - 1, 1, w.N // 2]
    sel_u = oracle.to_f64(u_np[rows], w.dtype)
    sel_k = k_np.astype(np.float64)
    got = y_last[torch.from_numpy(rows).to(dev), torch.from_numpy(ts).to(dev)]
    got = got.float().cpu().numpy().astype(np.float64)
    if op == "gated":
        sel_w, sel_v = (oracle.to_f64(a[rows], w.dtype) for a in g_np)
        want = oracle.gated_points(sel_u, sel_w, sel_v, sel_k, np.arange(48),
                                   ts, rows % w.H)
    elif op == "circular":
        want = oracle.op_points(sel_u, sel_k, "circular", np.arange(48), ts,
                                rows % w.H)
    elif op == "backward":
        sel_dy = oracle.to_f64(g_np[0][rows], w.dtype)
        want = oracle.op_points(sel_dy, sel_k, "causal_adjoint", np.arange(48),
                                ts, rows % w.H)
    elif op == "lowpass":
        # the band-limited route over the sampled rows, then the samples
        uh, inv = np.unique(rows % w.H, return_inverse=True)
        full = oracle.lowpass_fft(sel_u, sel_k[uh], args.lowpass, inv)
        want = full[np.arange(48), ts]
    elif op == "blocksparse":
        uh, inv = np.unique(rows % w.H, return_inverse=True)
        full = oracle.blocksparse_fft(sel_u, sel_k[uh], info["sparse_outer"], bs_a, bs_d, inv)
        want = full[np.arange(48), ts]
    else:
        want = oracle.conv_points(sel_u, sel_k, np.arange(48), ts, rows % w.H)
    scale = float(np.sqrt(np.mean(want ** 2))) or 1.0
    sample_err = float(np.max(np.abs(got - want)) / scale)
    if op == "backward":
        # dk at a few taps of two channels (all batch rows of each)
        hs_sel = np.unique(rng.integers(0, w.H, 2))
        rsel = np.array([b * w.H + h for h in hs_sel for b in range(w.B)])
        hloc = np.repeat(np.arange(len(hs_sel)), w.B)
        js = rng.integers(0, w.N, 8)
        js[:2] = [0, w.N - 1]
        hq = np.repeat(np.arange(len(hs_sel)), len(js))
        jq = np.tile(js, len(hs_sel))
        want_k = oracle.kgrad_points(oracle.to_f64(u_np[rsel], w.dtype),
                                     oracle.to_f64(g_np[0][rsel], w.dtype),
                                     len(hs_sel), hq, jq, "causal", hloc)
        dk_last = dks[(args.steps - 1) % nsets].cpu().numpy().astype(np.float64)
        got_k = dk_last[hs_sel[hq], jq]
        sk = float(np.sqrt(np.mean(want_k ** 2))) or 1.0
        sample_err = max(sample_err, float(np.max(np.abs(got_k - want_k)) / sk))

    # ---- CPU baseline: the fp64 oracle on a bounded sample of the rows
    cpu = None
    if not args.no_cpu:
        cores = oracle.num_threads()
        hidx = np.arange(w.rows) % w.H

        def cpu_run(n, passes=1):
            # inputs converted once; the timed region is the oracle's route
            # over the first n rows, `passes` times
            uh, inv = np.unique(hidx[:n], return_inverse=True)
            usel = oracle.to_f64(u_np[:n], w.dtype)
            ksel = k_np[uh].astype(np.float64)
            gsel = [oracle.to_f64(a[:n], w.dtype) for a in g_np]
            t0 = time.perf_counter()
            for _ in range(passes):
                if op == "gated":
                    oracle.gated_fft(usel, gsel[0], gsel[1], ksel, inv)
                elif op == "circular":
                    oracle.op_fft(usel, ksel, "circular", inv)
                elif op == "backward":
                    oracle.op_fft(gsel[0], ksel, "causal_adjoint", inv)
                    oracle.kgrad_fft(usel, gsel[0], len(uh), "causal", inv)
                elif op == "lowpass":
                    oracle.lowpass_fft(usel, ksel, args.lowpass, inv)
                elif op == "blocksparse":
                    oracle.blocksparse_fft(usel, ksel, info["sparse_outer"], bs_a, bs_d, inv)
                else:
                    oracle.conv_fft(usel, ksel, inv)
            return time.perf_counter() - t0
        probe = int(min(w.rows, max(1, (1 << 22) // w.N)))
        tp = cpu_run(probe)
        n = int(min(w.rows, max(probe, probe * args.cpu_seconds / max(tp, 1e-6))))
        passes = 1
        if n == w.rows:
            # the whole workload takes less than the sample time: repeat it
            # (the probe's rate predicts one pass)
            one = tp * w.rows / probe
            passes = int(min(100, max(1, round(args.cpu_seconds / max(one, 1e-6)))))
        tc = cpu_run(n, passes)
        what = {"gated": " with both gates", "circular": " (circular kind)",
                "backward": " (du by the adjoint and dk by the gradient "
                            "routes)",
                "lowpass": " (band-limited spectrum)",
                "blocksparse": " (digit-block sparse spectrum)"}.get(op, "")
        cpu = {"value": round(passes * n * w.N / tc, 1), "unit": "outputs/s",
               "cores": cores, "kind": "oracle",
               "sample": "%s%d of %d rows (B*H) at N=%d through the fp64 "
                         "radix-2 FFT route of the oracle%s, kernel spectra "
                         "included; %.1f s" % ("%d passes over " % passes if passes > 1 else "",
                                               n, w.rows, w.N, what, tc)}

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "outputs/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name + ("" if op == "plain" else " " + op),
                   "op": op, "cutoff": args.lowpass,
                   "blocksparse": ({"a": bs_a, "d": bs_d, "P": info["sparse_outer"],
                                    "sparsity": round(1.0 - float(
                                        __import__("oracle").blocksparse_mask(
                                            w.N, info["sparse_outer"], bs_a, bs_d).mean()), 4)}
                                   if op == "blocksparse" else None),
                   "B": w.B, "H": w.H, "N": w.N,
                   "io_dtype": w.dtype, "factors": info["factors"],
                   "path": info["path"], "global_batch": w.B,
                   "seq_len": w.N, "parallelism": "single-gpu"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "timing": {"ms_median_single_launch": round(ms_med, 5),
                   "wall_ms_per_step": round(wall / args.steps * 1e3, 5),
                   "buffer_sets": nsets,
                   "sampled_max_err_over_rms": sample_err,
                   "input_gen_s": round(gen_s, 2)},
    }
    if op == "plain" and not args.no_extra:
        # the other workloads, each timed the same way (one call per step,
        # inputs resident, HIP events around back-to-back calls)
        del us, gs, ys, ws, u0, g0, kf, k, dks
        torch.cuda.empty_cache()
        line["workloads"] = {n: time_workload(n, torch, dev)
                             for n in inputs.WORKLOADS if n != w.name}
    if op == "circular" and not args.no_extra:
        # the same workload on the causal plan (2N-point transform): its
        # causal call, and the circular operator through it (the doubled
        # kernel), each timed the same way
        del us, gs, ys, ws, u0, g0, kf, k, dks
        torch.cuda.empty_cache()
        line["compare"] = {
            "causal_plan_causal": time_workload(w.name, torch, dev),
            "causal_plan_circular_2n": time_workload(w.name, torch, dev, kind="circular")}
    print(json.dumps(line), flush=True)


def stream_copy_rate(torch, dev, nbytes=1 << 30, reps=20) -> float:
    """GB/s (bytes read + written) of fftconv_stream_copy over 1 GB."""
    from fft_long_convolution_amd.fftconv import stream_copy
    a = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(5):
        stream_copy(a, b)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    st = torch.cuda.current_stream()
    e0.record(st)
    for _ in range(reps):
        stream_copy(a, b)
    e1.record(st)
    torch.cuda.synchronize()
    return 2.0 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9


def time_workload(name: str, torch, dev, kind: str = "causal") -> dict:
    """One workload's forward call on the plan of fftconv_plan, its spectrum
    of operator `kind`, timed as the main line (>= 0.2 s warmup, ~0.5 s
    timed); its roofline fraction against the spec HBM peak."""
    from fft_long_convolution_amd import inputs
    from fft_long_convolution_amd.fftconv import FFTConv
    w = inputs.WORKLOADS[name]
    conv = FFTConv(w.N, dtype=w.dtype)
    u = to_torch(inputs.input_rows(w), w.dtype, torch).view(w.B, w.H, w.N).to(dev)
    k = torch.from_numpy(inputs.kernel_rows(w)).to(dev)
    kf = conv.kernel_spectrum(k, kind=kind)
    y = torch.empty_like(u)
    ws = torch.empty(max(conv.workspace_bytes(w.B, w.H), 16), dtype=torch.uint8, device=dev)
    st = torch.cuda.current_stream()

    def region(n):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(n):
            conv.forward(u, kf, out=y, workspace=ws)
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    est = max(region(3), 1e-3)
    region(max(5, int(math.ceil(200.0 / est))))
    steps = max(20, int(math.ceil(500.0 / est)))
    ms = region(steps)
    esz = 4 if w.dtype == "f32" else 2
    alg = 2 * w.rows * w.N * esz + kf_min_bytes(conv.info, w.H)
    gbs = alg / (ms * 1e-3) / 1e9
    out = {"ms_per_step": round(ms, 5), "steps": steps,
           "outputs_per_s": round(w.rows * w.N / (ms * 1e-3), 1),
           "kernel": conv.info["kernel"], "factors": conv.info["factors"],
           "algorithmic_bytes": int(alg), "achieved_gbs": round(gbs, 1),
           "frac": round(gbs / HBM_PEAK_GBS, 4)}
    del conv, u, k, kf, y, ws
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------- profiling
#
# --profile runs this script under rocprofv3 as child processes (the
# profiler's own program after "--", never through a shell): one kernel
# trace at the default lengths, then one counter pass per group below on a
# short run (1 warmup + 4 timed + 4 bracketed calls = 9 calls), and the same
# HBM byte counters on the library's streaming copy of the workload's input
# size, whose known bytes calibrate them.  It writes
# profiles/<kernel>_<workload>[_<op>].md and the HBM traffic record of
# profiles/traffic.json (tied to the sha1 of the library sources).

PMC_PASSES = [
    ["FETCH_SIZE"],
    ["WRITE_SIZE"],
    ["SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_WAVES",
     "SQ_BUSY_CU_CYCLES", "SQ_WAVE_CYCLES", "SQ_WAIT_INST_ANY", "GRBM_GUI_ACTIVE"],
    ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_LDS_BANK_CONFLICT",
     "SQ_LDS_IDX_ACTIVE", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_ANY", "GRBM_GUI_ACTIVE"],
]
# kernels of the untimed set-up (kernel spectrum), not of a call
SETUP_KERNELS = ("kpad_kernel", "stockham_kernel", "alphabeta_kernel", "coef_kernel",
                 "band_limit_kernel")


def _op_flags(args):
    if args.gated:
        return ["--gated"], "gated"
    if args.circular:
        return ["--circular"], "circular"
    if args.backward:
        return ["--backward"], "backward"
    if args.lowpass is not None:
        return ["--lowpass", str(args.lowpass)], "lowpass"
    if args.blocksparse is not None:
        return ["--blocksparse", args.blocksparse], "blocksparse"
    return [], "plain"


def _is_call_kernel(name: str) -> bool:
    return "fftconv::" in name and not any(k in name for k in SETUP_KERNELS) \
        and "stream_copy" not in name


def _run(cmd, log):
    import subprocess
    env = dict(os.environ, TMPDIR="/tmp")
    print("profile: " + " ".join(cmd), flush=True)
    r = subprocess.run(cmd, cwd="/tmp", env=env, capture_output=True, text=True, timeout=900)
    with open(log, "w") as f:
        f.write(r.stdout + "\n---- stderr ----\n" + r.stderr)
    if r.returncode != 0:
        raise RuntimeError("%s exited with %d (log %s)" % (cmd[0], r.returncode, log))
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    return json.loads(lines[-1]) if lines else None


def _csv_rows(root: str, suffix: str):
    import csv
    import glob
    rows = []
    for path in glob.glob(os.path.join(root, "**", "*" + suffix), recursive=True):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def _kernel_short(name: str) -> str:
    import re
    m = re.search(r"fftconv::(\w+)", name)
    return m.group(1) if m else name


def _counters(root: str, pred, by_kernel=None) -> dict:
    """Counter totals over the kernels `pred` accepts; with a dict
    `by_kernel`, also the totals per kernel (short name) added into it."""
    tot = {}
    for r in _csv_rows(root, "counter_collection.csv"):
        if not pred(r.get("Kernel_Name", "")):
            continue
        n = r["Counter_Name"]
        v = float(r["Counter_Value"])
        tot[n] = tot.get(n, 0.0) + v
        if by_kernel is not None:
            d = by_kernel.setdefault(_kernel_short(r["Kernel_Name"]), {})
            d[n] = d.get(n, 0.0) + v
    return tot


def profile(args):
    from fft_long_convolution_amd import inputs
    from fft_long_convolution_amd.fftconv import plan_query
    w = inputs.WORKLOADS[args.workload]
    flags, op = _op_flags(args)
    tag = w.name + ("" if op == "plain" else "_" + op)
    info = plan_query(w.N, 0, w.dtype, circular=(op == "circular"))
    out = os.path.join(os.path.abspath(args.profile_dir), tag)
    os.makedirs(out, exist_ok=True)
    me = [sys.executable, os.path.abspath(__file__), "--workload", w.name, "--no-extra"] + flags
    short = ["--steps", "4", "--warmup", "1", "--no-cpu"]
    calls_short = 1 + 4 + 4
    # 1. kernel trace at the default lengths
    tcmd = ["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv",
            "-d", os.path.join(out, "trace"), "-o", "trace", "--"] + me + ["--no-cpu"]
    tline = _run(tcmd, os.path.join(out, "trace.log"))
    calls = 13 + tline["warmup"] + tline["steps"] + min(tline["steps"], 20)
    stats = [r for r in _csv_rows(os.path.join(out, "trace"), "kernel_stats.csv")
             if _is_call_kernel(r["Name"])]
    trace_ns = sum(float(r["TotalDurationNs"]) for r in stats) / calls
    # 2. counters on short runs, and on the calibration copy
    pmc = {}
    per_k = {}
    for i, group in enumerate(PMC_PASSES):
        d = os.path.join(out, "pmc%d" % i)
        _run(["rocprofv3", "--pmc"] + group + ["--output-format", "csv", "-d", d, "-o", "pmc", "--"]
             + me + short, d + ".log")
        for k, v in _counters(d, _is_call_kernel, per_k).items():
            pmc[k] = v / calls_short
    cal = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        d = os.path.join(out, "copy_" + c)
        _run(["rocprofv3", "--pmc", c, "--output-format", "csv", "-d", d, "-o", "pmc", "--",
              sys.executable, os.path.abspath(__file__), "--workload", w.name,
              "--steps", "4", "--copy-calibration"], d + ".log")
        cal.update({k: v / 4 for k, v in _counters(d, lambda n: "stream_copy" in n).items()})
    esz = 4 if w.dtype == "f32" else 2
    copy_bytes = w.rows * w.N * esz
    f_scale = copy_bytes / (cal["FETCH_SIZE"] * 1024.0)
    w_scale = copy_bytes / (cal["WRITE_SIZE"] * 1024.0)
    traffic = int(round(pmc["FETCH_SIZE"] * 1024.0 * f_scale + pmc["WRITE_SIZE"] * 1024.0 * w_scale))
    alg = tline["roofline"]["algorithmic_bytes"]
    rows = w.rows
    # 3. summary
    kern = info["kernel"].split("+")[0] if op != "backward" else info["kernel"].split("+")[0] + "_kgrad"
    name = "%s_%s%s.md" % (kern, w.name, "" if op == "plain" else "_" + op)
    # GRBM_GUI_ACTIVE is reported once per XCD (8 on MI355X): the call's
    # busy cycles are the per-XCD value
    gui = pmc.get("GRBM_GUI_ACTIVE", 0.0) / 8.0
    simd = 4 * 256
    lines = [
        "# %s -- workload %s%s" % (kern, w.name, "" if op == "plain" else " (%s)" % op), "",
        "Workload %s: B=%d, H=%d, N=%d, %s I/O, factors %s, %s path; kernels of a call: %s." % (
            w.name, w.B, w.H, w.N, w.dtype, info["factors"], info["path"], info["kernel"]), "",
        "Generated by `python3 bench.py --profile --workload %s%s` (rocprofv3 runs of bench.py "
        "as child processes, from /tmp with TMPDIR=/tmp; `<repo>` is the repository root)." % (
            w.name, (" " + " ".join(flags)) if flags else ""), "",
        "## Kernel trace", "", "```",
        " ".join(tcmd).replace(os.path.join(out, "trace"), "<out>/trace")
        .replace(os.path.dirname(os.path.abspath(__file__)), "<repo>"), "```", "",
        "| kernel | calls | average ns | min ns | max ns |", "|---|---|---|---|---|"]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append("| `%s` | %s | %.0f | %s | %s |" % (r["Name"], r["Calls"], float(r["AverageNs"]),
                                                      r["MinNs"], r["MaxNs"]))
    lines += ["", "Kernel time per call in the trace: %.2f us over %d calls; the traced run's own "
              "line reports ms_per_step %.5f (%.2f us per call, the gaps between launches "
              "included)." % (trace_ns / 1e3, calls, tline["ms_per_step"], tline["ms_per_step"] * 1e3),
              "", "## bench.py line of the traced run", "", "```", json.dumps(tline), "```", "",
              "## Counters per call (rocprofv3 --pmc, one pass per group, %d calls per run)" % calls_short,
              "", "```"]
    for i, group in enumerate(PMC_PASSES):
        lines.append("rocprofv3 --pmc %s -- python3 <repo>/bench.py --workload %s%s %s" % (
            " ".join(group), w.name, (" " + " ".join(flags)) if flags else "", " ".join(short)))
    lines += ["rocprofv3 --pmc FETCH_SIZE (and WRITE_SIZE) -- python3 <repo>/bench.py --workload %s "
              "--steps 4 --copy-calibration" % w.name, "```", "",
              "| counter | per call |", "|---|---|"]
    for k in sorted(pmc):
        lines.append("| %s | %.6g |" % (k, pmc[k]))
    lines += ["",
              "| HBM bytes | FETCH_SIZE KiB | WRITE_SIZE KiB |", "|---|---|---|",
              "| streaming copy of %d B | %.1f | %.1f |" % (copy_bytes, cal["FETCH_SIZE"], cal["WRITE_SIZE"]),
              "| scale factor (true bytes / counter) | %.4f | %.4f |" % (f_scale, w_scale),
              "| one call | %.1f | %.1f |" % (pmc["FETCH_SIZE"], pmc["WRITE_SIZE"]), "",
              "HBM traffic per call %d B vs algorithmic %d B: ratio %.3f." % (traffic, alg, traffic / alg), ""]
    if len(per_k) > 1:
        # the same counters kernel by kernel (per call), with each kernel's
        # HBM bytes and rate over its traced time per call
        ks = sorted(per_k)
        tper = {}
        for r in stats:
            k = _kernel_short(r["Name"])
            tper[k] = tper.get(k, 0.0) + float(r["TotalDurationNs"]) / calls
        lines += ["Per kernel (per call):", "",
                  "| counter | " + " | ".join("`%s`" % k for k in ks) + " |",
                  "|---|" + "---|" * len(ks)]
        for c in sorted({c for k in ks for c in per_k[k]}):
            lines.append("| %s | " % c + " | ".join("%.6g" % (per_k[k].get(c, 0.0) / calls_short)
                                                  for k in ks) + " |")
        hb = {k: (per_k[k].get("FETCH_SIZE", 0.0) * f_scale + per_k[k].get("WRITE_SIZE", 0.0) * w_scale)
              * 1024.0 / calls_short for k in ks}
        lines.append("| HBM bytes (scaled) | " + " | ".join("%.4g" % hb[k] for k in ks) + " |")
        lines.append("| traced us per call | " + " | ".join("%.2f" % (tper.get(k, 0.0) / 1e3) for k in ks) + " |")
        lines.append("| HBM TB/s | " + " | ".join(
            "%.2f" % (hb[k] / (tper[k] * 1e-9) / 1e12 if tper.get(k) else 0.0) for k in ks) + " |")
        lines.append("| vector instructions per row | " + " | ".join(
            "%.1f" % (per_k[k].get("SQ_INSTS_VALU", 0.0) / calls_short / rows) for k in ks) + " |")
        lines.append("")
    if gui > 0:
        lines += ["Derived (GRBM_GUI_ACTIVE = %.0f cycles per call per XCD, %d SIMDs):" % (gui, simd), "",
                  "* matrix cores busy: %.1f%% of SIMD cycles (SQ_VALU_MFMA_BUSY_CYCLES)" % (
                      100.0 * pmc.get("SQ_VALU_MFMA_BUSY_CYCLES", 0) / (gui * simd)),
                  "* vector instructions per row: %.1f wave-instructions (SQ_INSTS_VALU / rows)" % (
                      pmc.get("SQ_INSTS_VALU", 0) / rows),
                  "* matrix instructions per row: %.1f (SQ_INSTS_MFMA / rows)" % (
                      pmc.get("SQ_INSTS_MFMA", 0) / rows),
                  "* LDS instructions per row: %.1f; bank-conflict cycles / LDS-active cycles: %.3f" % (
                      pmc.get("SQ_INSTS_LDS", 0) / rows,
                      pmc.get("SQ_LDS_BANK_CONFLICT", 0) / max(pmc.get("SQ_LDS_IDX_ACTIVE", 1), 1)),
                  "* waves waiting for an issue slot: %.1f%% of wave cycles (SQ_WAIT_INST_ANY / "
                  "SQ_WAVE_CYCLES)" % (100.0 * pmc.get("SQ_WAIT_INST_ANY", 0) /
                                       max(pmc.get("SQ_WAVE_CYCLES", 1), 1)), ""]
    os.makedirs(args.profile_out, exist_ok=True)
    with open(os.path.join(args.profile_out, name), "w") as f:
        f.write("\n".join(lines) + "\n")
    tfile = os.path.join(args.profile_out, "traffic.json")
    rec = {}
    for src in (tfile, TRAFFIC_FILE):
        try:
            with open(src) as f:
                rec = json.load(f)
            break
        except (OSError, ValueError):
            continue
    rec[tag] = {"traffic_bytes": traffic, "algorithmic_bytes": alg,
                "source_sha1": kernel_source_hash(), "summary": "profiles/" + name}
    with open(tfile, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    print(json.dumps({"profile": "profiles/" + name, "traffic_bytes": traffic,
                      "algorithmic_bytes": alg, "trace_us_per_call": round(trace_ns / 1e3, 3)}),
          flush=True)


if __name__ == "__main__":
    main()
