"""Shared helpers for the GPU parity tests: run the HIP library on seeded
workload rows and compare with the fp64 oracle."""
from __future__ import annotations

import numpy as np

import oracle
from fft_long_convolution_amd import inputs

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}


def to_torch(a: np.ndarray, dtype: str, device="cuda"):
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device)


def from_torch(t, dtype: str) -> np.ndarray:
    import torch
    t = t.detach().cpu()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def run_gpu(w: inputs.Workload, conv=None, p: int = 0):
    """GPU result for all rows of workload w, as fp64 [rows, N]."""
    import torch
    from fft_long_convolution_amd.fftconv import FFTConv
    if conv is None:
        conv = FFTConv(w.N, p=p, dtype=w.dtype)
    u = inputs.input_rows(w)
    k = inputs.kernel_rows(w)
    ud = to_torch(u, w.dtype).view(w.B, w.H, w.N)
    kd = torch.from_numpy(k).cuda()
    kf = conv.kernel_spectrum(kd)
    y = conv.forward(ud, kf)
    torch.cuda.synchronize()
    y64 = oracle.to_f64(from_torch(y, w.dtype).reshape(w.rows, w.N), w.dtype)
    return y64, u, k


def oracle_rows(w: inputs.Workload, u: np.ndarray, k: np.ndarray):
    """fp64 oracle for the same rows (FFT route; direct when N is small)."""
    u64 = oracle.to_f64(u, w.dtype).reshape(w.rows, w.N)
    k64 = k.astype(np.float64)
    hidx = np.arange(w.rows) % w.H
    if w.N <= 512:
        return oracle.conv_direct(u64, k64, hidx)
    return oracle.conv_fft(u64, k64, hidx)


def parity(w: inputs.Workload, p: int = 0):
    y, u, k = run_gpu(w, p=p)
    ref = oracle_rows(w, u, k)
    return oracle.rel_l2(y, ref), y, ref


def run_gpu_gated(w: inputs.Workload, conv=None, p: int = 0):
    """GPU gated result v * conv(u * w, k) for all rows, as fp64."""
    import torch
    from fft_long_convolution_amd.fftconv import FFTConv
    if conv is None:
        conv = FFTConv(w.N, p=p, dtype=w.dtype)
    u = inputs.input_rows(w)
    gw = inputs.gate_rows(w, "w")
    gv = inputs.gate_rows(w, "v")
    k = inputs.kernel_rows(w)
    dev = [to_torch(a, w.dtype).view(w.B, w.H, w.N) for a in (u, gw, gv)]
    kf = conv.kernel_spectrum(torch.from_numpy(k).cuda())
    y = conv.forward_gated(dev[0], dev[1], dev[2], kf)
    torch.cuda.synchronize()
    y64 = oracle.to_f64(from_torch(y, w.dtype).reshape(w.rows, w.N), w.dtype)
    return y64, (u, gw, gv), k


def oracle_gated_rows(w: inputs.Workload, ins, k: np.ndarray):
    """fp64 oracle of the gated convolution for the same rows."""
    u64, w64, v64 = (oracle.to_f64(a, w.dtype).reshape(w.rows, w.N)
                     for a in ins)
    k64 = k.astype(np.float64)
    hidx = np.arange(w.rows) % w.H
    if w.N <= 512:
        return oracle.gated_direct(u64, w64, v64, k64, hidx)
    return oracle.gated_fft(u64, w64, v64, k64, hidx)


def parity_gated(w: inputs.Workload, p: int = 0):
    y, ins, k = run_gpu_gated(w, p=p)
    ref = oracle_gated_rows(w, ins, k)
    return oracle.rel_l2(y, ref), y, ref


def run_gpu_op(w: inputs.Workload, kind: str, conv=None):
    """GPU result of operator ``kind`` (a spectrum of that kind fed to the
    plain forward call) for all rows, as fp64."""
    import torch
    from fft_long_convolution_amd.fftconv import FFTConv
    if conv is None:
        conv = FFTConv(w.N, dtype=w.dtype)
    u = inputs.input_rows(w)
    k = inputs.kernel_rows(w)
    ud = to_torch(u, w.dtype).view(w.B, w.H, w.N)
    kf = conv.kernel_spectrum(torch.from_numpy(k).cuda(), kind=kind)
    y = conv.forward(ud, kf)
    torch.cuda.synchronize()
    y64 = oracle.to_f64(from_torch(y, w.dtype).reshape(w.rows, w.N), w.dtype)
    return y64, u, k


def parity_op(w: inputs.Workload, kind: str):
    y, u, k = run_gpu_op(w, kind)
    u64 = oracle.to_f64(u, w.dtype).reshape(w.rows, w.N)
    hidx = np.arange(w.rows) % w.H
    if w.N <= 512:
        ref = oracle.op_direct(u64, k.astype(np.float64), kind, hidx)
    else:
        ref = oracle.op_fft(u64, k.astype(np.float64), kind, hidx)
    return oracle.rel_l2(y, ref), y, ref


def run_gpu_backward(w: inputs.Workload, conv=None):
    """GPU (du, dk) of the causal convolution for dy = inputs.dy_rows, as
    fp64 [rows, N] and [H, N]."""
    import torch
    from fft_long_convolution_amd.fftconv import FFTConv
    if conv is None:
        conv = FFTConv(w.N, dtype=w.dtype)
    u = inputs.input_rows(w)
    dy = inputs.dy_rows(w)
    k = inputs.kernel_rows(w)
    ud = to_torch(u, w.dtype).view(w.B, w.H, w.N)
    dyd = to_torch(dy, w.dtype).view(w.B, w.H, w.N)
    kfa = conv.kernel_spectrum(torch.from_numpy(k).cuda(), kind="causal_adjoint")
    du, dk = conv.backward(ud, dyd, kfa)
    torch.cuda.synchronize()
    du64 = oracle.to_f64(from_torch(du, w.dtype).reshape(w.rows, w.N), w.dtype)
    dk64 = dk.cpu().numpy().astype(np.float64)
    return du64, dk64, u, dy, k


def oracle_backward(w: inputs.Workload, u, dy, k):
    u64 = oracle.to_f64(u, w.dtype).reshape(w.rows, w.N)
    dy64 = oracle.to_f64(dy, w.dtype).reshape(w.rows, w.N)
    hidx = np.arange(w.rows) % w.H
    k64 = k.astype(np.float64)
    if w.N <= 512:
        du = oracle.op_direct(dy64, k64, "causal_adjoint", hidx)
        dk = oracle.kgrad_direct(u64, dy64, w.H, "causal", hidx)
    else:
        du = oracle.op_fft(dy64, k64, "causal_adjoint", hidx)
        dk = oracle.kgrad_fft(u64, dy64, w.H, "causal", hidx)
    return du, dk


def run_gpu_circular(w: inputs.Workload, kind: str = "circular", conv=None, gated: bool = False,
                     p: int = 0):
    """GPU result of a plan at FFT size N (fftconv_plan_circular) for all
    rows of w, operator ``kind`` (circular or circular_adjoint), as fp64;
    gated: v * op(u * w)."""
    import torch
    from fft_long_convolution_amd.fftconv import FFTConv
    if conv is None:
        conv = FFTConv(w.N, p=p, dtype=w.dtype, circular=True)
    u = inputs.input_rows(w)
    k = inputs.kernel_rows(w)
    kf = conv.kernel_spectrum(torch.from_numpy(k).cuda(), kind=kind)
    ins = (u,)
    if gated:
        ins = (u, inputs.gate_rows(w, "w"), inputs.gate_rows(w, "v"))
        dev = [to_torch(a, w.dtype).view(w.B, w.H, w.N) for a in ins]
        y = conv.forward_gated(dev[0], dev[1], dev[2], kf)
    else:
        y = conv.forward(to_torch(u, w.dtype).view(w.B, w.H, w.N), kf)
    torch.cuda.synchronize()
    y64 = oracle.to_f64(from_torch(y, w.dtype).reshape(w.rows, w.N), w.dtype)
    return y64, ins, k


def oracle_circular(w: inputs.Workload, ins, k, kind: str = "circular"):
    """fp64 oracle of the same rows: the operator by its definition (small
    N) or the oracle's FFT route; with three inputs the gated form."""
    u64 = oracle.to_f64(ins[0], w.dtype).reshape(w.rows, w.N)
    k64 = k.astype(np.float64)
    hidx = np.arange(w.rows) % w.H
    if len(ins) == 3:
        g = [oracle.to_f64(a, w.dtype).reshape(w.rows, w.N) for a in ins[1:]]
        u64 = u64 * g[0]
    if w.N <= 512:
        ref = oracle.op_direct(u64, k64, kind, hidx)
    else:
        ref = oracle.op_fft(u64, k64, kind, hidx)
    if len(ins) == 3:
        ref = g[1] * ref
    return ref
