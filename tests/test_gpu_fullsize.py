"""Parity at the full workload sizes, in the launch configuration bench.py
times (one fftconv_forward over the whole [B][H][N] tensor).

For every workload the whole output is compared with the fp64 oracle's FFT
route (streamed in row chunks), and a sample of single outputs is compared
with the convolution definition computed one by one (including t = 0,
t = N-1 and, for the genome workload, both sides of the end of its
one-hot region).
"""
import sys

import numpy as np
import pytest

import oracle
from fft_long_convolution_amd import inputs
from tests.gpu_helpers import TOL, from_torch, to_torch

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _run_full(w):
    import torch
    from fft_long_convolution_amd.fftconv import FFTConv
    conv = FFTConv(w.N, dtype=w.dtype)
    u = inputs.input_rows(w)
    k = inputs.kernel_rows(w)
    ud = to_torch(u, w.dtype).view(w.B, w.H, w.N)
    kf = conv.kernel_spectrum(torch.from_numpy(k).cuda())
    y = conv.forward(ud, kf)
    torch.cuda.synchronize()
    yh = from_torch(y, w.dtype).reshape(w.rows, w.N)
    del y, ud, kf
    torch.cuda.empty_cache()
    return u, k, yh


@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
def test_full_size(name):
    w = inputs.WORKLOADS[name]
    _say("full-size", name, "B=%d H=%d N=%d %s" % (w.B, w.H, w.N, w.dtype))
    u, k, yh = _run_full(w)
    hidx_all = np.arange(w.rows) % w.H
    # whole tensor against the FFT route, chunked to bound host memory.
    # Beside the whole-tensor bar, every row and every output get a bound of
    # their own, so that corrupted rows or single wrong outputs cannot hide
    # in the whole-tensor average.  Both are scaled by the row's conditioning
    # s_r = ||u_r||_2 max_f |K_h(f)| (K_h the 2N-point spectrum of the
    # row's kernel): the transforms are unitary, so the rounding errors of
    # the stages are relative to ||u_r|| and reach the output multiplied by
    # at most max|K_h|, while ||y_r|| itself can be far smaller when the
    # kernel attenuates where the row's energy is (a tone of the audio rows
    # in a notch of K_h).  s_r >= ||y_r||, and for unattenuated rows the two
    # are within a small factor.
    #  * rows: ||y_r - ref_r||_2 <= TOL s_r
    #  * outputs: |y - ref| <= u_io |ref| + 10 TOL s_r / sqrt(N), with u_io
    #    the unit roundoff of the output type (bf16 2^-8, f16 2^-11,
    #    fp32 2^-24)
    # One output off by the row's RMS breaks both.
    u_io = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11, "f32": 2.0 ** -24}[w.dtype]
    kmax = np.max(np.abs(oracle.kernel_spectrum(k.astype(np.float64))), axis=1)
    num = den = 0.0
    worst_row = worst_plain_row = worst_elem = 0.0
    chunk = max(1, min(w.rows, (1 << 27) // w.N))
    for r0 in range(0, w.rows, chunk):
        r1 = min(w.rows, r0 + chunk)
        hs = hidx_all[r0:r1]
        uh, inv = np.unique(hs, return_inverse=True)
        u64 = oracle.to_f64(u[r0:r1], w.dtype)
        ref = oracle.conv_fft(u64, k[uh].astype(np.float64), inv)
        got = oracle.to_f64(yh[r0:r1], w.dtype)
        d2 = np.sum((got - ref) ** 2, axis=1)
        r2 = np.sum(ref ** 2, axis=1)
        num += float(d2.sum())
        den += float(r2.sum())
        scale = np.sqrt(np.sum(u64 ** 2, axis=1)) * kmax[hs]
        live = scale > 0
        worst_row = max(worst_row, float(np.max(np.sqrt(d2[live]) / scale[live]))
                        if live.any() else 0.0)
        nz = r2 > 0
        if nz.any():
            worst_plain_row = max(worst_plain_row, float(np.max(np.sqrt(d2[nz] / r2[nz]))))
        excess = (np.abs(got - ref) - u_io * np.abs(ref)) / np.maximum(
            scale / np.sqrt(w.N), 1e-300)[:, None]
        worst_elem = max(worst_elem, float(np.max(excess)))
    err = (num / den) ** 0.5
    _say("  whole-tensor rel_l2", err)
    _say("  worst row ||y - ref|| / (||u|| max|K|)", worst_row,
         "(plain per-row rel_l2 max %.3e)" % worst_plain_row)
    _say("  worst output (|y - ref| - u_io|ref|) / (||u|| max|K| / sqrt(N))", worst_elem)
    assert err < TOL[w.dtype]
    assert worst_row < TOL[w.dtype]
    assert worst_elem < 10 * TOL[w.dtype]
    # sampled outputs by the definition
    rng = np.random.default_rng(1234)
    ns = 96 if w.N >= (1 << 20) else 256
    rows = rng.integers(0, w.rows, ns)
    ts = rng.integers(0, w.N, ns)
    ts[:4] = [0, w.N - 1, 1, w.N // 2]
    if name.startswith("genome"):
        ts[4:8] = [inputs.GENOME_LEN - 1, inputs.GENOME_LEN,
                   inputs.GENOME_LEN + 1000, w.N - 2]
    sel = np.unique(rows)
    pos = np.searchsorted(sel, rows)
    want = oracle.conv_points(oracle.to_f64(u[sel], w.dtype),
                              k.astype(np.float64), pos, ts,
                              hidx_all[sel])
    got = oracle.to_f64(yh[rows, ts], w.dtype)
    serr = oracle.rel_l2(got, want)
    _say("  sampled rel_l2 (%d points)" % ns, serr)
    # single points carry the output rounding of their own value only;
    # allow the sample estimate a little statistical slack
    assert serr < 1.5 * TOL[w.dtype]
