"""GPU parity of the frequency-sparse (band-limited) convolution:
fftconv_kernel_spectrum_lowpass + fftconv_forward_lowpass against the fp64
oracle's band-limited FFT route.  A cutoff below N/4 runs the variants of
the 32 x 32 engine (row kernel at N = 1024, wide kernel at 4K..16K,
multi-pass inner pass at >= 32K) that skip the matrix-core tiles of the
zeroed bins; other cutoffs and lengths compute the zero bins."""
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


def _round_io(x, dtype):
    if dtype == "bf16":
        return oracle.to_f64(inputs.f32_to_bf16_bits(x.astype(np.float32)), "bf16")
    if dtype == "f16":
        return x.astype(np.float16).astype(np.float64)
    return x.astype(np.float32).astype(np.float64)


def _run(w, cutoff, with_rounding=False):
    import torch
    from fft_long_convolution_amd.fftconv import FFTConv
    conv = FFTConv(w.N, dtype=w.dtype)
    u = inputs.input_rows(w)
    k = inputs.kernel_rows(w)
    kf = conv.kernel_spectrum_lowpass(torch.from_numpy(k).cuda(), cutoff)
    y = conv.forward_lowpass(to_torch(u, w.dtype).view(w.B, w.H, w.N), kf, cutoff)
    torch.cuda.synchronize()
    got = oracle.to_f64(from_torch(y, w.dtype).reshape(w.rows, w.N), w.dtype)
    ref = oracle.lowpass_fft(oracle.to_f64(u, w.dtype).reshape(w.rows, w.N),
                             k.astype(np.float64), cutoff, np.arange(w.rows) % w.H)
    if with_rounding:
        return oracle.rel_l2(got, ref), oracle.rel_l2(_round_io(ref, w.dtype), ref)
    return oracle.rel_l2(got, ref)


@pytest.mark.parametrize("N,dtype,B,H,cutoff", [
    (256, "f32", 1, 4, 40), (512, "f16", 3, 5, 100),
    (1024, "bf16", 3, 5, 255), (1024, "f16", 64, 3, 128),
    (1024, "bf16", 2, 7, 31), (1024, "bf16", 3, 5, 256),
    (1024, "f16", 3, 5, 700), (8192, "bf16", 2, 3, 1000),
    (4096, "f16", 3, 2, 500), (16384, "bf16", 2, 3, 4095),
    (8192, "f16", 2, 2, 2048), (32768, "bf16", 2, 3, 8191), (32768, "f16", 3, 2, 5000),
    (65536, "f16", 1, 3, 20000),
    (65536, "bf16", 2, 2, 16383), (262144, "f16", 1, 2, 3000),
    (1048576, "bf16", 1, 1, 200000), (4194304, "bf16", 1, 1, 500000),
    # the extremes: the DC bin alone, and no limit (cutoff = N)
    (1024, "bf16", 64, 64, 0), (8192, "f16", 4, 64, 0), (65536, "bf16", 1, 64, 0),
    (1024, "f16", 2, 3, 1024), (16384, "bf16", 1, 2, 16384), (131072, "f16", 1, 1, 131072)])
def test_lowpass(N, dtype, B, H, cutoff):
    w = inputs.Workload("lowpass", 260 + N.bit_length() + B, B, H, N, dtype,
                        "normal", "decay", "band-limited")
    err, rounding_only = _run(w, cutoff, with_rounding=True)
    _say("lowpass", N, dtype, B, H, cutoff, "rel_l2", err,
         "(oracle rounded to the I/O type: %.3e)" % rounding_only)
    if cutoff == 0:
        # With the DC bin alone every output of a row is the one value
        # sum(u) sum(k) / 2N, so the whole-tensor rel L2 averages over rows,
        # each weighted by (sum k)^2 of its channel, not over elements.  With
        # few channels one channel carries most of the weight and even the
        # exact result rounded to bf16 scatters around the bar (16 x 8 rows
        # at N = 1024: 2.04e-3).  The cases therefore span 64 channels; this
        # checks that the sample is wide enough for the bar to be meaningful.
        assert rounding_only < 0.9 * TOL[dtype]
    assert err < TOL[dtype]


def test_lowpass_full_size_hyena():
    # 75% sparsity (cutoff 255 of N = 1024: 511 of 2048 frequencies kept)
    err = _run(inputs.WORKLOADS["hyena_bf16_n1k"], 255)
    _say("lowpass full-size hyena rel_l2", err)
    assert err < TOL["bf16"]


def test_lowpass_errors():
    import torch
    from fft_long_convolution_amd import fftconv as fc
    conv = fc.FFTConv(1024, dtype="bf16")
    L = fc.lib()
    k = torch.randn(2, 1024, device="cuda")
    kf = torch.empty(conv.spectrum_bytes(2), dtype=torch.uint8, device="cuda")
    assert L.fftconv_kernel_spectrum_lowpass(conv._plan, k.data_ptr(), 2, 1025,
                                             kf.data_ptr(), None) == 1
    u = torch.randn(1, 2, 1024, device="cuda").to(torch.bfloat16)
    y = torch.empty_like(u)
    assert L.fftconv_forward_lowpass(conv._plan, u.data_ptr(), kf.data_ptr(), 1025,
                                     y.data_ptr(), 1, 2, 1024, None, 0, None) == 1
    torch.cuda.synchronize()
