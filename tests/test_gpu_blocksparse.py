"""GPU parity of the frequency-sparse convolution with zero blocks along the
transform's digits (fftconv_kernel_spectrum_blocksparse +
fftconv_forward_blocksparse) against the fp64 oracle's masked-spectrum
route.  Covers every kernel family and both kinds of skipped work: the
matrix-core tiles of the top digit's middle values (a >= 16) and the engine
passes of whole outer classes (d > 1: pairs of sub-rows in the wide kernel,
units of two slabs in the multi-pass inner pass)."""
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


def _run(w, a, d):
    import torch
    from fft_long_convolution_amd.fftconv import FFTConv
    conv = FFTConv(w.N, dtype=w.dtype)
    P = conv.info["sparse_outer"]
    u = inputs.input_rows(w)
    k = inputs.kernel_rows(w)
    kf = conv.kernel_spectrum_blocksparse(torch.from_numpy(k).cuda(), a, d)
    y = conv.forward_blocksparse(to_torch(u, w.dtype).view(w.B, w.H, w.N), kf, a, d)
    torch.cuda.synchronize()
    got = oracle.to_f64(from_torch(y, w.dtype).reshape(w.rows, w.N), w.dtype)
    ref = oracle.blocksparse_fft(oracle.to_f64(u, w.dtype).reshape(w.rows, w.N),
                                 k.astype(np.float64), P, a, d, np.arange(w.rows) % w.H)
    S = 1.0 - oracle.blocksparse_mask(w.N, P, a, d).mean()
    return oracle.rel_l2(got, ref), P, S


@pytest.mark.parametrize("N,dtype,B,H,a,d", [
    # row kernel (no outer digit): the top digit's middle 16 skipped
    (1024, "bf16", 3, 5, 16, 0), (1024, "f16", 8, 4, 24, 0), (1024, "bf16", 2, 3, 8, 0),
    # LDS-staged kernels (fp32, N = 2048)
    (2048, "f32", 2, 3, 16, 0), (256, "f32", 1, 4, 12, 0),
    # wide kernel P = 8, 16, 32: pairs of sub-rows skipped
    (8192, "f16", 3, 5, 0, 2), (8192, "bf16", 2, 3, 16, 4), (8192, "f16", 2, 2, 8, 7),
    (16384, "bf16", 2, 3, 0, 9), (32768, "bf16", 2, 3, 0, 16), (32768, "f16", 3, 2, 16, 31),
    # multi-pass: units skipped (one and two outer levels, matrix-core 4M)
    (65536, "bf16", 2, 3, 0, 6), (65536, "f16", 1, 2, 16, 15), (131072, "bf16", 1, 2, 8, 20),
    (1048576, "f16", 1, 2, 0, 100), (4194304, "bf16", 1, 1, 16, 600),
    # no zero blocks at all
    (8192, "bf16", 2, 2, 0, 0), (65536, "f16", 1, 2, 0, 0)])
def test_blocksparse(N, dtype, B, H, a, d):
    w = inputs.Workload("blocksparse", 290 + N.bit_length() + B + a + d, B, H, N, dtype,
                        "normal", "decay", "digit-block sparsity")
    err, P, S = _run(w, a, d)
    _say("blocksparse", N, dtype, B, H, "P=%d a=%d d=%d sparsity %.3f" % (P, a, d, S),
         "rel_l2", err)
    assert err < TOL[dtype]


def test_blocksparse_errors():
    import torch
    from fft_long_convolution_amd import fftconv as fc
    L = fc.lib()
    conv = fc.FFTConv(8192, dtype="f16")
    assert conv.info["sparse_outer"] == 8
    k = torch.randn(2, 8192, device="cuda")
    kf = torch.empty(conv.spectrum_bytes(2), dtype=torch.uint8, device="cuda")
    u = torch.randn(1, 2, 8192, device="cuda").half()
    y = torch.empty_like(u)
    ws = torch.empty(conv.workspace_bytes(1, 2), dtype=torch.uint8, device="cuda")
    for a, d in ((3, 0), (34, 0), (-2, 0), (0, 8), (0, -1)):
        assert L.fftconv_kernel_spectrum_blocksparse(conv._plan, k.data_ptr(), 2, a, d,
                                                     kf.data_ptr(), None) == 1
        assert L.fftconv_forward_blocksparse(conv._plan, u.data_ptr(), kf.data_ptr(), a, d,
                                             y.data_ptr(), 1, 2, 8192, ws.data_ptr(),
                                             ws.numel(), None) == 1
    row = fc.FFTConv(1024, dtype="bf16")
    assert row.info["sparse_outer"] == 1
    kf1 = torch.empty(row.spectrum_bytes(2), dtype=torch.uint8, device="cuda")
    assert L.fftconv_kernel_spectrum_blocksparse(row._plan, k[:, :1024].contiguous().data_ptr(),
                                                 2, 0, 1, kf1.data_ptr(), None) == 1
    torch.cuda.synchronize()
