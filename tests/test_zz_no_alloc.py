"""The allocation-free forward call (fftconv_forward_noalloc, through the C
ABI) against fftconv_forward on the same inputs: two calls in a row on each
plan, the second with a smaller batch, so the static scratch array's
leftover contents from the first call must not leak into the second."""
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


def _inputs(N, dtype, B, H, wid):
    import torch
    w = inputs.Workload("noalloc", wid, B, H, N, dtype, "normal", "decay", "")
    u = to_torch(inputs.input_rows(w), dtype).view(B, H, N)
    k = torch.from_numpy(inputs.kernel_rows(w)).cuda()
    return u, k


@pytest.mark.parametrize("N,dtype,calls", [
    # row kernel (no scratch), wide kernel (row-claim counters), one- and
    # two-level multi-pass (f16 chunks: 64K x 4 x 96 rows is 96 MiB, more
    # than the array, so it runs in chunks; 4M rows are 16 MiB each), the
    # LDS-staged fused kernel and the fp32 three-pass path
    (1024, "bf16", [(4, 96), (1, 5)]),
    (8192, "f16", [(3, 40), (2, 3)]),
    (32768, "bf16", [(4, 24), (1, 3)]),
    (65536, "bf16", [(4, 96), (1, 3)]),
    (4194304, "bf16", [(1, 6), (1, 1)]),
    (2048, "f16", [(2, 9), (1, 2)]),
    (32768, "f32", [(2, 5), (1, 3)]),
])
def test_noalloc_matches_forward(N, dtype, calls):
    import torch
    from fft_long_convolution_amd import fftconv as fc
    conv = fc.FFTConv(N, dtype=dtype)
    L = fc.lib()
    H_max = max(h for _, h in calls)
    for i, (B, H) in enumerate(calls):
        u, k = _inputs(N, dtype, B, H, 300 + N.bit_length() + i)
        kf = conv.kernel_spectrum(k)
        ref = conv.forward(u, kf)
        y = torch.full_like(u, float("nan"))
        st = L.fftconv_forward_noalloc(conv._plan, u.data_ptr(), kf.data_ptr(),
                                       y.data_ptr(), B, H, N, None)
        assert st == 0
        torch.cuda.synchronize()
        a = oracle.to_f64(from_torch(y, dtype).reshape(B * H, N), dtype)
        b = oracle.to_f64(from_torch(ref, dtype).reshape(B * H, N), dtype)
        err = oracle.rel_l2(a, b)
        same = bool(np.array_equal(a, b))
        _say("noalloc", N, dtype, "call", i, "B=%d H=%d" % (B, H),
             "rel_l2 vs forward", err, "bitwise equal", same)
        assert np.all(np.isfinite(a))
        assert err <= TOL[dtype]
    del H_max


def test_noalloc_errors():
    import torch
    from fft_long_convolution_amd import fftconv as fc
    L = fc.lib()
    # an fp32 multi-pass call needs B*H*N*8 bytes in one piece: 64 rows of
    # 256K points need 128 MiB, more than the static array
    conv = fc.FFTConv(262144, dtype="f32")
    u = torch.zeros(64, 1, 262144, device="cuda")
    kf = conv.kernel_spectrum(torch.zeros(1, 262144, device="cuda"))
    y = torch.empty_like(u)
    assert L.fftconv_forward_noalloc(conv._plan, u.data_ptr(), kf.data_ptr(),
                                     y.data_ptr(), 64, 1, 262144, None) == 4
    # argument checks as fftconv_forward: wrong N, output overlapping input
    assert L.fftconv_forward_noalloc(conv._plan, u.data_ptr(), kf.data_ptr(),
                                     y.data_ptr(), 1, 1, 1024, None) == 1
    assert L.fftconv_forward_noalloc(conv._plan, u.data_ptr(), kf.data_ptr(),
                                     u.data_ptr(), 1, 1, 262144, None) == 1
    assert L.fftconv_forward_noalloc(None, u.data_ptr(), kf.data_ptr(),
                                     y.data_ptr(), 1, 1, 262144, None) == 1
    torch.cuda.synchronize()
