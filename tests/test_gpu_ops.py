"""GPU parity of the operator family selected by the kernel spectrum
(fftconv_kernel_spectrum_kind): the causal adjoint (the input gradient of
the causal convolution), the non-causal circular convolution and its
adjoint, each through the unchanged forward kernels of every family,
against the fp64 oracle's independent definitions."""
import sys

import numpy as np
import pytest

import oracle
from fft_long_convolution_amd import inputs
from tests.gpu_helpers import TOL, from_torch, parity_op, to_torch

pytestmark = pytest.mark.gpu

KINDS = ["causal_adjoint", "circular", "circular_adjoint"]


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("N,dtype,B,H", [
    (256, "f32", 1, 4), (256, "bf16", 3, 5), (1024, "bf16", 3, 5),
    (512, "f16", 2, 3), (2048, "f32", 2, 3), (8192, "f16", 3, 5),
    (16384, "bf16", 2, 3), (32768, "f16", 2, 3), (65536, "bf16", 1, 3), (131072, "f32", 1, 2),
    (1048576, "f16", 1, 2), (4194304, "bf16", 1, 1)])
def test_operator_kinds(kind, N, dtype, B, H):
    # every kernel family: LDS-staged (256, 2048 fp32), row (512, 1024),
    # wide (8K, 16K), one-level multi-pass (64K), fp32 three-pass (128K),
    # two-level VALU (1M) and matrix-core (4M) column passes
    w = inputs.Workload("ops", 220 + N.bit_length() + B, B, H, N, dtype,
                        "normal", "decay", "operator kinds")
    err, _, _ = parity_op(w, kind)
    _say(kind, N, dtype, B, H, "rel_l2", err)
    assert err < TOL[dtype]


def test_circular_shift_exact():
    # a delta kernel at tap m makes the circular convolution a rotation by
    # m (torch.roll), independently of the oracle
    import torch
    from fft_long_convolution_amd.fftconv import FFTConv
    N, m = 1024, 37
    conv = FFTConv(N, dtype="f32")
    u = torch.randn(2, 3, N, device="cuda")
    k = torch.zeros(3, N, device="cuda")
    k[:, m] = 1.0
    kf = conv.kernel_spectrum(k, kind="circular")
    y = conv.forward(u, kf)
    torch.cuda.synchronize()
    want = torch.roll(u, m, dims=2)
    err = float((y - want).norm() / want.norm())
    _say("circular shift rel_l2", err)
    assert err < TOL["f32"]


@pytest.mark.parametrize("name", ["hyena_bf16_n1k", "m2bert_f16_n8k"])
def test_circular_full_size(name):
    # the non-causal convolution at a full workload shape, whole tensor
    import torch
    from fft_long_convolution_amd.fftconv import FFTConv
    w = inputs.WORKLOADS[name]
    _say("circular full-size", name)
    conv = FFTConv(w.N, dtype=w.dtype)
    u = inputs.input_rows(w)
    k = inputs.kernel_rows(w)
    kf = conv.kernel_spectrum(torch.from_numpy(k).cuda(), kind="circular")
    y = conv.forward(to_torch(u, w.dtype).view(w.B, w.H, w.N), kf)
    torch.cuda.synchronize()
    yh = from_torch(y, w.dtype).reshape(w.rows, w.N)
    hidx_all = np.arange(w.rows) % w.H
    num = den = 0.0
    chunk = max(1, min(w.rows, (1 << 26) // w.N))
    for r0 in range(0, w.rows, chunk):
        r1 = min(w.rows, r0 + chunk)
        uh, inv = np.unique(hidx_all[r0:r1], return_inverse=True)
        ref = oracle.op_fft(oracle.to_f64(u[r0:r1], w.dtype),
                            k[uh].astype(np.float64), "circular", inv)
        got = oracle.to_f64(yh[r0:r1], w.dtype)
        num += float(np.sum((got - ref) ** 2))
        den += float(np.sum(ref ** 2))
    err = (num / den) ** 0.5
    _say("  whole-tensor rel_l2", err)
    assert err < TOL[w.dtype]
