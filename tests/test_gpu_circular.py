"""GPU parity of the plans at FFT size N (fftconv_plan_circular): the
circular convolution and its adjoint through an N-point real transform
(M = N/2 packed points, none of them padding), every length from 512 to 4M
on every kernel family the plans reach, plain and gated, against the fp64
oracle's own definitions (the O(N^2) sums for small N, its size-N FFT route
otherwise), plus an exact rotation check that does not use the oracle."""
import sys

import numpy as np
import pytest

import oracle
from fft_long_convolution_amd import inputs
from tests.gpu_helpers import (TOL, from_torch, oracle_circular, run_gpu_circular,
                               to_torch)

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _case(tag, seed, B, H, N, dtype):
    return inputs.Workload(tag, seed, B, H, N, dtype, "normal", "decay", "circular plan")


def _kmax_n(k):
    """max_f |K_h(f)| of each kernel's N-point spectrum (the even bins of
    the oracle's 2N-point spectrum of the zero-padded kernel)."""
    return np.max(np.abs(oracle.kernel_spectrum(k.astype(np.float64))[:, ::2]), axis=1)


def _worst_row(got, ref, u64, kmax_rows):
    """max_r ||y_r - ref_r|| / (||u_r|| max|K_h|): the transforms are
    unitary, so each row's rounding error is relative to ||u_r|| and reaches
    the output scaled by at most max|K_h| (a few wrong outputs in one row
    exceed the bar here even when the whole-tensor norm hides them)."""
    scale = np.linalg.norm(u64, axis=1) * kmax_rows
    return float(np.max(np.linalg.norm(got - ref, axis=1) / scale))


@pytest.mark.parametrize("N", [1 << lg for lg in range(9, 23)])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_circular_plan_sweep(N, dtype):
    # every length on every I/O type: LDS-staged fused (M <= 16K, fp32; M =
    # 256 and 2048 for 16-bit), row (M = 512, 1024), wide (M = 4K..16K),
    # 16-bit multi-pass (M >= 32K: one and two outer levels), fp32 three-pass
    B, H = (2, 3) if N <= (1 << 17) else (1, 1)
    w = _case("circ", 400 + N.bit_length(), B, H, N, dtype)
    y, ins, k = run_gpu_circular(w)
    err = oracle.rel_l2(y, oracle_circular(w, ins, k))
    _say("circular plan", N, dtype, B, H, "rel_l2", err)
    assert err < TOL[dtype]


@pytest.mark.parametrize("N,dtype,B,H", [
    (512, "bf16", 3, 5), (1024, "f16", 5, 3), (2048, "bf16", 3, 5), (4096, "f16", 2, 3),
    (8192, "bf16", 3, 2), (16384, "f16", 2, 3), (32768, "bf16", 2, 2), (65536, "f16", 1, 3),
    (131072, "bf16", 2, 1), (524288, "f16", 1, 2), (1 << 22, "bf16", 1, 1),
    (1024, "f32", 2, 3), (65536, "f32", 1, 2)])
def test_circular_plan_adjoint(N, dtype, B, H):
    w = _case("circa", 430 + N.bit_length() + B, B, H, N, dtype)
    y, ins, k = run_gpu_circular(w, kind="circular_adjoint")
    err = oracle.rel_l2(y, oracle_circular(w, ins, k, "circular_adjoint"))
    _say("circular plan adjoint", N, dtype, B, H, "rel_l2", err)
    assert err < TOL[dtype]


@pytest.mark.parametrize("N,dtype,B,H", [
    (512, "f16", 2, 3), (1024, "bf16", 3, 5), (2048, "f16", 2, 3), (8192, "bf16", 2, 3),
    (16384, "f16", 3, 2), (32768, "f16", 1, 3), (65536, "bf16", 2, 2), (262144, "f16", 1, 2),
    (1 << 21, "bf16", 1, 1), (2048, "f32", 2, 2), (131072, "f32", 1, 2)])
def test_circular_plan_gated(N, dtype, B, H):
    w = _case("circg", 450 + N.bit_length() + B, B, H, N, dtype)
    y, ins, k = run_gpu_circular(w, gated=True)
    err = oracle.rel_l2(y, oracle_circular(w, ins, k))
    _say("circular plan gated", N, dtype, B, H, "rel_l2", err)
    assert err < TOL[dtype]


@pytest.mark.parametrize("N,dtype,B,H", [
    (1024, "bf16", 17, 37), (1024, "f16", 1, 1), (2048, "bf16", 64, 33),
    (2048, "f16", 7, 1), (8192, "f16", 9, 13), (16384, "bf16", 5, 11), (32768, "bf16", 3, 7)])
def test_circular_plan_shapes(N, dtype, B, H):
    # ragged batch x channel counts on the register-resident kernels (more
    # channels than a workgroup's slice, single rows, odd counts)
    w = _case("circs", 470 + N.bit_length() + B + H, B, H, N, dtype)
    y, ins, k = run_gpu_circular(w)
    ref = oracle_circular(w, ins, k)
    err = oracle.rel_l2(y, ref)
    _say("circular plan shape", N, dtype, B, H, "rel_l2", err)
    assert err < TOL[dtype]
    # every row within the bar, relative to its conditioning
    u64 = oracle.to_f64(ins[0], dtype).reshape(w.rows, N)
    worst = _worst_row(y, ref, u64, _kmax_n(k)[np.arange(w.rows) % H])
    _say("  worst row (conditioned)", worst)
    assert worst < TOL[dtype]


@pytest.mark.parametrize("N,dtype", [(512, "f32"), (1024, "bf16"), (2048, "f16"), (4096, "f16"),
                                     (16384, "bf16"), (65536, "f16"), (1 << 21, "bf16")])
def test_circular_plan_rotation(N, dtype):
    # a delta kernel at tap m makes the circular convolution the rotation
    # y[t] = u[(t - m) mod N] (and its adjoint the rotation by -m): checked
    # against torch.roll of the same input, no oracle involved
    import torch
    from fft_long_convolution_amd.fftconv import FFTConv
    conv = FFTConv(N, dtype=dtype, circular=True)
    m = 37 + N // 3
    B, H = 2, 3
    g = torch.Generator().manual_seed(N + 5)
    u32 = torch.randn(B, H, N, generator=g)
    u = u32.to({"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]).cuda()
    k = torch.zeros(H, N)
    k[:, m] = 1.0
    for kind, shift in (("circular", m), ("circular_adjoint", -m)):
        kf = conv.kernel_spectrum(k.cuda(), kind=kind)
        y = conv.forward(u, kf)
        torch.cuda.synchronize()
        want = torch.roll(u.float(), shift, dims=2)
        err = float((y.float() - want).norm() / want.norm())
        _say("circular plan rotation", N, dtype, kind, "rel_l2", err)
        assert err < TOL[dtype]


@pytest.mark.parametrize("name", ["hyena_bf16_n1k", "m2bert_f16_n8k"])
def test_circular_plan_full_size(name):
    # the workload shapes through plans at FFT size N, whole tensor, and
    # the per-row bound
    import torch
    from fft_long_convolution_amd.fftconv import FFTConv
    w = inputs.WORKLOADS[name]
    _say("circular plan full-size", name)
    conv = FFTConv(w.N, dtype=w.dtype, circular=True)
    u = inputs.input_rows(w)
    k = inputs.kernel_rows(w)
    kf = conv.kernel_spectrum(torch.from_numpy(k).cuda(), kind="circular")
    y = conv.forward(to_torch(u, w.dtype).view(w.B, w.H, w.N), kf)
    torch.cuda.synchronize()
    yh = from_torch(y, w.dtype).reshape(w.rows, w.N)
    del y
    hidx_all = np.arange(w.rows) % w.H
    kmax = _kmax_n(k)
    num = den = 0.0
    worst = 0.0
    chunk = max(1, min(w.rows, (1 << 26) // w.N))
    for r0 in range(0, w.rows, chunk):
        r1 = min(w.rows, r0 + chunk)
        uh, inv = np.unique(hidx_all[r0:r1], return_inverse=True)
        u64 = oracle.to_f64(u[r0:r1], w.dtype)
        ref = oracle.op_fft(u64, k[uh].astype(np.float64), "circular", inv)
        got = oracle.to_f64(yh[r0:r1], w.dtype)
        num += float(((got - ref) ** 2).sum())
        den += float((ref ** 2).sum())
        worst = max(worst, _worst_row(got, ref, u64, kmax[hidx_all[r0:r1]]))
    err = (num / den) ** 0.5
    _say("  rel_l2", err, "worst row (conditioned)", worst)
    assert err < TOL[w.dtype]
    assert worst < TOL[w.dtype]


def test_circular_plan_noalloc_and_errors():
    import torch
    from fft_long_convolution_amd import fftconv as fc
    N, B, H = 65536, 2, 3
    conv = fc.FFTConv(N, dtype="bf16", circular=True)
    w = _case("circn", 490, B, H, N, "bf16")
    u = to_torch(inputs.input_rows(w), "bf16").view(B, H, N)
    kf = conv.kernel_spectrum(torch.from_numpy(inputs.kernel_rows(w)).cuda())
    y1 = conv.forward(u, kf)
    y2 = conv.forward_noalloc(u, kf, torch.empty_like(u))
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    L = fc.lib()
    k = torch.zeros(H, N, device="cuda")
    buf = torch.empty(conv.spectrum_bytes(H), dtype=torch.uint8, device="cuda")
    # the causal kinds, band limits, digit blocks and the backward call are
    # refused on a plan at FFT size N
    for kind in (0, 1):
        assert L.fftconv_kernel_spectrum_kind(conv._plan, k.data_ptr(), H, kind,
                                              buf.data_ptr(), None) == 2
    assert L.fftconv_kernel_spectrum(conv._plan, k.data_ptr(), H, buf.data_ptr(), None) == 2
    assert L.fftconv_kernel_spectrum_lowpass(conv._plan, k.data_ptr(), H, 10,
                                             buf.data_ptr(), None) == 2
    assert L.fftconv_kernel_spectrum_blocksparse(conv._plan, k.data_ptr(), H, 0, 0,
                                                 buf.data_ptr(), None) == 2
    dk = torch.empty(H, N, device="cuda")
    assert L.fftconv_backward(conv._plan, u.data_ptr(), u.data_ptr(), None, None,
                              dk.data_ptr(), B, H, N, None, 0, None) == 2
    assert conv.info["circular"] and conv.info["M"] == N // 2
    torch.cuda.synchronize()
