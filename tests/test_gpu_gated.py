"""GPU parity of the gated convolution y = v * ((u * w) conv k) (the gating
of H3/Hyena-style layers fused into the convolution kernels) through the
C ABI entry point fftconv_forward_gated, against the fp64 oracle.

Every kernel family is covered: the LDS-staged kernel (fp32 and forced for
16-bit rows), the register-resident row kernel, the one-workgroup-per-row
kernel, the one-level and two-level multi-pass passes, and the fp32
three-pass path; at the full workload sizes the whole output is compared
(sampled points by the definition for the 4M workload).
"""
import sys

import numpy as np
import pytest

import oracle
from fft_long_convolution_amd import inputs
from tests.gpu_helpers import TOL, from_torch, parity_gated, to_torch

pytestmark = pytest.mark.gpu

W = inputs.WORKLOADS


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def test_tiny_fp32_gated():
    err, _, _ = parity_gated(W["tiny_f32_n256"])
    _say("tiny gated rel_l2", err)
    assert err < TOL["f32"]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("N", [256, 512, 1024, 2048, 4096, 8192, 16384,
                               32768, 65536, 131072])
def test_gated_length_sweep(N, dtype):
    # 3 x 5 rows: ragged against every kernel's tiling
    w = inputs.Workload("gsweep", 140 + N.bit_length(), 3, 5, N, dtype,
                        "normal", "decay", "gated sweep")
    err, _, _ = parity_gated(w)
    _say("gated sweep", N, dtype, "rel_l2", err)
    assert err < TOL[dtype]


@pytest.mark.parametrize("N,dtype", [(1024, "bf16"), (4096, "f16"),
                                     (16384, "bf16")])
def test_gated_generic_kernel(N, dtype, monkeypatch):
    # the LDS-staged kernel at lengths the register-resident kernels own
    monkeypatch.setenv("FFTCONV_KERNEL", "generic")
    w = inputs.Workload("ggeneric", 160 + N.bit_length(), 2, 7, N, dtype,
                        "normal", "decay", "gated generic kernel")
    err, _, _ = parity_gated(w)
    _say("gated generic", N, dtype, "rel_l2", err)
    assert err < TOL[dtype]


@pytest.mark.parametrize("N,dtype,B,H", [
    (512, "f16", 33, 4), (1024, "bf16", 64, 3), (8192, "bf16", 5, 9), (32768, "bf16", 7, 5),
    (262144, "f16", 1, 3), (524288, "bf16", 1, 2), (1048576, "f16", 1, 2),
    (2097152, "bf16", 1, 1), (4194304, "bf16", 1, 1),
    (4194304, "f16", 1, 1)])
def test_gated_shapes_and_multipass(N, dtype, B, H):
    # ragged row-kernel and wide-kernel slices, and every two-level factor
    # pair (8x8 ... 32x16 on the vector ALU, 32x32 on the matrix cores)
    w = inputs.Workload("gshape", 180 + N.bit_length() + B, B, H, N, dtype,
                        "normal", "decay", "gated shapes")
    err, _, _ = parity_gated(w)
    _say("gated shapes", N, dtype, B, H, "rel_l2", err)
    assert err < TOL[dtype]


def test_gated_unit_gates_match_plain():
    # w = v = 1 reduces the gated call to the plain convolution; the two
    # entry points then agree to the tolerance (the gated row kernel feeds
    # the first stage f16 operands where the plain one uses a bf16 pair)
    import torch
    from fft_long_convolution_amd.fftconv import FFTConv
    for N, dtype in [(1024, "bf16"), (8192, "f16"), (65536, "bf16")]:
        w = inputs.Workload("gunit", 200 + N.bit_length(), 2, 3, N, dtype,
                            "normal", "decay", "unit gates")
        conv = FFTConv(N, dtype=dtype)
        u = to_torch(inputs.input_rows(w), dtype).view(2, 3, N)
        kf = conv.kernel_spectrum(torch.from_numpy(inputs.kernel_rows(w)).cuda())
        one = torch.ones_like(u)
        yg = conv.forward_gated(u, one, one, kf)
        yp = conv.forward(u, kf)
        torch.cuda.synchronize()
        a = oracle.to_f64(from_torch(yg, dtype).reshape(6, N), dtype)
        b = oracle.to_f64(from_torch(yp, dtype).reshape(6, N), dtype)
        err = oracle.rel_l2(a, b)
        _say("unit gates", N, dtype, "rel_l2 vs plain", err)
        assert err < TOL[dtype]


def test_gated_error_paths():
    import torch
    from fft_long_convolution_amd import fftconv as fc
    conv = fc.FFTConv(1024, dtype="bf16")
    L = fc.lib()
    k = torch.randn(3, 1024, device="cuda")
    kf = conv.kernel_spectrum(k)
    u = torch.randn(2, 3, 1024, device="cuda").to(torch.bfloat16)
    g = torch.randn(2, 3, 1024, device="cuda").to(torch.bfloat16)
    y = torch.empty_like(u)
    args = lambda uu, ww, vv, yy: (conv._plan, uu, ww, vv, kf.data_ptr(), yy,
                                   2, 3, 1024, None, 0, None)
    # a missing gate
    assert L.fftconv_forward_gated(*args(u.data_ptr(), None, g.data_ptr(),
                                         y.data_ptr())) == 1
    # output overlapping a gate
    assert L.fftconv_forward_gated(*args(u.data_ptr(), g.data_ptr(),
                                         g.data_ptr(), g.data_ptr())) == 1
    # misaligned gate
    assert L.fftconv_forward_gated(*args(u.data_ptr(), g.data_ptr() + 2,
                                         g.data_ptr(), y.data_ptr())) == 3
    # gates may alias u and each other
    assert L.fftconv_forward_gated(*args(u.data_ptr(), u.data_ptr(),
                                         u.data_ptr(), y.data_ptr())) == 0
    # an empty batch is a no-op, gates or not
    assert L.fftconv_forward_gated(conv._plan, None, None, None,
                                   kf.data_ptr(), None, 0, 3, 1024, None, 0,
                                   None) == 0
    torch.cuda.synchronize()


def _full_gated(w):
    import torch
    from fft_long_convolution_amd.fftconv import FFTConv
    conv = FFTConv(w.N, dtype=w.dtype)
    ins = [inputs.input_rows(w), inputs.gate_rows(w, "w"),
           inputs.gate_rows(w, "v")]
    k = inputs.kernel_rows(w)
    dev = [to_torch(a, w.dtype).view(w.B, w.H, w.N) for a in ins]
    kf = conv.kernel_spectrum(torch.from_numpy(k).cuda())
    y = conv.forward_gated(dev[0], dev[1], dev[2], kf)
    torch.cuda.synchronize()
    yh = from_torch(y, w.dtype).reshape(w.rows, w.N)
    del y, dev, kf
    torch.cuda.empty_cache()
    return ins, k, yh


@pytest.mark.parametrize("name", ["hyena_bf16_n1k", "m2bert_f16_n8k",
                                  "audio_bf16_n64k", "genome_bf16_n4m"])
def test_gated_full_size(name):
    w = W[name]
    _say("gated full-size", name, "B=%d H=%d N=%d %s" % (w.B, w.H, w.N, w.dtype))
    ins, k, yh = _full_gated(w)
    hidx_all = np.arange(w.rows) % w.H
    if w.N < (1 << 20):
        # whole tensor against the oracle's FFT route, in row chunks
        num = den = 0.0
        chunk = max(1, min(w.rows, (1 << 26) // w.N))
        for r0 in range(0, w.rows, chunk):
            r1 = min(w.rows, r0 + chunk)
            uh, inv = np.unique(hidx_all[r0:r1], return_inverse=True)
            u64, w64, v64 = (oracle.to_f64(a[r0:r1], w.dtype) for a in ins)
            ref = oracle.gated_fft(u64, w64, v64, k[uh].astype(np.float64), inv)
            got = oracle.to_f64(yh[r0:r1], w.dtype)
            num += float(np.sum((got - ref) ** 2))
            den += float(np.sum(ref ** 2))
        err = (num / den) ** 0.5
        _say("  whole-tensor rel_l2", err)
        assert err < TOL[w.dtype]
    # sampled outputs by the definition
    rng = np.random.default_rng(4321)
    ns = 96 if w.N >= (1 << 20) else 256
    rows = rng.integers(0, w.rows, ns)
    ts = rng.integers(0, w.N, ns)
    ts[:4] = [0, w.N - 1, 1, w.N // 2]
    sel = np.unique(rows)
    pos = np.searchsorted(sel, rows)
    u64, w64, v64 = (oracle.to_f64(a[sel], w.dtype) for a in ins)
    want = oracle.gated_points(u64, w64, v64, k.astype(np.float64), pos, ts,
                               hidx_all[sel])
    got = oracle.to_f64(yh[rows, ts], w.dtype)
    serr = oracle.rel_l2(got, want)
    _say("  sampled rel_l2 (%d points)" % ns, serr)
    assert serr < 1.5 * TOL[w.dtype]
