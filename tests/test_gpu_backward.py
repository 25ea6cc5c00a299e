"""GPU parity of the backward pass of the causal convolution through the C
ABI entry point fftconv_backward: the input gradient (the forward kernels
with the adjoint spectrum) and the kernel gradient (conj(U) DY accumulated
per channel: on the row, wide and multi-pass engines for 16-bit I/O, on
LDS-staged kernels otherwise), against the fp64 oracle's definitions and
convolution-theorem routes.  dk is fp32 for every I/O
type; its bar is the I/O type's (the inputs' quantisation is exact in the
oracle, the error is the transforms').
"""
import sys

import numpy as np
import pytest

import oracle
from fft_long_convolution_amd import inputs
from tests.gpu_helpers import TOL, from_torch, oracle_backward, run_gpu_backward, to_torch

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("N,dtype,B,H", [
    (256, "f32", 1, 4), (256, "bf16", 3, 5), (512, "f16", 4, 3),
    (1024, "bf16", 5, 3), (1024, "f16", 64, 4), (1024, "bf16", 1, 1),
    (1024, "bf16", 8, 256), (1024, "f16", 16, 256),
    (1024, "f32", 2, 2), (2048, "f16", 3, 2),
    (4096, "bf16", 2, 3), (4096, "f16", 1, 1), (8192, "f16", 3, 2),
    (8192, "bf16", 17, 5), (16384, "bf16", 2, 3), (16384, "f16", 4, 2),
    (32768, "f32", 1, 2), (32768, "bf16", 3, 2), (65536, "f16", 2, 1),
    (131072, "f16", 2, 3), (262144, "bf16", 1, 2), (524288, "bf16", 2, 1),
    (1048576, "f16", 1, 1), (2097152, "f16", 1, 2), (4194304, "bf16", 1, 1)])
def test_backward(N, dtype, B, H):
    # the row engine at N = 1024 (batch slices of one row up to more rows
    # than slices; eight slices of a channel -- B = 8 and 16 at H = 256, and
    # the full-size shape -- sum in one workgroup's LDS) and the wide engine
    # at N = 4K..16K with 16-bit I/O, the
    # multi-pass engine at N >= 32K with 16-bit I/O (forward column passes
    # of u and dy, the accumulating inner pass on one- and two-level outer
    # factors, the inverse column passes into fp32 dk), the LDS-staged
    # kernel-gradient kernels for fp32; the input gradient through every
    # forward family
    w = inputs.Workload("bwd", 240 + N.bit_length() + B, B, H, N, dtype,
                        "normal", "decay", "backward")
    du, dk, u, dy, k = run_gpu_backward(w)
    rdu, rdk = oracle_backward(w, u, dy, k)
    edu, edk = oracle.rel_l2(du, rdu), oracle.rel_l2(dk, rdk)
    _say("backward", N, dtype, B, H, "du rel_l2", edu, "dk rel_l2", edk)
    assert edu < TOL[dtype]
    assert edk < TOL[dtype]


def test_backward_pieces_and_errors():
    import torch
    from fft_long_convolution_amd import fftconv as fc
    w = inputs.Workload("bwdp", 250, 3, 2, 1024, "bf16", "normal", "decay", "")
    conv = fc.FFTConv(1024, dtype="bf16")
    u = to_torch(inputs.input_rows(w), "bf16").view(3, 2, 1024)
    dy = to_torch(inputs.dy_rows(w), "bf16").view(3, 2, 1024)
    kfa = conv.kernel_spectrum(torch.from_numpy(inputs.kernel_rows(w)).cuda(),
                               kind="causal_adjoint")
    du_all, dk_all = conv.backward(u, dy, kfa)
    du_only, none1 = conv.backward(None, dy, kfa, need_dk=False)
    none2, dk_only = conv.backward(u, dy, None, need_du=False)
    torch.cuda.synchronize()
    assert none1 is None and none2 is None
    assert torch.equal(du_all.view(torch.int16), du_only.view(torch.int16))
    assert torch.equal(dk_all, dk_only)
    # an empty batch: dk = 0
    e = torch.empty(0, 2, 1024, dtype=torch.bfloat16, device="cuda")
    _, dk0 = conv.backward(e, e, None, need_du=False)
    torch.cuda.synchronize()
    assert dk0.shape == (2, 1024) and not dk0.any()
    L = fc.lib()
    dk = torch.empty(2, 1024, device="cuda")
    # nothing requested, dk overlapping u, misaligned dk
    assert L.fftconv_backward(conv._plan, u.data_ptr(), dy.data_ptr(), None,
                              None, None, 3, 2, 1024, None, 0, None) == 1
    assert L.fftconv_backward(conv._plan, u.data_ptr(), dy.data_ptr(), None,
                              None, u.data_ptr(), 3, 2, 1024, None, 0,
                              None) == 1
    assert L.fftconv_backward(conv._plan, u.data_ptr(), dy.data_ptr(), None,
                              None, dk.data_ptr() + 4, 3, 2, 1024, None, 0,
                              None) == 3
    # a multi-pass kernel gradient needs its workspace (rows of u, dy and the
    # result in f16 complex)
    conv2 = fc.FFTConv(32768, dtype="f16")
    u2 = torch.randn(1, 1, 32768, device="cuda").half()
    dk2 = torch.empty(1, 32768, device="cuda")
    need = conv2.backward_workspace_bytes(1, 1)
    assert need >= 3 * 32768 * 4
    assert L.fftconv_backward(conv2._plan, u2.data_ptr(), u2.data_ptr(), None,
                              None, dk2.data_ptr(), 1, 1, 32768, None, 0,
                              None) == 4
    # a workspace overlapping du or dy is rejected before anything launches
    ws2 = torch.empty(need + 2 * 32768 * 2, dtype=torch.uint8, device="cuda")
    dy_in_ws = ws2[need:].view(torch.float16)[:32768]
    du2 = torch.empty(1, 1, 32768, device="cuda").half()
    kfa2 = conv2.kernel_spectrum(torch.randn(1, 32768, device="cuda"),
                                 kind="causal_adjoint")
    assert L.fftconv_backward(conv2._plan, u2.data_ptr(), dy_in_ws.data_ptr(), kfa2.data_ptr(),
                              du2.data_ptr(), dk2.data_ptr(), 1, 1, 32768,
                              ws2.data_ptr() + 2 * 32768 * 2, need, None) == 1
    du_in_ws = ws2.view(torch.float16)[:32768]
    assert L.fftconv_backward(conv2._plan, u2.data_ptr(), u2.data_ptr(), kfa2.data_ptr(),
                              du_in_ws.data_ptr(), dk2.data_ptr(), 1, 1, 32768,
                              ws2.data_ptr(), need, None) == 1
    # where du runs from dk's workspace, an adjoint spectrum inside any part
    # of that workspace is rejected too
    conv3 = fc.FFTConv(65536, dtype="f16")
    u3 = torch.randn(1, 1, 65536, device="cuda").half()
    du3 = torch.empty_like(u3)
    dk3 = torch.empty(1, 65536, device="cuda")
    need3 = conv3.backward_workspace_bytes(1, 1)
    ws3 = torch.empty(need3, dtype=torch.uint8, device="cuda")
    kf_in_ws = ws3.data_ptr() + ((need3 - conv3.spectrum_bytes(1)) & ~255)
    assert L.fftconv_backward(conv3._plan, u3.data_ptr(), u3.data_ptr(), kf_in_ws,
                              du3.data_ptr(), dk3.data_ptr(), 1, 1, 65536,
                              ws3.data_ptr(), need3, None) == 1
    torch.cuda.synchronize()


@pytest.mark.parametrize("N,dtype,B,H", [(65536, "f16", 2, 3), (1048576, "bf16", 1, 2),
                                         (4194304, "bf16", 1, 1)])
def test_backward_pieces_multipass(N, dtype, B, H):
    # on the multi-pass engine a call that asks for both gradients runs du
    # from dk's column pass of dy: it must give the bits of the separate calls
    # (one-level passes, two-level passes, the matrix-core pair at 4M)
    import torch
    from fft_long_convolution_amd import fftconv as fc
    w = inputs.Workload("bwdm", 260 + N.bit_length(), B, H, N, dtype, "normal", "decay", "")
    _say("backward pieces", N, dtype, B, H)
    conv = fc.FFTConv(N, dtype=dtype)
    u_h, dy_h, k = inputs.input_rows(w), inputs.dy_rows(w), inputs.kernel_rows(w)
    u = to_torch(u_h, dtype).view(B, H, N)
    dy = to_torch(dy_h, dtype).view(B, H, N)
    kfa = conv.kernel_spectrum(torch.from_numpy(k).cuda(), kind="causal_adjoint")
    du_all, dk_all = conv.backward(u, dy, kfa)
    du_only, _ = conv.backward(None, dy, kfa, need_dk=False)
    _, dk_only = conv.backward(u, dy, None, need_du=False)
    torch.cuda.synchronize()
    assert torch.equal(du_all.view(torch.int16), du_only.view(torch.int16))
    assert torch.equal(dk_all, dk_only)
    rdu, rdk = oracle_backward(w, u_h, dy_h, k)
    edu = oracle.rel_l2(oracle.to_f64(from_torch(du_all, dtype).reshape(B * H, N), dtype), rdu)
    edk = oracle.rel_l2(dk_all.cpu().numpy().astype(np.float64), rdk)
    _say("  du rel_l2", edu, "dk rel_l2", edk)
    assert edu < TOL[dtype]
    assert edk < TOL[dtype]


@pytest.mark.parametrize("name", ["hyena_bf16_n1k", "m2bert_f16_n8k",
                                  "audio_bf16_n64k"])
def test_backward_full_size(name):
    w = inputs.WORKLOADS[name]
    _say("backward full-size", name)
    du, dk, u, dy, k = run_gpu_backward(w)
    rdu, rdk = oracle_backward(w, u, dy, k)
    edu, edk = oracle.rel_l2(du, rdu), oracle.rel_l2(dk, rdk)
    _say("  du rel_l2", edu, "dk rel_l2", edk)
    assert edu < TOL[w.dtype]
    assert edk < TOL[w.dtype]


def test_backward_channel_chunks():
    # the multi-pass kernel gradient runs over chunks of channels whose rows
    # of u and dy fit the 1 GB workspace chunk (here two channels of 128
    # rows at N = 1M): every channel's whole dk row, on both sides of the
    # chunk boundary, against the oracle's FFT route at the bar
    import torch
    from fft_long_convolution_amd.fftconv import FFTConv
    N, B, H, dtype = 1048576, 128, 3, "f16"
    w = inputs.Workload("kchunk", 261, B, H, N, dtype, "normal", "decay", "kgrad chunks")
    conv = FFTConv(N, dtype=dtype)
    u = inputs.input_rows(w)
    dy = inputs.dy_rows(w)
    _say("kgrad channel chunks", N, B, H, dtype)
    du, dk = conv.backward(to_torch(u, dtype).view(B, H, N), to_torch(dy, dtype).view(B, H, N),
                           None, need_du=False)
    torch.cuda.synchronize()
    assert du is None
    got = dk.cpu().numpy().astype(np.float64)
    del dk
    want = oracle.kgrad_fft(oracle.to_f64(u, dtype).reshape(B * H, N),
                            oracle.to_f64(dy, dtype).reshape(B * H, N), H, "causal",
                            np.arange(B * H) % H)
    for h in range(H):
        err = oracle.rel_l2(got[h], want[h])
        _say("  channel", h, "dk rel_l2", err)
        assert err < TOL[dtype]


@pytest.mark.parametrize("B,H,dtype", [(128, 3, "f16"), (257, 1, "bf16")])
def test_backward_shared_dy_chunks(B, H, dtype):
    # both gradients at once across workspace chunks (two channels per
    # chunk at B = 128, 256 batch rows per chunk at B = 257): du runs from dk's
    # column pass of dy chunk by chunk; its bits must equal the du-only
    # call's, and the rows on both sides of each chunk boundary are held to
    # the bar against the oracle
    import torch
    from fft_long_convolution_amd.fftconv import FFTConv
    N = 1048576
    w = inputs.Workload("sdchunk", 263 + B, B, H, N, dtype, "normal", "decay", "shared dy chunks")
    conv = FFTConv(N, dtype=dtype)
    u_h, dy_h, k = inputs.input_rows(w), inputs.dy_rows(w), inputs.kernel_rows(w)
    _say("shared dy chunks", N, B, H, dtype)
    u = to_torch(u_h, dtype).view(B, H, N)
    dy = to_torch(dy_h, dtype).view(B, H, N)
    del u_h
    kfa = conv.kernel_spectrum(torch.from_numpy(k).cuda(), kind="causal_adjoint")
    du_all, dk_all = conv.backward(u, dy, kfa)
    del dk_all
    du_only, _ = conv.backward(None, dy, kfa, need_dk=False)
    torch.cuda.synchronize()
    assert torch.equal(du_all.view(torch.int16), du_only.view(torch.int16))
    del du_only
    # rows r = b * H + h around the boundaries: channels 1 | 2 of batch rows
    # 0 and B - 1, or batch rows 255 | 256
    rows = [1, 2, (B - 1) * H + 1, (B - 1) * H + 2] if H == 3 else [0, 255, 256]
    got = from_torch(du_all.view(B * H, N)[rows], dtype)
    del du_all
    hidx = np.array(rows) % H
    uh, inv = np.unique(hidx, return_inverse=True)
    ref = oracle.op_fft(oracle.to_f64(dy_h[rows], dtype), k[uh].astype(np.float64),
                        "causal_adjoint", inv)
    for i, r in enumerate(rows):
        err = oracle.rel_l2(oracle.to_f64(got[i:i + 1], dtype), ref[i:i + 1])
        _say("  du row", r, "rel_l2", err)
        assert err < TOL[dtype]


def test_backward_batch_chunks():
    # more batch rows of one channel than the 1 GB workspace chunk holds (256
    # rows at N = 1M): the multi-pass kernel gradient runs per batch chunk and
    # the second chunk adds its share to dk; the whole dk row against the
    # oracle's FFT route at the bar
    import torch
    from fft_long_convolution_amd.fftconv import FFTConv
    N, B, H, dtype = 1048576, 257, 1, "bf16"
    w = inputs.Workload("kbchunk", 262, B, H, N, dtype, "normal", "decay", "kgrad batch chunks")
    conv = FFTConv(N, dtype=dtype)
    u = inputs.input_rows(w)
    dy = inputs.dy_rows(w)
    _say("kgrad batch chunks", N, B, H, dtype)
    _, dk = conv.backward(to_torch(u, dtype).view(B, H, N), to_torch(dy, dtype).view(B, H, N),
                          None, need_du=False)
    torch.cuda.synchronize()
    got = dk.cpu().numpy().astype(np.float64)
    del dk
    # dk is a sum over the batch rows: the oracle computes it as the sum of
    # the gradients of 16 disjoint row groups (the oracle's threads run over
    # channels, so the groups are passed as 16 channels and summed here)
    part = oracle.kgrad_fft(oracle.to_f64(u, dtype).reshape(B, N),
                            oracle.to_f64(dy, dtype).reshape(B, N), 16, "causal",
                            np.arange(B, dtype=np.int64) % 16)
    want = part.sum(axis=0)
    err = oracle.rel_l2(got[0], want)
    _say("  dk rel_l2", err)
    assert err < TOL[dtype]
