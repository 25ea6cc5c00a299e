"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Tolerances are the relative L2 bounds the method is held to: 2e-3 for
16-bit I/O (bf16 output rounding alone costs ~1.7e-3), 1e-5 for fp32 I/O.
"""
import sys

import numpy as np
import pytest

from fft_long_convolution_amd import inputs
from tests.gpu_helpers import TOL, from_torch, oracle_rows, parity, run_gpu, to_torch
import oracle

pytestmark = pytest.mark.gpu

W = inputs.WORKLOADS


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def test_tiny_fp32_full():
    w = W["tiny_f32_n256"]
    err, _, _ = parity(w)
    _say("tiny_f32_n256 rel_l2", err)
    assert err < TOL["f32"]


@pytest.mark.parametrize("name,B,H", [
    ("hyena_bf16_n1k", 2, 48),
    ("m2bert_f16_n8k", 1, 24),
    ("audio_bf16_n64k", 1, 6),
    ("genome_bf16_n4m", 1, 2),
])
def test_workload_rows(name, B, H):
    w = inputs.shrink(W[name], B=B, H=H)
    err, _, _ = parity(w)
    _say(name, B, H, "rel_l2", err)
    assert err < TOL[w.dtype]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("N", [256, 512, 1024, 2048, 4096, 8192, 16384,
                               32768, 65536, 131072])
def test_length_sweep(N, dtype):
    # seeded N(0,1) input and decaying kernel at every supported length;
    # B*H = 3*5 rows so tiles see a ragged row count
    base = W["hyena_bf16_n1k"]
    w = inputs.Workload("sweep", 40 + N.bit_length(), 3, 5, N, dtype,
                        "normal", "decay", "sweep")
    err, _, _ = parity(w)
    _say("sweep", N, dtype, "rel_l2", err)
    assert err < TOL[dtype]


@pytest.mark.parametrize("N,dtype", [(512, "bf16"), (1024, "bf16"),
                                     (1024, "f16"), (4096, "bf16"),
                                     (8192, "f16"), (16384, "bf16")])
def test_generic_kernel_at_row_lengths(N, dtype, monkeypatch):
    # lengths 32*16, 32*32 and P*32*32 normally run the register-resident
    # row and wide kernels; the LDS-staged kernel must agree with the oracle
    # there too
    monkeypatch.setenv("FFTCONV_KERNEL", "generic")
    w = inputs.Workload("generic", 60 + N.bit_length(), 4, 7, N, dtype,
                        "normal", "decay", "generic kernel")
    err, _, _ = parity(w)
    _say("generic", N, dtype, "rel_l2", err)
    assert err < TOL[dtype]


@pytest.mark.parametrize("B,H", [(1, 1), (3, 2), (5, 9), (64, 3), (33, 4)])
def test_row_kernel_batch_shapes(B, H):
    # batch sizes that leave workgroups and waves partly empty
    w = inputs.Workload("rowshape", 70 + B, B, H, 1024, "bf16", "normal",
                        "decay", "row kernel shapes")
    err, _, _ = parity(w)
    _say("row shapes", B, H, "rel_l2", err)
    assert err < TOL["bf16"]


@pytest.mark.parametrize("dtype,B,H", [("bf16", 5, 77), ("f16", 64, 7), ("bf16", 3, 512),
                                         ("f16", 1, 1000), ("bf16", 7, 1)])
def test_row_pairs_every_row(dtype, B, H):
    # plain N = 1024 rows go two per wave: odd slices (the last pair holds
    # one row), pairs that straddle a channel boundary, slices over several
    # channels; every row held to the bar relative to its conditioning, so
    # that one wrong row of a pair cannot hide in the whole-tensor norm
    w = inputs.Workload("rowpairs", 90 + B + H, B, H, 1024, dtype, "normal", "decay",
                        "paired rows")
    err, y, ref = parity(w)
    u64 = oracle.to_f64(inputs.input_rows(w), dtype).reshape(w.rows, w.N)
    kmax = np.max(np.abs(oracle.kernel_spectrum(inputs.kernel_rows(w).astype(np.float64))), axis=1)
    scale = np.linalg.norm(u64, axis=1) * kmax[np.arange(w.rows) % H]
    worst = float(np.max(np.linalg.norm(y - ref, axis=1) / scale))
    _say("row pairs", dtype, B, H, "rel_l2", err, "worst row (conditioned)", worst)
    assert err < TOL[dtype]
    assert worst < TOL[dtype]


@pytest.mark.parametrize("N,dtype,B,H", [
    (4096, "f16", 1, 1), (4096, "bf16", 7, 3), (8192, "f16", 1, 1),
    (8192, "f16", 5, 9), (8192, "bf16", 33, 2), (16384, "f16", 3, 1),
    (16384, "bf16", 2, 7), (32768, "f16", 1, 1), (32768, "bf16", 3, 5),
    (32768, "f16", 17, 3), (32768, "bf16", 64, 9)])
def test_wide_kernel_batch_shapes(N, dtype, B, H):
    # row counts that leave the persistent workgroups' slices ragged and
    # cross channel boundaries inside a slice
    w = inputs.Workload("wideshape", 80 + N.bit_length() + B, B, H, N, dtype,
                        "normal", "decay", "wide kernel shapes")
    err, _, _ = parity(w)
    _say("wide shapes", N, dtype, B, H, "rel_l2", err)
    assert err < TOL[dtype]


@pytest.mark.parametrize("N,dtype,B,H", [
    (262144, "f16", 1, 3), (262144, "bf16", 2, 1), (524288, "bf16", 1, 2),
    (1048576, "f16", 1, 2), (2097152, "bf16", 1, 1), (4194304, "f16", 1, 1)])
def test_two_level_multipass(N, dtype, B, H):
    # every factor pair of the two outer levels (8x8, 16x8, 16x16, 32x16,
    # 32x32) through the passes that keep level 1 in LDS
    w = inputs.Workload("twolevel", 100 + N.bit_length() + B, B, H, N, dtype,
                        "normal", "decay", "two-level multi-pass")
    err, _, _ = parity(w)
    _say("two-level", N, dtype, B, H, "rel_l2", err)
    assert err < TOL[dtype]


@pytest.mark.parametrize("N,B,H", [(262144, 1, 3), (1048576, 1, 2),
                                   (4194304, 1, 1)])
def test_fp32_multipass(N, B, H):
    # fp32 I/O above 128K runs the LDS-staged passes with two outer levels
    # and an fp32 workspace (8192-point slabs from 512K on); held at the
    # fp32 bar
    w = inputs.Workload("f32mp", 140 + N.bit_length(), B, H, N, "f32",
                        "normal", "decay", "fp32 multi-pass")
    err, _, _ = parity(w)
    _say("fp32 multi-pass", N, B, H, "rel_l2", err)
    assert err < TOL["f32"]


def _plan_and_spectrum(N, dtype, H=3):
    import torch
    from fft_long_convolution_amd.fftconv import FFTConv
    conv = FFTConv(N, dtype=dtype)
    k = torch.from_numpy(inputs.kernel_rows(
        inputs.Workload("edge", 90, 1, H, N, dtype, "normal", "decay", ""))).cuda()
    return conv, conv.kernel_spectrum(k)


def test_empty_batch_is_a_noop():
    import torch
    conv, kf = _plan_and_spectrum(1024, "bf16")
    u = torch.empty(0, 3, 1024, dtype=torch.bfloat16, device="cuda")
    y = conv.forward(u, kf)
    torch.cuda.synchronize()
    assert y.shape == (0, 3, 1024)


def test_error_paths():
    import torch
    from fft_long_convolution_amd import fftconv as fc
    conv, kf = _plan_and_spectrum(1024, "bf16")
    L = fc.lib()
    u = torch.randn(2, 3, 1024, device="cuda").to(torch.bfloat16)
    y = torch.empty_like(u)
    s = None
    # wrong N
    assert L.fftconv_forward(conv._plan, u.data_ptr(), kf.data_ptr(),
                             y.data_ptr(), 2, 3, 512, None, 0, s) == 1
    # misaligned input pointer
    assert L.fftconv_forward(conv._plan, u.data_ptr() + 2, kf.data_ptr(),
                             y.data_ptr(), 2, 3, 1024, None, 0, s) == 3
    # output overlapping the input
    assert L.fftconv_forward(conv._plan, u.data_ptr(), kf.data_ptr(),
                             u.data_ptr() + 1024, 2, 3, 1024, None, 0, s) == 1
    # null spectrum
    assert L.fftconv_forward(conv._plan, u.data_ptr(), None, y.data_ptr(),
                             2, 3, 1024, None, 0, s) == 1
    # multi-pass plan with a missing / short workspace
    conv2, kf2 = _plan_and_spectrum(65536, "bf16", H=1)
    u2 = torch.randn(1, 1, 65536, device="cuda").to(torch.bfloat16)
    y2 = torch.empty_like(u2)
    need = conv2.workspace_bytes(1, 1)
    # one f16 complex row (a single-channel chunk) and the claim counters
    assert need == 65536 * 4 + 1024
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    assert L.fftconv_forward(conv2._plan, u2.data_ptr(), kf2.data_ptr(),
                             y2.data_ptr(), 1, 1, 65536, None, 0, s) == 4
    assert L.fftconv_forward(conv2._plan, u2.data_ptr(), kf2.data_ptr(),
                             y2.data_ptr(), 1, 1, 65536, ws.data_ptr(),
                             need - 16, s) == 4
    assert L.fftconv_forward(conv2._plan, u2.data_ptr(), kf2.data_ptr(),
                             y2.data_ptr(), 1, 1, 65536, ws.data_ptr(),
                             need, s) == 0
    torch.cuda.synchronize()
    with pytest.raises(fc.FFTConvError):
        fc.FFTConv(1000, dtype="bf16")


@pytest.mark.parametrize("N", [1024, 8192, 65536])
def test_deterministic_and_stream(N):
    import torch
    conv, kf = _plan_and_spectrum(N, "bf16")
    u = torch.randn(4, 3, N, device="cuda").to(torch.bfloat16)
    y1 = conv.forward(u, kf)
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        y2 = conv.forward(u, kf)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("N,B,dtype", [(1048576, 257, "f16"), (4194304, 65, "bf16")])
def test_multipass_batch_chunks(N, B, dtype):
    # one channel's rows exceed the 1 GB workspace chunk: the passes run over
    # slices of the batch.  The whole rows on both sides of every slice
    # boundary (and the first and last row) are compared with the oracle's
    # FFT route, each row on its own at the bar
    import torch
    from fft_long_convolution_amd.fftconv import FFTConv
    w = inputs.Workload("bchunk", 120 + N.bit_length(), B, 1, N, dtype,
                        "normal", "decay", "batch chunks")
    conv = FFTConv(N, dtype=dtype)
    u = inputs.input_rows(w)
    k = inputs.kernel_rows(w)
    kf = conv.kernel_spectrum(torch.from_numpy(k).cuda())
    y = conv.forward(to_torch(u, dtype).view(B, 1, N), kf)
    torch.cuda.synchronize()
    slice_rows = (1 << 30) // (N * 4)
    assert slice_rows < B
    rows = sorted({0, B - 1} | {r for s0 in range(slice_rows, B, slice_rows)
                                for r in (s0 - 1, s0)})
    got = oracle.to_f64(from_torch(y, dtype).reshape(B, N)[rows], dtype)
    del y
    want = oracle.conv_fft(oracle.to_f64(u[rows], dtype), k.astype(np.float64),
                           np.zeros(len(rows), dtype=np.int64))
    for i, r in enumerate(rows):
        err = oracle.rel_l2(got[i], want[i])
        _say("batch chunks", N, B, dtype, "row", r, "rel_l2", err)
        assert err < TOL[dtype]
