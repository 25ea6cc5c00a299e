"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Tolerances are the relative L2 bounds the method is held to: 2e-3 for
16-bit I/O (bf16 output rounding alone costs ~1.7e-3), 1e-5 for fp32 I/O.
"""
import sys

import numpy as np
import pytest

from fft_long_convolution_amd import inputs
from tests.gpu_helpers import TOL, oracle_rows, parity, run_gpu

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
                               32768, 65536])
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
                                     (1024, "f16")])
def test_generic_kernel_at_row_lengths(N, dtype, monkeypatch):
    # lengths 32*16 and 32*32 normally run the register-resident row
    # kernel; the LDS-staged kernel must agree with the oracle there too
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
