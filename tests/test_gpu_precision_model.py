"""The row kernel against its rounding model (tests/precision_model.py) on
the same rows: the model's predicted error must match the kernel's measured
error, and the kernel's outputs must sit far closer to the model's than to
the exact result (the model reproduces where the error comes from, not
just its size)."""
import sys
from dataclasses import replace

import numpy as np
import pytest

import oracle
from fft_long_convolution_amd import inputs
from tests import precision_model as pm
from tests.gpu_helpers import run_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_row_kernel_matches_rounding_model(dtype):
    w = replace(inputs.WORKLOADS["hyena_bf16_n1k"], B=2, H=128, dtype=dtype)
    print("rounding model", dtype, w.B, w.H, w.N, flush=True)
    y, u, k = run_gpu(w)
    u64 = oracle.to_f64(u, dtype)
    k64 = k.astype(np.float64)
    hidx = np.arange(w.rows) % w.H
    ref = oracle.conv_fft(u64, k64, hidx)
    model = pm.row_kernel(u64, k64, hidx, dtype)
    e_gpu, e_model = oracle.rel_l2(y, ref), oracle.rel_l2(model, ref)
    e_between = oracle.rel_l2(y, model)
    print("  measured", e_gpu, "predicted", e_model, "kernel vs model", e_between, flush=True)
    sys.stdout.flush()
    # measured on MI355X: bf16 1.77419e-3 against 1.77420e-3 predicted, the
    # kernel 2.4e-4 from the model; f16 6.778e-4 against 6.777e-4, 7.9e-5
    assert abs(e_gpu - e_model) < 0.01 * e_model
    assert e_between < 0.2 * e_gpu
