"""The row kernel's rounding model (tests/precision_model.py), pinned: with
no rounding it is the causal convolution (the oracle's FFT route and the
definition), its rounding helpers are the IEEE operations they stand for,
and its prediction for the Hyena-shaped rows sits between the output
rounding alone and the 2e-3 bar (the GPU comparison is in
test_gpu_precision_model.py)."""
from dataclasses import replace

import numpy as np
import torch

import oracle
from fft_long_convolution_amd import inputs
from tests import precision_model as pm


def _rows(dtype, B=2, H=128):
    w = replace(inputs.WORKLOADS["hyena_bf16_n1k"], B=B, H=H, dtype=dtype)
    u64 = oracle.to_f64(inputs.input_rows(w), dtype)
    k64 = inputs.kernel_rows(w).astype(np.float64)
    return w, u64, k64, np.arange(w.rows) % w.H


def test_exact_model_is_the_convolution():
    # every stage, the pairing coefficients and the index maps, with no
    # rounding: the causal convolution to fp64 accuracy
    w, u64, k64, hidx = _rows("bf16", B=2, H=5)
    y = pm.row_kernel(u64, k64, hidx, "bf16", exact=True)
    assert oracle.rel_l2(y, oracle.conv_fft(u64, k64, hidx)) < 1e-12
    assert oracle.rel_l2(y[:3], oracle.conv_direct(u64[:3], k64, hidx[:3])) < 1e-12


def test_pair_coefficients_special_cases():
    # a delta kernel at tap 0 is the identity: alpha = 1, beta = 0
    k = np.zeros((1, pm.M))
    k[0, 0] = 1.0
    al, be = pm.pair_coefficients(k)
    assert np.allclose(al, 1.0, atol=1e-12) and np.allclose(be, 0.0, atol=1e-12)
    # a delta at tap 2 shifts the packed row by one point: alpha = W_M^k
    k[0, 0], k[0, 2] = 0.0, 1.0
    al, be = pm.pair_coefficients(k)
    kk = np.arange(pm.M)
    assert np.allclose(al[0], np.exp(-2j * np.pi * kk / pm.M), atol=1e-12)
    assert np.allclose(be, 0.0, atol=1e-12)


def test_rounding_helpers_are_ieee():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(4096) * 10.0 ** rng.uniform(-3, 3, 4096)
    # bf16: torch's round-to-nearest-even conversion
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).float().numpy()
    assert np.array_equal(pm._bf16(x), want.astype(np.float64))
    # packed f16 complex products: one f16 rounding per multiply and per
    # fused multiply-add, so within 2 ulp of the exact product per half
    a = pm._f16(rng.standard_normal(4096) + 1j * rng.standard_normal(4096))
    t = pm._f16(np.exp(1j * rng.uniform(0, 2 * np.pi, 4096)))
    for conj in (False, True):
        exact = a * (np.conj(t) if conj else t)
        got = pm._hmul(a, t, conj)
        ulp = np.spacing(np.abs(exact).astype(np.float16)).astype(np.float64)
        assert np.all(np.abs(got - exact) <= 2.5 * ulp)
    # the pairing: a z + b conj(p), four roundings per half
    z, p = a, pm._f16(a[::-1] * 0.7)
    exact = t * z + t[::-1] * np.conj(p)
    got = pm._hpair(t, z, t[::-1], p)
    scale = np.abs(z) + np.abs(p)
    assert np.all(np.abs(got - exact) <= 4 * np.spacing(scale.astype(np.float16)).astype(np.float64))


def test_model_prediction_hyena_rows():
    # bf16 I/O: above the output rounding alone (the stages' f16 roundings
    # add to it), below the bar; f16 I/O: below the bar by a wide margin
    w, u64, k64, hidx = _rows("bf16")
    ref = oracle.conv_fft(u64, k64, hidx)
    pred = oracle.rel_l2(pm.row_kernel(u64, k64, hidx, "bf16"), ref)
    floor = oracle.rel_l2(pm._bf16(ref), ref)
    print("bf16 predicted", pred, "output rounding alone", floor)
    assert floor < pred < 2e-3
    w, u64, k64, hidx = _rows("f16")
    ref = oracle.conv_fft(u64, k64, hidx)
    pred = oracle.rel_l2(pm.row_kernel(u64, k64, hidx, "f16"), ref)
    print("f16 predicted", pred)
    assert pred < 1e-3
