"""The seeded workload generators (no GPU)."""
import numpy as np
import pytest
import torch

from fft_long_convolution_amd import inputs


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.uniform(
        -30, 30, 100000), [0.0, -0.0, 1.0, 65504.0, 1e-40, 3.0e38]])
    x32 = x.astype(np.float32)
    want = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16)
    got = inputs.f32_to_bf16_bits(x32).view(np.int16)
    np.testing.assert_array_equal(got, want.numpy())


def test_reproducible_and_row_independent():
    w = inputs.shrink(inputs.WORKLOADS["hyena_bf16_n1k"], B=2, H=8)
    a = inputs.input_rows(w)
    b = inputs.input_rows(w, [3, 9, 15])
    np.testing.assert_array_equal(a[[3, 9, 15]], b)
    ka = inputs.kernel_rows(w)
    kb = inputs.kernel_rows(w, [5])
    np.testing.assert_array_equal(ka[5], kb[0])
    assert a.dtype == np.uint16 and ka.dtype == np.float32
    assert a.shape == (16, 1024) and ka.shape == (8, 1024)


def test_distributions():
    w = inputs.shrink(inputs.WORKLOADS["m2bert_f16_n8k"], B=1, H=16)
    u = inputs.input_rows(w).astype(np.float64)
    assert u.shape == (16, 8192)
    assert abs(u.mean()) < 0.02 and abs(u.std() - 1.0) < 0.02
    a = inputs.decay_rates(inputs.WORKLOADS["hyena_bf16_n1k"])
    assert a.shape == (768,) and a.min() >= 1e-3 and a.max() <= 1e-1
    lg = np.log10(a)
    assert abs(lg.mean() + 2.0) < 0.1          # log-uniform on [-3, -1]
    k = inputs.kernel_rows(w, [0]).astype(np.float64)[0]
    # the envelope decays: late taps are much smaller than early ones
    assert np.abs(k[-1000:]).max() < np.abs(k[:100]).max()


def test_tiny_kernel_scale():
    w = inputs.WORKLOADS["tiny_f32_n256"]
    k = inputs.kernel_rows(w).astype(np.float64)
    assert k.shape == (4, 256)
    assert abs(k.std() * 16.0 - 1.0) < 0.1     # N(0,1)/sqrt(256)


def test_audio_has_tones():
    w = inputs.shrink(inputs.WORKLOADS["audio_bf16_n64k"], B=1, H=2)
    bits = inputs.input_rows(w, [1])
    x = (bits.astype(np.uint32) << 16).view(np.float32)[0].astype(float)
    spec = np.abs(np.fft.rfft(x))
    # 8 tones stand far above the 0.1 noise floor
    top = np.sort(spec)[-8:]
    assert top.min() > 20 * np.median(spec)


def test_genome_one_hot():
    w = inputs.shrink(inputs.WORKLOADS["genome_bf16_n4m"], N=4194304)
    rows = [0, 31, 32, 64, 127]
    bits = inputs.input_rows(w, rows)
    x = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert set(np.unique(x)) <= {0.0, 1.0}
    assert x[:, inputs.GENOME_LEN:].sum() == 0
    # rows 0 and 31 are the same channel group; groups 0, 1, 2 are disjoint
    np.testing.assert_array_equal(x[0], x[1])
    assert (x[0] * x[2]).sum() == 0 and (x[2] * x[3]).sum() == 0
    frac = x[:, :inputs.GENOME_LEN].mean(axis=1)
    assert np.all(np.abs(frac - 0.25) < 0.01)


@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
def test_workload_shapes(name):
    w = inputs.WORKLOADS[name]
    assert w.N & (w.N - 1) == 0 and w.N >= 256
    assert w.dtype in ("f32", "f16", "bf16")


def test_gate_rows():
    w = inputs.shrink(inputs.WORKLOADS["hyena_bf16_n1k"], B=2, H=4)
    gw = inputs.gate_rows(w, "w")
    gv = inputs.gate_rows(w, "v")
    assert gw.shape == (8, 1024) and gw.dtype == np.uint16
    # reproducible, row-independent, and distinct from u and from each other
    np.testing.assert_array_equal(inputs.gate_rows(w, "w", [5])[0], gw[5])
    u = inputs.input_rows(w)
    assert not np.array_equal(gw, gv) and not np.array_equal(gw, u)
    x = (gv.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert abs(x.mean()) < 0.05 and abs(x.std() - 1.0) < 0.05
