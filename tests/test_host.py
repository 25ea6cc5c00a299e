"""Host-side checks of libfftconv (no GPU): the shared library loads, exports
every function include/fftconv.h declares, plans every supported length,
and rejects bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

from fft_long_convolution_amd import fftconv as fc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    src = open(os.path.join(ROOT, "include", "fftconv.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fftconv_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = _header_functions()
    assert len(names) >= 10
    L = fc.lib()
    for n in names:
        assert hasattr(L, n), n
    assert fc.lib().fftconv_version().startswith(b"fftconv")


def test_status_strings():
    L = fc.lib()
    for s in range(6):
        assert L.fftconv_status_string(s)
    assert L.fftconv_status_string(99) == b"unknown status"


@pytest.mark.parametrize("lg", range(8, 23))
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_plan_query_every_length(lg, dtype):
    N = 1 << lg
    info = fc.plan_query(N, 0, dtype)
    prod = 1
    fac = info["factors"]
    for i, f in enumerate(fac):
        if info["kernel"] == "wide_kernel" and i == 0:
            # vector-ALU outer stage of radix 4..16 before the 32 x 32 engine
            assert f in (4, 8, 16)
        elif info["kernel"].startswith("mp_") and i == len(fac) - 3:
            # multi-pass: 4096-point inner slabs, 4 x 32 x 32
            assert f == 4
        else:
            assert f in (8, 16, 32)
        prod *= f
    assert prod == N and info["M"] == N
    assert info["factors"][-1] in (16, 32)
    assert info["path"] == ("fused" if N <= 16384 else "multipass")
    entry = 16 if dtype == "f32" else 8
    assert info["spectrum_bytes_per_channel"] == N * entry
    # workspace: f16 complex on the 16-bit multi-pass path, fp32 otherwise
    ws = 0 if N <= 16384 else (8 * N if dtype == "f32" else 4 * N)
    assert info["workspace_bytes_per_row"] == ws
    if N > 16384 and dtype != "f32":
        # one outer level up to P_o = 32 (N = 128K), two above
        two = N > 131072
        assert info["outer_factors"] == (2 if two else 1)
        if not two:
            assert info["kernel"] == "mp_col_kernel+mp_inner_kernel"
        elif fac[:2] == [32, 32]:
            assert info["kernel"] == "mp_col2m_fwd_kernel+mp_inner_kernel+mp_col2m_inv_kernel"
        else:
            assert info["kernel"] == "mp_col2_kernel+mp_inner_kernel"
        assert fac[-3:] == [4, 32, 32]
    # matrix-core flops: 16 M (N_1/2 + sum_{i>1} N_i) per row
    f = info["factors"]
    want = 16.0 * N * (f[0] / 2 + sum(f[1:]))
    assert info["mfma_flops_per_row"] == pytest.approx(want)


def test_default_orders_follow_length():
    assert fc.plan_query(1024)["factors"] == [32, 32]
    # 16-bit I/O at 4K..16K: P x 32 x 32 on the wide kernel
    for lg, P in ((12, 4), (13, 8), (14, 16)):
        for dt in ("f16", "bf16"):
            info = fc.plan_query(1 << lg, 0, dt)
            assert info["factors"] == [P, 32, 32]
            assert info["kernel"] == "wide_kernel"
    assert fc.plan_query(8192, 0, "f32")["factors"] == [32, 16, 16]
    assert fc.plan_query(8192, 0, "f32")["kernel"] == "fused_kernel"
    assert fc.plan_query(65536)["order"] == 4
    assert fc.plan_query(1 << 22)["order"] == 5


def test_requested_order():
    assert fc.plan_query(1024, 3)["factors"] == [8, 8, 16]
    assert fc.plan_query(8192, 3)["factors"] == [8, 32, 32]
    assert fc.plan_query(8192, 3, "f32")["factors"] == [32, 16, 16]
    for N, p in ((256, 3), (4096, 2)):   # needs a radix outside 8..32
        with pytest.raises(fc.FFTConvError) as e:
            fc.plan_query(N, p)
        assert e.value.status == 2


@pytest.mark.parametrize("N", [0, 1, 128, 255, 1000, 3 << 10, 1 << 23])
def test_unsupported_lengths(N):
    with pytest.raises(fc.FFTConvError) as e:
        fc.plan_query(N, 0, "bf16")
    assert e.value.status == 2


def test_bad_dtype_and_order():
    L = fc.lib()
    info = fc.PlanInfo()
    assert L.fftconv_plan_query(1024, 0, 7, ctypes.byref(info)) == 2
    assert L.fftconv_plan_query(1024, 1, 2, ctypes.byref(info)) == 2
    assert L.fftconv_plan_query(1024, -1, 2, ctypes.byref(info)) == 2
    assert L.fftconv_plan_query(1024, 0, 2, None) == 1


def test_null_plan_is_rejected_without_device():
    L = fc.lib()
    assert L.fftconv_forward(None, 16, 16, 16, 1, 1, 256, None, 0, None) == 1
    assert L.fftconv_forward_gated(None, 16, 16, 16, 16, 16, 1, 1, 256, None,
                                   0, None) == 1
    assert L.fftconv_backward(None, 16, 16, 16, 16, 16, 1, 1, 256, None, 0,
                              None) == 1
    assert L.fftconv_backward_workspace_bytes(None, 1, 1) == 0
    assert L.fftconv_kernel_spectrum_kind(None, 16, 1, 0, 16, None) == 1
    assert L.fftconv_kernel_spectrum(None, 16, 1, 16, None) == 1
    assert L.fftconv_spectrum_bytes(None, 4) == 0
    assert L.fftconv_workspace_bytes(None, 1, 1) == 0
    assert L.fftconv_plan(1024, 0, 2, None) == 1
    info = fc.PlanInfo()
    assert L.fftconv_plan_get_info(None, ctypes.byref(info)) == 1
    L.fftconv_plan_destroy(None)


def test_python_binding_marshals_only():
    # the binding module must not carry any transform arithmetic: no FFT,
    # no torch.fft, no matmul -- every step runs in the HIP library
    src = open(fc.__file__).read()
    for bad in ("torch.fft", "np.fft", "matmul", "einsum", "import oracle",
                "from oracle"):
        assert bad not in src
