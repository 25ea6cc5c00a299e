"""MI355X-native causal FFT long convolution.

``y[b,h,t] = sum_{s<=t} u[b,h,s] * k[h,t-s]`` computed as a zero-padded
(2N) FFT convolution whose DFTs are factored into small dense DFT-matrix
products on the gfx950 matrix cores (the Monarch form of the FFT described
on the FlashFFTConv page, section 3.4).

The compute path is the HIP library ``libfftconv.so`` behind the C ABI in
``include/fftconv.h``; :mod:`fft_long_convolution_amd.fftconv` is a thin
ctypes binding over it that uses PyTorch only for device memory and streams.
Importing this package loads nothing; the library is opened on first use.
"""
import importlib

__all__ = ["FFTConv", "fftconv", "inputs"]


def __getattr__(name):
    if name in ("fftconv", "inputs"):
        return importlib.import_module(__name__ + "." + name)
    if name == "FFTConv":
        return importlib.import_module(__name__ + ".fftconv").FFTConv
    raise AttributeError(name)
