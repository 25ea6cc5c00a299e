"""fp64 CPU oracle for the causal long convolution -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never loads it, and it
shares no code with the GPU library.

It wraps ``oracle.c`` (plain C, fp64, OpenMP over rows), which computes
(page "FlashFFTConv: Efficient Convolutions for Long Sequences with Tensor
Cores", section 3.4):

* ``conv_direct``  -- the causal convolution by its definition,
  ``y[r, t] = sum_{s<=t} u[r, s] * k[h(r), t - s]``;
* ``conv_fft``     -- the same through the convolution theorem with both
  sequences zero-padded to 2N (iterative radix-2 FFT, no packing tricks);
* ``conv_points``  -- single outputs by the definition (for sampled checks);
* ``fft``          -- the radix-2 DFT itself, exposed for the oracle's pins;
* ``op_direct`` / ``op_fft`` / ``op_points`` -- the operator family of
  ``oracle.c`` by kind: "causal" (the convolution above), "causal_adjoint"
  (its transpose, ``y[s] = sum_{t>=s} u[t] k[t-s]``, the input gradient),
  "circular" (``y[t] = sum_s u[s] k[(t-s) mod N]``, the non-causal
  convolution with an FFT of size N) and "circular_adjoint";
* ``kgrad_direct`` / ``kgrad_fft`` / ``kgrad_points`` -- the kernel
  gradient ``dk[h][j] = sum_{rows of h} sum_t dy[t] u[t-j]`` (t-j mod N for
  the circular kinds);
* ``lowpass_fft`` -- the frequency-sparse (band-limited) convolution: the
  2N-point kernel spectrum zeroed beyond a cutoff frequency F;
* ``masked_fft`` / ``blocksparse_mask`` / ``blocksparse_fft`` -- the
  frequency-sparse convolution whose zero blocks follow the transform's
  digits (a bins of the top digit, d outer classes);
* ``gated_direct`` / ``gated_fft`` / ``gated_points`` -- the gated
  convolution ``y = v * ((u * w) conv k)`` (elementwise gates on the input
  and on the output; same page, section 3 "Technical Approach",
  "Domain-Specific Optimizations", gating operation fusion), by the same
  three routes.

Inputs are the exact values stored in the I/O dtype (bf16 bit patterns are
widened exactly); everything is evaluated in fp64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (-O2 -fopenmp)."""
    if (not force and os.path.exists(_LIB_PATH)
            and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC)):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        d = ctypes.POINTER(ctypes.c_double)
        lp = ctypes.POINTER(ctypes.c_long)
        L = ctypes.c_long
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_conv_direct.argtypes = [d, d, lp, d, L, L]
        lib.oracle_conv_direct.restype = None
        lib.oracle_conv_points.argtypes = [d, d, lp, L, lp, lp, L, d]
        lib.oracle_conv_points.restype = None
        lib.oracle_fft.argtypes = [d, d, L, ctypes.c_int]
        lib.oracle_fft.restype = None
        lib.oracle_kernel_spectrum.argtypes = [d, L, L, d, d]
        lib.oracle_kernel_spectrum.restype = None
        lib.oracle_conv_fft.argtypes = [d, d, lp, d, L, L, L]
        lib.oracle_conv_fft.restype = ctypes.c_int
        I = ctypes.c_int
        lib.oracle_op_direct.argtypes = [d, d, lp, d, L, L, I]
        lib.oracle_op_direct.restype = None
        lib.oracle_op_points.argtypes = [d, d, lp, L, lp, lp, L, I, d]
        lib.oracle_op_points.restype = None
        lib.oracle_op_fft.argtypes = [d, d, lp, d, L, L, L, I]
        lib.oracle_op_fft.restype = ctypes.c_int
        lib.oracle_kgrad_direct.argtypes = [d, d, lp, d, L, L, L, I]
        lib.oracle_kgrad_direct.restype = None
        lib.oracle_kgrad_fft.argtypes = [d, d, lp, d, L, L, L, I]
        lib.oracle_kgrad_fft.restype = ctypes.c_int
        lib.oracle_kgrad_points.argtypes = [d, d, lp, L, L, lp, lp, L, I, d]
        lib.oracle_kgrad_points.restype = None
        lib.oracle_lowpass_fft.argtypes = [d, d, lp, d, L, L, L, L]
        lib.oracle_lowpass_fft.restype = ctypes.c_int
        lib.oracle_masked_fft.argtypes = [d, d, lp, d, L, L, L, d]
        lib.oracle_masked_fft.restype = ctypes.c_int
        _lib = lib
    return _lib


def num_threads() -> int:
    """Threads the oracle's OpenMP loops use."""
    return int(_load().oracle_num_threads())


def _dp(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _lp(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_long))


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 value of stored data.  ``dtype`` is 'f32', 'f16' or 'bf16'
    (bf16 is carried as uint16 bit patterns)."""
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    return np.asarray(a).astype(np.float64)


def _rows(u, k, hidx):
    u = np.ascontiguousarray(u, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    R, N = u.shape
    if k.ndim != 2 or k.shape[1] != N:
        raise ValueError("kernel rows must have the same length as u rows")
    if hidx is None:
        hidx = np.arange(R) % k.shape[0]
    hidx = np.ascontiguousarray(hidx, dtype=np.int64)
    if hidx.shape != (R,) or (R and (hidx.min() < 0 or hidx.max() >= k.shape[0])):
        raise ValueError("bad kernel row index")
    return u, k, hidx, R, N


def conv_direct(u, k, hidx=None) -> np.ndarray:
    """y[r, t] = sum_{s<=t} u[r, s] k[hidx[r], t-s]  (fp64, O(N^2) per row).
    ``u``: [R, N]; ``k``: [Hk, N]; default ``hidx[r] = r % Hk`` (the
    [B][H][N] row order)."""
    u, k, hidx, R, N = _rows(u, k, hidx)
    y = np.empty((R, N), dtype=np.float64)
    _load().oracle_conv_direct(_dp(u), _dp(k), _lp(hidx), _dp(y), R, N)
    return y


def conv_fft(u, k, hidx=None) -> np.ndarray:
    """Same result via zero-padded (2N) radix-2 FFT convolution (fp64)."""
    u, k, hidx, R, N = _rows(u, k, hidx)
    if N & (N - 1):
        raise ValueError("conv_fft needs a power-of-two N")
    y = np.empty((R, N), dtype=np.float64)
    rc = _load().oracle_conv_fft(_dp(u), _dp(k), _lp(hidx), _dp(y), R,
                                 k.shape[0], N)
    if rc != 0:
        raise MemoryError("oracle_conv_fft: allocation failed")
    return y


def conv_points(u, k, rows, ts, hidx=None) -> np.ndarray:
    """out[i] = y[rows[i], ts[i]] by the definition."""
    u, k, hidx, R, N = _rows(u, k, hidx)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    ts = np.ascontiguousarray(ts, dtype=np.int64)
    if rows.shape != ts.shape or rows.ndim != 1:
        raise ValueError("rows and ts must be 1-D of equal length")
    if len(rows) and (rows.min() < 0 or rows.max() >= R or ts.min() < 0
                      or ts.max() >= N):
        raise ValueError("sample index out of range")
    out = np.empty(len(rows), dtype=np.float64)
    _load().oracle_conv_points(_dp(u), _dp(k), _lp(hidx), N, _lp(rows),
                               _lp(ts), len(rows), _dp(out))
    return out


KINDS = {"causal": 0, "causal_adjoint": 1, "circular": 2,
         "circular_adjoint": 3}


def _kind(kind: str) -> int:
    if kind not in KINDS:
        raise ValueError("unknown operator kind %r" % (kind,))
    return KINDS[kind]


def op_direct(u, k, kind: str, hidx=None) -> np.ndarray:
    """Operator ``kind`` by its definition (fp64, O(N^2) per row)."""
    kd = _kind(kind)
    u, k, hidx, R, N = _rows(u, k, hidx)
    y = np.empty((R, N), dtype=np.float64)
    _load().oracle_op_direct(_dp(u), _dp(k), _lp(hidx), _dp(y), R, N, kd)
    return y


def op_fft(u, k, kind: str, hidx=None) -> np.ndarray:
    """Operator ``kind`` through the convolution theorem (2N zero padding
    for the causal kinds, size N for the circular ones; the adjoints use the
    conjugate kernel spectrum)."""
    kd = _kind(kind)
    u, k, hidx, R, N = _rows(u, k, hidx)
    if N & (N - 1):
        raise ValueError("op_fft needs a power-of-two N")
    y = np.empty((R, N), dtype=np.float64)
    if _load().oracle_op_fft(_dp(u), _dp(k), _lp(hidx), _dp(y), R,
                             k.shape[0], N, kd) != 0:
        raise MemoryError("oracle_op_fft: allocation failed")
    return y


def op_points(u, k, kind: str, rows, ts, hidx=None) -> np.ndarray:
    """out[i] = y[rows[i], ts[i]] of operator ``kind`` by the definition."""
    kd = _kind(kind)
    u, k, hidx, R, N = _rows(u, k, hidx)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    ts = np.ascontiguousarray(ts, dtype=np.int64)
    if rows.shape != ts.shape or rows.ndim != 1:
        raise ValueError("rows and ts must be 1-D of equal length")
    if len(rows) and (rows.min() < 0 or rows.max() >= R or ts.min() < 0
                      or ts.max() >= N):
        raise ValueError("sample index out of range")
    out = np.empty(len(rows), dtype=np.float64)
    _load().oracle_op_points(_dp(u), _dp(k), _lp(hidx), N, _lp(rows),
                             _lp(ts), len(rows), kd, _dp(out))
    return out


def _grad_rows(u, dy, Hk, hidx):
    u = np.ascontiguousarray(u, dtype=np.float64)
    dy = np.ascontiguousarray(dy, dtype=np.float64)
    if u.shape != dy.shape or u.ndim != 2:
        raise ValueError("u and dy must be [R, N] of the same shape")
    R, N = u.shape
    if hidx is None:
        hidx = np.arange(R) % Hk
    hidx = np.ascontiguousarray(hidx, dtype=np.int64)
    if hidx.shape != (R,) or (R and (hidx.min() < 0 or hidx.max() >= Hk)):
        raise ValueError("bad kernel row index")
    return u, dy, hidx, R, N


def kgrad_direct(u, dy, Hk: int, kind: str = "causal", hidx=None) -> np.ndarray:
    """Kernel gradient dk [Hk, N] of operator ``kind`` (its own kind or its
    adjoint give the same gradient of the forward kernel) by the
    definition: dk[h][j] = sum over rows r of channel h of
    sum_t dy[r][t] u[r][t-j]."""
    kd = _kind(kind)
    u, dy, hidx, R, N = _grad_rows(u, dy, Hk, hidx)
    dk = np.empty((Hk, N), dtype=np.float64)
    _load().oracle_kgrad_direct(_dp(u), _dp(dy), _lp(hidx), _dp(dk), R, Hk,
                                N, kd)
    return dk


def kgrad_fft(u, dy, Hk: int, kind: str = "causal", hidx=None) -> np.ndarray:
    """The kernel gradient through the convolution theorem:
    IFFT(sum_r conj(FFT u_r) . FFT dy_r)[0:N]."""
    kd = _kind(kind)
    u, dy, hidx, R, N = _grad_rows(u, dy, Hk, hidx)
    if N & (N - 1):
        raise ValueError("kgrad_fft needs a power-of-two N")
    dk = np.empty((Hk, N), dtype=np.float64)
    if _load().oracle_kgrad_fft(_dp(u), _dp(dy), _lp(hidx), _dp(dk), R, Hk,
                                N, kd) != 0:
        raise MemoryError("oracle_kgrad_fft: allocation failed")
    return dk


def kgrad_points(u, dy, Hk: int, hs, js, kind: str = "causal",
                 hidx=None) -> np.ndarray:
    """out[i] = dk[hs[i], js[i]] by the definition."""
    kd = _kind(kind)
    u, dy, hidx, R, N = _grad_rows(u, dy, Hk, hidx)
    hs = np.ascontiguousarray(hs, dtype=np.int64)
    js = np.ascontiguousarray(js, dtype=np.int64)
    if hs.shape != js.shape or hs.ndim != 1:
        raise ValueError("hs and js must be 1-D of equal length")
    out = np.empty(len(hs), dtype=np.float64)
    _load().oracle_kgrad_points(_dp(u), _dp(dy), _lp(hidx), R, N, _lp(hs),
                                _lp(js), len(hs), kd, _dp(out))
    return out


def lowpass_fft(u, k, F: int, hidx=None) -> np.ndarray:
    """Frequency-sparse causal convolution: IFFT_2N(U . K_F)[0:N] where the
    kernel spectrum keeps only frequencies f with min(f, 2N - f) <= F."""
    u, k, hidx, R, N = _rows(u, k, hidx)
    if N & (N - 1):
        raise ValueError("lowpass_fft needs a power-of-two N")
    if F < 0:
        raise ValueError("cutoff must be >= 0")
    y = np.empty((R, N), dtype=np.float64)
    if _load().oracle_lowpass_fft(_dp(u), _dp(k), _lp(hidx), _dp(y), R,
                                  k.shape[0], N, int(F)) != 0:
        raise MemoryError("oracle_lowpass_fft: allocation failed")
    return y


def masked_fft(u, k, mask, hidx=None) -> np.ndarray:
    """Causal convolution with a masked kernel spectrum:
    IFFT_2N(U . K . mask)[0:N], mask[f] in {0, 1} for f in [0, 2N)."""
    u, k, hidx, R, N = _rows(u, k, hidx)
    mask = np.ascontiguousarray(mask, dtype=np.float64)
    if mask.shape != (2 * N,):
        raise ValueError("mask needs 2N entries")
    if N & (N - 1):
        raise ValueError("masked_fft needs a power-of-two N")
    y = np.empty((R, N), dtype=np.float64)
    if _load().oracle_masked_fft(_dp(u), _dp(k), _lp(hidx), _dp(y), R,
                                 k.shape[0], N, _dp(mask)) != 0:
        raise MemoryError("oracle_masked_fft: allocation failed")
    return y


def blocksparse_mask(N: int, P: int, a: int, d: int) -> np.ndarray:
    """Kept (1) and zeroed (0) frequencies f in [0, 2N) of the frequency-
    sparse convolution whose zero blocks follow the digits of the transform
    (FlashFFTConv page, section 3.4, "Frequency-sparse convolutions": the
    kernel spectrum reshaped along the decomposition's factors, a whole
    number of rows zeroed along each one).  Reading taken here:

    * the 2N-point spectrum is used through N packed bins; frequencies f and
      f + N share the bin k = f mod N (the real-input packing), so the mask
      is a mask of bins;
    * a bin is written k = k_out + P k_in, k_out < P the outer digit of a
      P x (N / P) decomposition, and its top digit of 32 is
      k_b = floor(32 k_in P / N);
    * a: the a middle values of k_b are zeroed (16 - a/2 <= k_b < 16 + a/2;
      a even) -- the highest frequencies of every outer class;
    * d: the d outer classes nearest P/2 are zeroed (0 < |k_out - P/2| <=
      d // 2, and k_out = P/2 itself when d is odd);
    * a bin is also zeroed when its mirror bin -k mod N is, which keeps the
      spectrum Hermitian (the output real).
    """
    if N < 2 or N & (N - 1) or P < 1 or N % P:
        raise ValueError("bad N or P")
    if a < 0 or a > 32 or a % 2 or d < 0 or d >= max(P, 1) or (P == 1 and d):
        raise ValueError("bad a or d")
    k = np.arange(N)
    k_out = k % P
    k_in = k // P
    k_b = (k_in * 32 * P) // N
    zero_b = (k_b >= 16 - a // 2) & (k_b < 16 + a // 2)
    dist = np.abs(k_out - P / 2.0)
    zero_out = (dist > 0) & (dist <= d // 2)
    if d % 2:
        zero_out |= (k_out * 2 == P)
    z = zero_b | zero_out
    z = z | z[(-k) % N]
    return np.concatenate([~z, ~z]).astype(np.float64)


def blocksparse_fft(u, k, P: int, a: int, d: int, hidx=None) -> np.ndarray:
    """The frequency-sparse causal convolution of blocksparse_mask."""
    N = np.asarray(u).shape[-1]
    return masked_fft(u, k, blocksparse_mask(N, P, a, d), hidx)


def _gates(u, w, v):
    u = np.asarray(u, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if w.shape != u.shape or v.shape != u.shape:
        raise ValueError("gates must have the shape of u")
    return u, w, v


def gated_direct(u, w, v, k, hidx=None) -> np.ndarray:
    """y[r, t] = v[r, t] * sum_{s<=t} u[r, s] w[r, s] k[hidx[r], t-s]: the
    input gate multiplies u before the convolution, the output gate
    multiplies its result (fp64; the products of stored 16-bit values are
    exact in fp64)."""
    u, w, v = _gates(u, w, v)
    return v * conv_direct(u * w, k, hidx)


def gated_fft(u, w, v, k, hidx=None) -> np.ndarray:
    """The gated convolution with the convolution by the 2N-point FFT route."""
    u, w, v = _gates(u, w, v)
    return v * conv_fft(u * w, k, hidx)


def gated_points(u, w, v, k, rows, ts, hidx=None) -> np.ndarray:
    """out[i] = y[rows[i], ts[i]] of the gated convolution by the definition."""
    u, w, v = _gates(u, w, v)
    rows = np.asarray(rows, dtype=np.int64)
    ts = np.asarray(ts, dtype=np.int64)
    return v[rows, ts] * conv_points(u * w, k, rows, ts, hidx)


def fft(x, inverse: bool = False) -> np.ndarray:
    """Radix-2 DFT of a complex vector (power-of-two length).
    forward: X[k] = sum_j x[j] e^{-2 pi i jk/n}; inverse includes 1/n."""
    x = np.asarray(x, dtype=np.complex128)
    n = x.shape[0]
    if n < 1 or n & (n - 1):
        raise ValueError("fft needs a power-of-two length")
    re = np.ascontiguousarray(x.real, dtype=np.float64).copy()
    im = np.ascontiguousarray(x.imag, dtype=np.float64).copy()
    _load().oracle_fft(_dp(re), _dp(im), n, 1 if inverse else 0)
    return re + 1j * im


def kernel_spectrum(k) -> np.ndarray:
    """FFT_2N of each zero-padded kernel row: [Hk, 2N] complex."""
    k = np.ascontiguousarray(k, dtype=np.float64)
    Hk, N = k.shape
    kre = np.empty((Hk, 2 * N))
    kim = np.empty((Hk, 2 * N))
    _load().oracle_kernel_spectrum(_dp(k), Hk, N, _dp(kre), _dp(kim))
    return kre + 1j * kim


def rel_l2(y, y_ref) -> float:
    """||y - y_ref||_2 / ||y_ref||_2 in fp64."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    num = float(np.sum((y - y_ref) ** 2))
    den = float(np.sum(y_ref ** 2))
    return (num / den) ** 0.5 if den > 0 else (0.0 if num == 0 else float("inf"))
