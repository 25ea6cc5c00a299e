"""Rounding model of the register-resident row kernel (N = 1024, M = 1024
packed points, 32 x 32 Monarch stages) -- TEST INFRASTRUCTURE ONLY.

It replays the kernel's dataflow in numpy, with every rounding the kernel
performs placed where the kernel performs it, and nothing else:

* the packed row z[m] = u[2m] + i u[2m+1], m = 32 n_a + n_b (n_a < 16
  nonzero: the causal zero half);
* F1, the 32-point DFT over n_a on the matrix cores: 16-bit operands, exact
  products, fp32 accumulation.  For bf16 rows the DFT matrix is a hi/lo pair
  of bf16 values (two products per entry), for f16 rows one f16 value;
* the twiddle W_M^{k_a n_b}: the fp32 accumulators rounded to f16, then one
  packed-f16 complex product (a multiply and a fused multiply-add per half);
* F2, the 32-point DFT over n_b: f16 operands, fp32 accumulation, rounded to
  f16;
* the spectrum product with mirror pairing Z'[k] = alpha_k Z[k] +
  beta_k conj(Z[-k]): packed f16, alpha and beta stored as f16, one multiply
  and three fused multiply-adds per half;
* I2 (inverse over k_b) and its conjugate twiddle, I1 (inverse over k_a,
  only n_a < 16) as F2 and F1, the output rounded to the I/O type.

Every DFT stage is scaled to be unitary (1/sqrt(32) per stage), as in the
kernel's tables.  With ``exact=True`` no rounding happens and the model is
the real-FFT convolution of the page "FlashFFTConv: Efficient Convolutions
for Long Sequences with Tensor Cores" (section 3.4, the FFT convolution and
its real-valued FFT optimisation) evaluated in fp64: the tests pin that
against the oracle, so the rounded model differs from the exact result only
through the roundings listed above.

The model shares no code with the library or the oracle.  The matrix cores'
internal accumulation order is not modelled: products are summed in fp64
and the sum rounded once to fp32 (the fp32 accumulation error is far below
the f16 roundings that set the total).
"""
from __future__ import annotations

import numpy as np

M = 1024
R = 32


def _f16(x):
    """Round to f16, real and imaginary parts separately (fp64 in, fp64
    out)."""
    if np.iscomplexobj(x):
        return (x.real.astype(np.float16).astype(np.float64)
                + 1j * x.imag.astype(np.float16).astype(np.float64))
    return x.astype(np.float16).astype(np.float64)


def _f32(x):
    if np.iscomplexobj(x):
        return (x.real.astype(np.float32).astype(np.float64)
                + 1j * x.imag.astype(np.float32).astype(np.float64))
    return x.astype(np.float32).astype(np.float64)


def _bf16(x):
    """Round fp64 values to bf16 (nearest, ties to even) through fp32."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def _bf16c(x):
    return _bf16(x.real) + 1j * _bf16(x.imag)


def _dft(n, inverse=False):
    j = np.arange(n)
    sign = 1.0 if inverse else -1.0
    return np.exp(sign * 2j * np.pi * np.outer(j, j) / n) / np.sqrt(n)


def _fma16(a, b, c):
    """f16 fused multiply-add of f16 values: exact in fp64, one rounding."""
    return _f16(a * b + c)


def _hmul(d, t, conj=False):
    """The kernel's packed-f16 complex product d * t (d * conj(t) when
    conj): re = fma(-d.y, t.y, rnd(d.x t.x)), im = fma(d.x, t.y,
    rnd(d.y t.x)), with the signs of d's swapped halves flipped for the
    conjugate."""
    dx, dy, tx, ty = d.real, d.imag, t.real, t.imag
    if conj:
        re = _fma16(dy, ty, _f16(dx * tx))
        im = _fma16(-dx, ty, _f16(dy * tx))
    else:
        re = _fma16(-dy, ty, _f16(dx * tx))
        im = _fma16(dx, ty, _f16(dy * tx))
    return re + 1j * im


def _hpair(a, z, b, p):
    """a z + b conj(p) in packed f16: one multiply, three fused
    multiply-adds per half, in the kernel's order."""
    rx = _fma16(a.imag, -z.imag, _f16(a.real * z.real))
    ry = _fma16(a.imag, z.real, _f16(a.real * z.imag))
    rx = _fma16(b.real, p.real, rx)
    ry = _fma16(b.real, -p.imag, ry)
    rx = _fma16(b.imag, p.imag, rx)
    ry = _fma16(b.imag, p.real, ry)
    return rx + 1j * ry


def pair_coefficients(k64: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """alpha_k, beta_k (k = 0..M-1) of each kernel row such that the packed
    spectrum of the causal output is alpha_k Z[k] + beta_k conj(Z[-k]), Z
    the packed input's M-point DFT (unitary transforms both ways).

    From the real-FFT unpacking: with E = (Z[k] + conj Z[-k]) / 2 and
    O = (Z[k] - conj Z[-k]) / (2i) the spectra of the even and odd samples,
    w = exp(-2 pi i k / 2M) and K0 = K[k], K1 = K[k + M] the kernel's
    2M-point spectrum, the product spectrum is X[k] K0 at k and X[k+M] K1 at
    k + M with X = E +- w O; repacking the output's even/odd spectra gives
    Z'[k] = E A + O B with A = (K0 + K1)/2 + i (K0 - K1) / (2w) and
    B = w (K0 - K1)/2 + i (K0 + K1)/2, hence alpha = (A - iB)/2 and
    beta = (A + iB)/2."""
    kp = np.zeros((k64.shape[0], 2 * M))
    kp[:, :k64.shape[1]] = k64
    K = np.fft.fft(kp, axis=1)
    K0, K1 = K[:, :M], K[:, M:]
    w = np.exp(-2j * np.pi * np.arange(M) / (2 * M))
    A = (K0 + K1) / 2 + 1j * (K0 - K1) / (2 * w)
    B = w * (K0 - K1) / 2 + 1j * (K0 + K1) / 2
    return (A - 1j * B) / 2, (A + 1j * B) / 2


def row_kernel(u64: np.ndarray, k64: np.ndarray, hidx: np.ndarray, io: str,
               exact: bool = False) -> np.ndarray:
    """Causal outputs y[r, 0:1024] of rows u64 [rows, 1024] (the values
    stored in the I/O type, as fp64) with kernel rows k64 [H, 1024]; row r
    uses channel hidx[r].  io is 'bf16' or 'f16'.  exact=True drops every
    rounding."""
    assert u64.shape[1] == M and io in ("bf16", "f16")
    idn = (lambda x: x)
    r16 = idn if exact else _f16
    r32 = idn if exact else _f32
    rows = u64.shape[0]
    # packed row as [rows, n_a, n_b], n_a < 16 nonzero
    z = (u64[:, 0::2] + 1j * u64[:, 1::2]).reshape(rows, R // 2, R)
    F = _dft(R)
    Fi = _dft(R, inverse=True)
    ka = np.arange(R)
    tw = np.exp(-2j * np.pi * np.outer(np.arange(R), ka) / M)   # [n_b, k_a]
    if exact:
        F1, Fm, I1m, twq = F, F, Fi, tw
    else:
        if io == "bf16":
            hi = _bf16c(F)
            F1 = hi + _bf16c(F - hi)
        else:
            F1 = _f16(F)
        Fm, I1m, twq = _f16(F), _f16(Fi), _f16(tw)
    # F1 over n_a (rows of z beyond 16 are zero)
    c = r32(np.einsum("ran,ak->rnk", z, F1[:R // 2, :]))          # [r, n_b, k_a]
    c = r16(c)
    c = (c * twq[None]) if exact else _hmul(c, twq[None])
    # F2 over n_b: Z[k_a + 32 k_b] at [r, k_b, k_a]
    Z = r16(r32(np.einsum("bn,rnk->rbk", Fm, c)))
    # bins in natural order k = k_a + 32 k_b (kk: bin of position 32 k_a + k_b)
    kk = (ka[:, None] + R * np.arange(R)[None, :]).reshape(-1)
    Zk = np.empty((rows, M), dtype=np.complex128)
    Zk[:, kk] = Z.transpose(0, 2, 1).reshape(rows, M)
    al, be = pair_coefficients(k64)
    if not exact:
        al, be = _f16(al), _f16(be)
    al, be = al[hidx], be[hidx]
    Zneg = Zk[:, (-np.arange(M)) % M]                             # Z[-k]
    P = al * Zk + be * np.conj(Zneg) if exact else _hpair(al, Zk, be, Zneg)
    # back to [r, k_b, k_a]
    Pb = P[:, kk].reshape(rows, R, R).transpose(0, 2, 1)
    # I2 over k_b -> [r, n_b, k_a], then the conjugate twiddle
    d = r16(r32(np.einsum("nb,rbk->rnk", I1m, Pb)))
    d = (d * np.conj(twq)[None]) if exact else _hmul(d, twq[None], conj=True)
    # I1 over k_a, n_a < 16 -> [r, n_a, n_b]
    o = r32(np.einsum("ak,rnk->ran", I1m[:R // 2, :], d))
    out = o.reshape(rows, M // 2)
    y = np.empty((rows, 2 * (M // 2)))
    y[:, 0::2] = out.real
    y[:, 1::2] = out.imag
    if not exact:
        y = _bf16(y) if io == "bf16" else _f16(y)
    return y
