"""Pins for the fp64 CPU oracle (no GPU).

The oracle is checked against things it does not compute itself: values
worked by hand (tests/golden), closed forms, identities of the convolution
and of the DFT, brute force on tiny inputs, and numpy's independent FFT.
Each check is chosen so that a plausible slip in the oracle (a dropped term,
a wrong sign or index, a reversed kernel, a missing normalisation, wrap-around
from too little padding) fails at least one of them.
"""
import math

import numpy as np
import pytest

import oracle
from tests.conftest import golden_path


def _read_cases(name):
    cases, cur = [], {}
    with open(golden_path(name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("case"):
                if cur:
                    cases.append(cur)
                cur = {}
                continue
            key, vals = line.split(":", 1)
            cur[key.strip()] = vals.split()
    if cur:
        cases.append(cur)
    return cases


# ---------------------------------------------------------------- golden

def test_golden_hand_worked_convolutions():
    for case in _read_cases("causal_conv_hand.txt"):
        u = np.array([float(v) for v in case["u"]])[None, :]
        k = np.array([float(v) for v in case["k"]])[None, :]
        y = np.array([float(v) for v in case["y"]])
        np.testing.assert_array_equal(oracle.conv_direct(u, k)[0], y)
        n = u.shape[1]
        if n & (n - 1) == 0:
            np.testing.assert_allclose(oracle.conv_fft(u, k)[0], y,
                                       atol=1e-12)


def test_golden_hand_worked_dft():
    case = _read_cases("dft_hand.txt")[0]
    x = np.array([float(v) for v in case["x"]])
    X = np.array([complex(*map(float, p.split(","))) for p in case["X"]])
    np.testing.assert_allclose(oracle.fft(x), X, atol=1e-12)
    np.testing.assert_allclose(oracle.fft(X, inverse=True), x, atol=1e-12)


# ----------------------------------------------------------- brute force

def _brute(u, k):
    # direct double loop over all (t, s) pairs with the causal mask written
    # as an explicit index test (a different loop shape from the oracle's)
    n = len(u)
    y = [0.0] * n
    for s in range(n):
        for j in range(n):
            if s + j < n:
                y[s + j] += u[s] * k[j]
    return y


@pytest.mark.parametrize("n", [1, 2, 3, 5, 8])
def test_brute_force_tiny(n):
    rng = np.random.default_rng(n)
    u = rng.standard_normal((3, n))
    k = rng.standard_normal((2, n))
    hidx = np.array([1, 0, 1])
    yd = oracle.conv_direct(u, k, hidx)
    for r in range(3):
        np.testing.assert_allclose(yd[r], _brute(u[r], k[hidx[r]]),
                                   rtol=0, atol=1e-13)
    if n & (n - 1) == 0:
        np.testing.assert_allclose(oracle.conv_fft(u, k, hidx), yd,
                                   rtol=0, atol=1e-12)


def test_exhaustive_delta_basis_small():
    # every (input delta, kernel delta) pair for N <= 16: y = delta at s + d
    for n in (2, 4, 8, 16):
        eye = np.eye(n)
        for s in range(n):
            u = np.repeat(eye[s][None, :], n, axis=0)
            y_fft = oracle.conv_fft(u, eye, np.arange(n))
            y_dir = oracle.conv_direct(u, eye, np.arange(n))
            for d in range(n):
                want = np.zeros(n)
                if s + d < n:
                    want[s + d] = 1.0
                np.testing.assert_allclose(y_fft[d], want, atol=1e-12)
                np.testing.assert_array_equal(y_dir[d], want)


# --------------------------------------------------------------- identities

@pytest.mark.parametrize("n", [256, 1024])
def test_delta_identities(n):
    rng = np.random.default_rng(7)
    u = rng.standard_normal((2, n))
    kd = np.zeros((3, n))
    kd[0, 0] = 1.0                    # identity
    kd[1, 5] = 1.0                    # delay by 5
    kd[2, n - 1] = 1.0                # delay by n-1
    for conv in (oracle.conv_direct, oracle.conv_fft):
        y0 = conv(u, kd, [0, 0])
        np.testing.assert_allclose(y0, u, atol=1e-12)
        y5 = conv(u, kd, [1, 1])
        want = np.zeros_like(u)
        want[:, 5:] = u[:, :-5]
        np.testing.assert_allclose(y5, want, atol=1e-12)
        yl = conv(u, kd, [2, 2])
        want = np.zeros_like(u)
        want[:, n - 1] = u[:, 0]
        np.testing.assert_allclose(yl, want, atol=1e-12)
        # a delta input reproduces the kernel
        ud = np.zeros((1, n))
        ud[0, 0] = 1.0
        kk = rng.standard_normal((1, n))
        np.testing.assert_allclose(conv(ud, kk), kk, atol=1e-12)


def test_closed_form_geometric_kernel():
    # k[t] = r^t, u = 1  =>  y[t] = (1 - r^(t+1)) / (1 - r)
    n, r = 1024, 0.99
    t = np.arange(n)
    k = (r ** t)[None, :]
    u = np.ones((1, n))
    want = (1 - r ** (t + 1)) / (1 - r)
    for conv in (oracle.conv_direct, oracle.conv_fft):
        np.testing.assert_allclose(conv(u, k)[0], want, rtol=1e-12)


def test_closed_form_ramp():
    # u = 1, k = 1  =>  y[t] = t + 1 (counts the causal window)
    n = 512
    y = oracle.conv_fft(np.ones((1, n)), np.ones((1, n)))[0]
    np.testing.assert_allclose(y, np.arange(1, n + 1), rtol=1e-12)


def test_linearity():
    rng = np.random.default_rng(3)
    n = 512
    u1, u2 = rng.standard_normal((2, 1, n))
    k1, k2 = rng.standard_normal((2, 1, n))
    a, b = 1.75, -0.3
    for conv in (oracle.conv_direct, oracle.conv_fft):
        lhs = conv(a * u1 + b * u2, k1)
        rhs = a * conv(u1, k1) + b * conv(u2, k1)
        np.testing.assert_allclose(lhs, rhs, atol=1e-10)
        lhs = conv(u1, a * k1 + b * k2)
        rhs = a * conv(u1, k1) + b * conv(u1, k2)
        np.testing.assert_allclose(lhs, rhs, atol=1e-10)


def test_causality():
    # changing u[s] may only change y[t] for t >= s; with padding to 2N the
    # FFT route must not wrap the late inputs around onto early outputs
    rng = np.random.default_rng(11)
    n = 1024
    u = rng.standard_normal((1, n))
    k = rng.standard_normal((1, n))
    base = oracle.conv_fft(u, k)
    for s in (0, 1, 300, n - 1):
        u2 = u.copy()
        u2[0, s] += 10.0
        y2 = oracle.conv_fft(u2, k)
        np.testing.assert_allclose(y2[0, :s], base[0, :s], atol=1e-10)
        assert np.abs(y2[0, s:] - base[0, s:]).max() > 1.0


def test_commutes_in_u_and_k():
    rng = np.random.default_rng(12)
    n = 256
    u = rng.standard_normal((1, n))
    k = rng.standard_normal((1, n))
    np.testing.assert_allclose(oracle.conv_fft(u, k), oracle.conv_fft(k, u),
                               atol=1e-11)


# ---------------------------------------------------------------- the DFT

def _naive_dft(x):
    n = len(x)
    out = []
    for kk in range(n):
        acc = 0j
        for j in range(n):
            ang = -2.0 * math.pi * j * kk / n
            acc += x[j] * complex(math.cos(ang), math.sin(ang))
        out.append(acc)
    return np.array(out)


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64])
def test_fft_vs_naive_dft(n):
    rng = np.random.default_rng(n)
    x = rng.standard_normal(n) + 1j * rng.standard_normal(n)
    np.testing.assert_allclose(oracle.fft(x), _naive_dft(list(x)),
                               atol=1e-11 * max(1, n))


def test_fft_round_trip_parseval_hermitian():
    rng = np.random.default_rng(5)
    n = 4096
    x = rng.standard_normal(n)
    X = oracle.fft(x)
    np.testing.assert_allclose(oracle.fft(X, inverse=True).real, x,
                               atol=1e-12)
    # Parseval: sum |x|^2 = (1/n) sum |X|^2
    assert abs(np.sum(x ** 2) - np.sum(np.abs(X) ** 2) / n) < 1e-9 * n
    # Hermitian symmetry of a real input's spectrum
    np.testing.assert_allclose(X[1:], np.conj(X[1:][::-1]), atol=1e-10)


def test_fft_integer_bin_cosine():
    n, m = 256, 17
    j = np.arange(n)
    X = oracle.fft(np.cos(2 * np.pi * m * j / n))
    want = np.zeros(n, dtype=complex)
    want[m] = want[n - m] = n / 2
    np.testing.assert_allclose(X, want, atol=1e-9)


def test_fft_matches_numpy():
    rng = np.random.default_rng(9)
    for n in (2, 128, 2048, 65536):
        x = rng.standard_normal(n) + 1j * rng.standard_normal(n)
        np.testing.assert_allclose(oracle.fft(x), np.fft.fft(x),
                                   atol=1e-9 * np.sqrt(n))


# ------------------------------------------- the two routes agree, and numpy

@pytest.mark.parametrize("n", [2, 4, 16, 64, 256, 1024, 4096])
def test_fft_route_matches_definition(n):
    rng = np.random.default_rng(100 + n)
    u = rng.standard_normal((4, n))
    k = rng.standard_normal((3, n)) * np.exp(-0.01 * np.arange(n))
    hidx = np.array([0, 1, 2, 1])
    yd = oracle.conv_direct(u, k, hidx)
    yf = oracle.conv_fft(u, k, hidx)
    assert oracle.rel_l2(yf, yd) < 1e-12


def test_fft_route_matches_numpy_rfft():
    rng = np.random.default_rng(21)
    n = 8192
    u = rng.standard_normal((2, n))
    k = rng.standard_normal((2, n))
    L = 2 * n
    want = np.fft.irfft(np.fft.rfft(u, L) * np.fft.rfft(k, L), L)[:, :n]
    assert oracle.rel_l2(oracle.conv_fft(u, k), want) < 1e-12


def test_kernel_spectrum_matches_numpy():
    rng = np.random.default_rng(22)
    k = rng.standard_normal((3, 512))
    want = np.fft.fft(np.concatenate([k, np.zeros_like(k)], axis=1), axis=1)
    np.testing.assert_allclose(oracle.kernel_spectrum(k), want, atol=1e-9)


def test_points_match_full():
    rng = np.random.default_rng(23)
    n = 2048
    u = rng.standard_normal((5, n))
    k = rng.standard_normal((2, n))
    hidx = np.array([0, 1, 0, 1, 1])
    y = oracle.conv_direct(u, k, hidx)
    rows = np.array([0, 4, 2, 3, 1, 1])
    ts = np.array([0, n - 1, 1000, 7, 0, 2047])
    np.testing.assert_array_equal(oracle.conv_points(u, k, rows, ts, hidx),
                                  y[rows, ts])


def test_rel_l2():
    a = np.array([3.0, 4.0])
    assert oracle.rel_l2(a, a) == 0.0
    assert abs(oracle.rel_l2(a * 1.01, a) - 0.01) < 1e-12


def test_exact_widening_of_stored_dtypes():
    bits = np.array([0x3F80, 0xC000, 0x3E20, 0x0001], dtype=np.uint16)
    np.testing.assert_array_equal(oracle.to_f64(bits, "bf16"),
                                  [1.0, -2.0, 0.15625, 2.0 ** -133])
    h = np.array([1.0, 0.5, -65504.0], dtype=np.float16)
    np.testing.assert_array_equal(oracle.to_f64(h, "f16"), h.astype(float))


# ----------------------------------------------------------------- gated

def test_golden_hand_worked_gated():
    for case in _read_cases("gated_conv_hand.txt"):
        u, w, v, k = (np.array([float(x) for x in case[key]])[None, :]
                      for key in ("u", "w", "v", "k"))
        y = np.array([float(x) for x in case["y"]])
        np.testing.assert_array_equal(oracle.gated_direct(u, w, v, k)[0], y)


def _brute_gated(u, w, v, k):
    # explicit triple product per (t, s) pair, gates applied term by term
    n = len(u)
    y = [0.0] * n
    for t in range(n):
        acc = 0.0
        for s in range(t + 1):
            acc += u[s] * w[s] * k[t - s]
        y[t] = v[t] * acc
    return y


@pytest.mark.parametrize("n", [1, 2, 4, 7, 8])
def test_gated_brute_force_tiny(n):
    rng = np.random.default_rng(100 + n)
    u, w, v = (rng.standard_normal((3, n)) for _ in range(3))
    k = rng.standard_normal((2, n))
    hidx = np.array([0, 1, 1])
    yd = oracle.gated_direct(u, w, v, k, hidx)
    for r in range(3):
        np.testing.assert_allclose(yd[r], _brute_gated(u[r], w[r], v[r], k[hidx[r]]),
                                   rtol=0, atol=1e-13)
    if n & (n - 1) == 0:
        np.testing.assert_allclose(oracle.gated_fft(u, w, v, k, hidx), yd,
                                   rtol=0, atol=1e-12)


def test_gated_special_cases():
    rng = np.random.default_rng(7)
    u = rng.standard_normal((2, 16))
    k = rng.standard_normal((2, 16))
    one = np.ones_like(u)
    # unit gates: the plain convolution
    np.testing.assert_array_equal(oracle.gated_direct(u, one, one, k),
                                  oracle.conv_direct(u, k))
    # a zero output gate zeroes the output; a zero input gate zeroes it too
    assert not oracle.gated_direct(u, one, np.zeros_like(u), k).any()
    assert not oracle.gated_direct(u, np.zeros_like(u), one, k).any()
    # constant gates scale: w = a, v = b gives a * b * (u * k)
    a, b = 0.75, -2.0
    np.testing.assert_allclose(oracle.gated_direct(u, a * one, b * one, k),
                               a * b * oracle.conv_direct(u, k), rtol=1e-14)
    # the input gate acts before the convolution: gating u by a delta at s0
    # keeps only u[s0] k[t - s0] (t >= s0)
    s0 = 5
    wd = np.zeros_like(u)
    wd[:, s0] = 1.0
    yd = oracle.gated_direct(u, wd, one, k)
    for r in range(2):
        want = np.zeros(16)
        want[s0:] = u[r, s0] * k[r, :16 - s0]
        np.testing.assert_allclose(yd[r], want, atol=1e-14)


def test_gated_points_match_full():
    rng = np.random.default_rng(11)
    u, w, v = (rng.standard_normal((4, 32)) for _ in range(3))
    k = rng.standard_normal((2, 32))
    full = oracle.gated_direct(u, w, v, k)
    rows = np.array([0, 3, 2, 1, 3])
    ts = np.array([0, 31, 7, 16, 1])
    np.testing.assert_allclose(oracle.gated_points(u, w, v, k, rows, ts),
                               full[rows, ts], rtol=0, atol=1e-12)


# ------------------------------------------- circular, adjoints, gradients

def test_golden_hand_worked_operators():
    (case,) = _read_cases("ops_hand.txt")
    f = lambda key: np.array([float(x) for x in case[key]])[None, :]
    u, k, dy = f("u"), f("k"), f("dy")
    for kind in ("circular", "causal_adjoint", "circular_adjoint"):
        np.testing.assert_array_equal(oracle.op_direct(u, k, kind), f(kind))
        np.testing.assert_allclose(oracle.op_fft(u, k, kind), f(kind),
                                   atol=1e-14)
    np.testing.assert_array_equal(oracle.kgrad_direct(u, dy, 1, "causal"),
                                  f("kgrad_causal"))
    np.testing.assert_array_equal(oracle.kgrad_direct(u, dy, 1, "circular"),
                                  f("kgrad_circular"))
    np.testing.assert_allclose(oracle.kgrad_fft(u, dy, 1, "causal"),
                               f("kgrad_causal"), atol=1e-14)
    np.testing.assert_allclose(oracle.kgrad_fft(u, dy, 1, "circular"),
                               f("kgrad_circular"), atol=1e-14)


def _brute_op(u, k, kind):
    # the definitions with the sum index running over the kernel taps
    n = len(u)
    y = [0.0] * n
    for a in range(n):
        for j in range(n):
            if kind == "circular":
                y[a] += k[j] * u[(a - j) % n]
            elif kind == "circular_adjoint":
                y[a] += k[j] * u[(a + j) % n]
            elif kind == "causal_adjoint":
                if a + j < n:
                    y[a] += k[j] * u[a + j]
            else:
                if a - j >= 0:
                    y[a] += k[j] * u[a - j]
    return y


@pytest.mark.parametrize("kind", list(oracle.KINDS))
@pytest.mark.parametrize("n", [1, 2, 4, 8])
def test_operators_brute_force_and_fft(kind, n):
    rng = np.random.default_rng(300 + n)
    u = rng.standard_normal((3, n))
    k = rng.standard_normal((2, n))
    hidx = np.array([1, 0, 1])
    yd = oracle.op_direct(u, k, kind, hidx)
    for r in range(3):
        np.testing.assert_allclose(yd[r], _brute_op(u[r], k[hidx[r]], kind),
                                   atol=1e-13)
    np.testing.assert_allclose(oracle.op_fft(u, k, kind, hidx), yd,
                               atol=1e-12)
    rows = np.array([0, 2, 1, 2])
    ts = np.array([0, n - 1, n // 2, 0])
    np.testing.assert_allclose(oracle.op_points(u, k, kind, rows, ts, hidx),
                               yd[rows, ts], atol=1e-13)


def test_adjoint_identities():
    # <A u, y> = <u, A^T y> for the causal and the circular operator
    rng = np.random.default_rng(17)
    N = 64
    u, y = rng.standard_normal((2, 5, N))
    k = rng.standard_normal((5, N))
    for kind in ("causal", "circular"):
        lhs = np.sum(oracle.op_fft(u, k, kind) * y)
        rhs = np.sum(u * oracle.op_fft(y, k, kind + "_adjoint"))
        assert abs(lhs - rhs) < 1e-10 * (abs(lhs) + 1)


def test_circular_special_cases():
    rng = np.random.default_rng(23)
    N = 32
    u = rng.standard_normal((2, N))
    # a delta kernel at m is a circular shift by m
    for m in (0, 1, 7, N - 1):
        d = np.zeros((1, N))
        d[0, m] = 1.0
        np.testing.assert_allclose(oracle.op_fft(u, d, "circular", [0, 0]),
                                   np.roll(u, m, axis=1), atol=1e-13)
    # with u and k both confined to the first half there is no wrap-around:
    # the circular result is the causal one
    uh = u.copy()
    uh[:, N // 2:] = 0.0
    kh = rng.standard_normal((1, N))
    kh[:, N // 2:] = 0.0
    np.testing.assert_allclose(oracle.op_direct(uh, kh, "circular", [0, 0]),
                               oracle.conv_direct(uh, kh, [0, 0]), atol=1e-13)
    # a constant kernel sums the whole row into every output
    c = np.full((1, N), 0.5)
    y = oracle.op_direct(u, c, "circular", [0, 0])
    np.testing.assert_allclose(y, 0.5 * u.sum(axis=1, keepdims=True) *
                               np.ones((1, N)), atol=1e-12)


def test_circular_against_numpy_fft():
    rng = np.random.default_rng(29)
    N = 128
    u = rng.standard_normal((3, N))
    k = rng.standard_normal((3, N))
    want = np.fft.irfft(np.fft.rfft(u) * np.fft.rfft(k), n=N)
    np.testing.assert_allclose(oracle.op_fft(u, k, "circular"), want,
                               atol=1e-12)
    want = np.fft.irfft(np.fft.rfft(u) * np.conj(np.fft.rfft(k)), n=N)
    np.testing.assert_allclose(oracle.op_fft(u, k, "circular_adjoint"), want,
                               atol=1e-12)


def test_kernel_gradient_is_the_derivative():
    # L(k) = <dy, A_k u> is linear in k, so dL/dk[j] = L(e_j) exactly;
    # L(e_j) goes through the operator's definition, not the gradient code
    rng = np.random.default_rng(31)
    N, B, H = 16, 3, 2
    u = rng.standard_normal((B * H, N))
    dy = rng.standard_normal((B * H, N))
    for kind in ("causal", "circular"):
        dk = oracle.kgrad_direct(u, dy, H, kind)
        for h in range(H):
            for j in range(N):
                e = np.zeros((H, N))
                e[h, j] = 1.0
                want = np.sum(dy * oracle.op_direct(u, e, kind))
                assert abs(dk[h, j] - want) < 1e-12
        np.testing.assert_allclose(oracle.kgrad_fft(u, dy, H, kind), dk,
                                   atol=1e-12)
        hs = np.array([0, 1, 1, 0])
        js = np.array([0, N - 1, 3, 9])
        np.testing.assert_allclose(oracle.kgrad_points(u, dy, H, hs, js, kind),
                                   dk[hs, js], atol=1e-12)


def test_kernel_gradient_against_numpy_fft():
    rng = np.random.default_rng(37)
    N, B, H = 64, 4, 3
    u = rng.standard_normal((B * H, N))
    dy = rng.standard_normal((B * H, N))
    hidx = np.arange(B * H) % H
    for kind, L in (("causal", 2 * N), ("circular", N)):
        g = np.conj(np.fft.fft(u, n=L)) * np.fft.fft(dy, n=L)
        want = np.stack([np.fft.ifft(g[hidx == h].sum(axis=0)).real[:N]
                         for h in range(H)])
        np.testing.assert_allclose(oracle.kgrad_fft(u, dy, H, kind), want,
                                   atol=1e-11)


# ------------------------------------------------- frequency-sparse (low-pass)

def _dirichlet_kernel(c, F):
    # the 2N-periodic kernel whose spectrum is that of c band-limited to
    # |f| <= F, by circular convolution with the Dirichlet kernel
    # D_F[j] = sin(pi (2F+1) j / L) / (L sin(pi j / L)), D_F[0] = (2F+1)/L
    L = len(c)
    j = np.arange(L)
    D = np.empty(L)
    D[0] = (2 * F + 1) / L
    jj = j[1:]
    D[1:] = np.sin(np.pi * (2 * F + 1) * jj / L) / (L * np.sin(np.pi * jj / L))
    out = np.zeros(L)
    for n in range(L):
        out[n] = sum(c[m] * D[(n - m) % L] for m in range(L))
    return out


@pytest.mark.parametrize("N,F", [(8, 2), (16, 5), (16, 0), (32, 11)])
def test_lowpass_time_domain(N, F):
    # independent route: band-limit the padded kernel in time (Dirichlet),
    # then the 2N-point circular convolution by its definition
    rng = np.random.default_rng(400 + N + F)
    u = rng.standard_normal((2, N))
    k = rng.standard_normal((2, N))
    L = 2 * N
    want = np.zeros((2, N))
    for r in range(2):
        c = _dirichlet_kernel(np.concatenate([k[r], np.zeros(N)]), F)
        up = np.concatenate([u[r], np.zeros(N)])
        for t in range(N):
            want[r, t] = sum(up[s] * c[(t - s) % L] for s in range(L))
    np.testing.assert_allclose(oracle.lowpass_fft(u, k, F), want, atol=1e-12)


def test_lowpass_special_cases():
    rng = np.random.default_rng(41)
    N = 64
    u = rng.standard_normal((3, N))
    k = rng.standard_normal((3, N))
    # no band limit: the causal convolution
    np.testing.assert_allclose(oracle.lowpass_fft(u, k, N), oracle.conv_direct(u, k),
                               atol=1e-12)
    # DC only: every output is sum(u) sum(k) / 2N
    y0 = oracle.lowpass_fft(u, k, 0)
    want = (u.sum(axis=1) * k.sum(axis=1) / (2 * N))[:, None] * np.ones((1, N))
    np.testing.assert_allclose(y0, want, atol=1e-12)
    # against numpy: the same band limit applied to numpy's spectra
    L = 2 * N
    f = np.arange(L)
    mask = np.minimum(f, L - f) <= 9
    want = np.fft.ifft(np.fft.fft(u, n=L) * np.fft.fft(k, n=L) * mask).real[:, :N]
    np.testing.assert_allclose(oracle.lowpass_fft(u, k, 9), want, atol=1e-12)


# ---- frequency-sparse convolution with zero blocks along the digits

def _blocksparse_cases():
    out = []
    for line in open(golden_path("blocksparse_mask_hand.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        head, _, kept = line.partition(":")
        N, P, a, d = (int(x) for x in head.split())
        out.append((N, P, a, d, [int(x) for x in kept.split()]))
    return out


def test_blocksparse_mask_hand_worked():
    cases = _blocksparse_cases()
    assert len(cases) == 5
    for N, P, a, d, kept in cases:
        m = oracle.blocksparse_mask(N, P, a, d)
        assert m.shape == (2 * N,)
        assert sorted(np.flatnonzero(m).tolist()) == kept, (N, P, a, d)


@pytest.mark.parametrize("N,P", [(1024, 1), (8192, 8), (32768, 32), (65536, 16)])
def test_blocksparse_mask_structure(N, P):
    # Hermitian (f and 2N - f kept together), bins f and f + N together,
    # and the zeroed fraction of the digit sets plus only the mirror closure
    for a in (0, 8, 16, 24):
        for d in ((0, 1, 2, P // 2, P - 2) if P > 2 else (0,)):
            m = oracle.blocksparse_mask(N, P, a, d)
            f = np.arange(2 * N)
            assert np.array_equal(m, m[(2 * N - f) % (2 * N)])
            assert np.array_equal(m[:N], m[N:])
            kept = m[:N].mean()
            want = (32 - a) / 32.0 * (P - d) / P
            # the mirror closure only adds zeros in outer class 0 (at most
            # the bins of its k_a = 0 column: N / (32 P) of N)
            assert want - 1.0 / (32 * P) - 1e-12 <= kept <= want + 1e-12


def test_blocksparse_special_cases():
    rng = np.random.default_rng(3)
    N, P = 512, 4
    u = rng.standard_normal((3, N))
    k = rng.standard_normal((2, N)) * np.exp(-0.01 * np.arange(N))
    hidx = np.array([0, 1, 1])
    # no zero blocks: the causal convolution
    np.testing.assert_allclose(oracle.blocksparse_fft(u, k, P, 0, 0, hidx),
                               oracle.conv_direct(u, k, hidx), rtol=0, atol=1e-10)
    # every bin zero: no output
    assert np.max(np.abs(oracle.blocksparse_fft(u, k, P, 32, 0, hidx))) < 1e-12
    # the masked route with the band-limit mask is the band-limited route
    F = 100
    f = np.arange(2 * N)
    band = (np.minimum(f, 2 * N - f) <= F).astype(np.float64)
    np.testing.assert_allclose(oracle.masked_fft(u, k, band, hidx),
                               oracle.lowpass_fft(u, k, F, hidx), rtol=0, atol=1e-10)
    # numpy's FFT with the same mask (an independent transform)
    for a, d in ((16, 0), (8, 1), (0, 2), (24, 3)):
        m = oracle.blocksparse_mask(N, P, a, d)
        U = np.fft.fft(u, 2 * N)
        K = np.fft.fft(k, 2 * N)
        want = np.fft.ifft(U * K[hidx] * m)[:, :N]
        assert np.max(np.abs(want.imag)) < 1e-9     # the mask keeps it real
        np.testing.assert_allclose(oracle.blocksparse_fft(u, k, P, a, d, hidx),
                                   want.real, rtol=0, atol=1e-9)


def test_blocksparse_mask_rejects_bad_counts():
    for args in ((1024, 1, 0, 1), (1024, 4, 3, 0), (1024, 4, 34, 0), (1000, 4, 0, 0),
                 (1024, 4, 0, 4)):
        with pytest.raises(ValueError):
            oracle.blocksparse_mask(*args)
