// Fused kernel for rows of N = P * 1024 (P = 4, 8, 16) with 16-bit I/O: one
// workgroup of P/2 wavefronts per row, the whole 2N-point transform held in
// LDS and registers (page "FlashFFTConv: Efficient Convolutions for Long
// Sequences with Tensor Cores", section 3.4 and Algorithm 1: an order-3
// Monarch decomposition P x 32 x 32, with the real-input packing and the
// implicit zero padding of section 3.3).
//
// Packed row z[n], n = n1*Q + n' (Q = 1024, n1 < P/2 nonzero), bins
// k = k1 + P*k', k' = k_a + 32*k_b (the 32 x 32 engine of the row kernel).
//
//  1. Outer stage (all threads, vector ALU, packed f16): for every column n'
//     A_k1[n'] = sum_{n1 < P/2} W_P^{n1 k1} z[n1 Q + n'], then the twiddle
//     w_k1[n'] = W_M^{n' k1}.  Results go to LDS, one region per sub-row.
//  2. Engine (one wavefront per pair of sub-rows, matrix cores): the
//     1024-point DFT of each sub-row (32-point stage, twiddle, 32-point
//     stage), the spectrum product, and the inverse 1024-point DFT.
//  3. Outer inverse (all threads): conjugate twiddle and the P-point
//     inverse DFT, only the n1 < P/2 outputs (t < N), store.
//
// Mirror pairing.  Bin k pairs with -k.  For 0 < k1 < P/2 the partner bins
// live in sub-row P - k1.  That sub-row is pushed through the engine as
// w_k1 * conj(A_{P-k1}) -- the same twiddle as sub-row k1 -- which returns
// conj(Z[-k]) in exactly the register that holds Z[k]: the spectrum product
// of a pair becomes element-wise, and the partner's inverse result is the
// conjugate of the engine output.  Sub-row 0 pairs within itself by
// negation (as in the row kernel) and sub-row P/2 by reversal
// k' <-> 1023 - k', whose partner sits one lane over (a DPP rotation).
#include "fftconv_mfma.h"

#include <type_traits>

namespace fftconv {

namespace {

// cos(2 pi k / 32) for k = 0..8, then by symmetry
__host__ __device__ constexpr float c32q(int k) {
    return k == 0 ? 1.0f : k == 1 ? 0.98078528040323044f : k == 2 ? 0.92387953251128674f
         : k == 3 ? 0.83146961230254524f : k == 4 ? 0.70710678118654752f
         : k == 5 ? 0.55557023301960222f : k == 6 ? 0.38268343236508977f
         : k == 7 ? 0.19509032201612827f : 0.0f;
}
__host__ __device__ constexpr float cos32(int k) {
    k &= 31;
    return k <= 8 ? c32q(k) : k <= 16 ? -c32q(16 - k) : k <= 24 ? -c32q(k - 16) : c32q(32 - k);
}
// W_32^k = exp(-2 pi i k / 32)
__host__ __device__ constexpr float w32re(int k) { return cos32(k); }
__host__ __device__ constexpr float w32im(int k) { return -cos32(k - 8); }

typedef float rfloat2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ rhalf2 h2c(float re, float im) {
    rhalf2 r;
    r.x = (_Float16)re;
    r.y = (_Float16)im;
    return r;
}
// Complex helpers for the outer stages, over packed f16 (rhalf2) or fp32
// (rfloat2) pairs (re, im).
template <class V>
__device__ __forceinline__ V cnj(V a) {
    const V r = {a.x, -a.y};
    return r;
}
// -i * a
template <class V>
__device__ __forceinline__ V mul_mi(V a) {
    const V r = {a.y, -a.x};
    return r;
}
__device__ __forceinline__ rfloat2 fmul(rfloat2 d, rfloat2 t) {
    const rfloat2 r = {d.x * t.x - d.y * t.y, d.x * t.y + d.y * t.x};
    return r;
}
__device__ __forceinline__ rfloat2 fmulc(rfloat2 d, rfloat2 t) {
    const rfloat2 r = {d.x * t.x + d.y * t.y, d.y * t.x - d.x * t.y};
    return r;
}
// a * W_32^k for a compile-time k (trivial factors cost nothing)
template <int K, class V>
__device__ __forceinline__ V mulw(V a) {
    constexpr int k = K & 31;
    if constexpr (k == 0) return a;
    else if constexpr (k == 8) return mul_mi(a);
    else if constexpr (k == 16) return -a;
    else if constexpr (k == 24) return -mul_mi(a);
    else if constexpr (sizeof(V) == 4) return hmul(a, h2c(w32re(k), w32im(k)));
    else {
        const rfloat2 w = {w32re(k), w32im(k)};
        return fmul(a, w);
    }
}
// a*z + b*p (swizzles on the data, as in hpair)
__device__ __forceinline__ rhalf2 hcmla(rhalf2 a, rhalf2 z, rhalf2 b, rhalf2 p) {
    const rhalf2 axx = {a.x, a.x}, ayy = {a.y, a.y};
    const rhalf2 bxx = {b.x, b.x}, byy = {b.y, b.y};
    const rhalf2 zn = {-z.y, z.x}, pn = {-p.y, p.x};
    rhalf2 r = __builtin_elementwise_fma(ayy, zn, axx * z);
    r = __builtin_elementwise_fma(bxx, p, r);
    return __builtin_elementwise_fma(byy, pn, r);
}

// a * W_32^k for k known after unrolling
template <class V>
__device__ __forceinline__ V mulw_k(V a, int k) {
    switch (k & 31) {
#define FFTCONV_W(K) case K: return mulw<K>(a);
        FFTCONV_W(0) FFTCONV_W(1) FFTCONV_W(2) FFTCONV_W(3) FFTCONV_W(4) FFTCONV_W(5)
        FFTCONV_W(6) FFTCONV_W(7) FFTCONV_W(8) FFTCONV_W(9) FFTCONV_W(10) FFTCONV_W(11)
        FFTCONV_W(12) FFTCONV_W(13) FFTCONV_W(14) FFTCONV_W(15) FFTCONV_W(16) FFTCONV_W(17)
        FFTCONV_W(18) FFTCONV_W(19) FFTCONV_W(20) FFTCONV_W(21) FFTCONV_W(22) FFTCONV_W(23)
        FFTCONV_W(24) FFTCONV_W(25) FFTCONV_W(26) FFTCONV_W(27) FFTCONV_W(28) FFTCONV_W(29)
        FFTCONV_W(30) FFTCONV_W(31)
#undef FFTCONV_W
    }
    return a;
}

// In-place n-point DFT (n = 1, 2, 4, 8), natural order in and out; INV
// uses W^-1.
template <int n, bool INV, class V>
__device__ __forceinline__ void dft_small(V (&v)[n]) {
    if constexpr (n == 2) {
        const V a = v[0] + v[1], b = v[0] - v[1];
        v[0] = a;
        v[1] = b;
    } else if constexpr (n == 4) {
        const V t0 = v[0] + v[2], t1 = v[0] - v[2], t2 = v[1] + v[3];
        V t3 = v[1] - v[3];
        t3 = INV ? -mul_mi(t3) : mul_mi(t3);   // W_4^{+-1}
        v[0] = t0 + t2;
        v[2] = t0 - t2;
        v[1] = t1 + t3;
        v[3] = t1 - t3;
    } else if constexpr (n == 8) {
        V e[4] = {v[0], v[2], v[4], v[6]}, o[4] = {v[1], v[3], v[5], v[7]};
        dft_small<4, INV>(e);
        dft_small<4, INV>(o);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const V t = mulw_k(o[k], INV ? -4 * k : 4 * k);   // W_8^{+-k}
            v[k] = e[k] + t;
            v[k + 4] = e[k] - t;
        }
    }
}

// A[k] = sum_{m < P/2} W_P^{m k} x[m], k < P (the other P/2 inputs are zero)
template <int P, class V>
__device__ __forceinline__ void dft_half_in(const V (&x)[P / 2], V (&A)[P]) {
    V e[P / 2], o[P / 2];
#pragma unroll
    for (int m = 0; m < P / 2; ++m) {
        e[m] = x[m];
        o[m] = mulw_k(x[m], m * (32 / P));   // odd outputs see x[m] W_P^m
    }
    dft_small<P / 2, false>(e);
    dft_small<P / 2, false>(o);
#pragma unroll
    for (int j = 0; j < P / 2; ++j) {
        A[2 * j] = e[j];
        A[2 * j + 1] = o[j];
    }
}

// z[m] = sum_k W_P^{-m k} B[k] for m < P/2 only
template <int P, class V>
__device__ __forceinline__ void idft_half_out(const V (&B)[P], V (&z)[P / 2]) {
    V e[P / 2], o[P / 2];
#pragma unroll
    for (int j = 0; j < P / 2; ++j) {
        e[j] = B[2 * j];
        o[j] = B[2 * j + 1];
    }
    dft_small<P / 2, true>(e);
    dft_small<P / 2, true>(o);
#pragma unroll
    for (int m = 0; m < P / 2; ++m) z[m] = e[m] + mulw_k(o[m], -m * (32 / P));
}

// Outer-stage arithmetic: packed f16 for f16 I/O; fp32 for bf16 I/O, whose
// output rounding (2^-9) leaves little room for extra f16 roundings.
template <int IO>
struct Outer {
    typedef typename std::conditional<IO == IO_BF16, rfloat2, rhalf2>::type V;
    static __device__ __forceinline__ V from_io(uint32_t v) {
        if constexpr (IO == IO_BF16) {
            const rfloat2 r = {__uint_as_float(v << 16), __uint_as_float(v & 0xffff0000u)};
            return r;
        } else {
            return as_h2(v);
        }
    }
    static __device__ __forceinline__ V from_h2(uint32_t v) {
        if constexpr (IO == IO_BF16) {
            const rhalf2 h = as_h2(v);
            const rfloat2 r = {(float)h.x, (float)h.y};
            return r;
        } else {
            return as_h2(v);
        }
    }
    static __device__ __forceinline__ uint32_t to_h2(V a) {
        if constexpr (IO == IO_BF16) return pk2(a.x, a.y);
        else return as_u32(a);
    }
    static __device__ __forceinline__ uint32_t to_io(V a) {
        if constexpr (IO == IO_BF16) return pk2io<IO_BF16>(a.x, a.y);
        else return as_u32(a);
    }
    // a * t and a * conj(t), t a packed-f16 twiddle
    static __device__ __forceinline__ V mul(V a, uint32_t t) {
        if constexpr (IO == IO_BF16) {
            const rhalf2 h = as_h2(t);
            const rfloat2 w = {(float)h.x, (float)h.y};
            return fmul(a, w);
        } else {
            return hmul(a, as_h2(t));
        }
    }
    static __device__ __forceinline__ V mulc(V a, uint32_t t) {
        if constexpr (IO == IO_BF16) {
            const rhalf2 h = as_h2(t);
            const rfloat2 w = {(float)h.x, (float)h.y};
            return fmulc(a, w);
        } else {
            return hmulc(a, as_h2(t));
        }
    }
};

// DPP row rotation: lane x of every 16-lane row reads lane (x + 1) mod 16
// (UP) or lane (x - 1) mod 16 (DOWN).
__device__ __forceinline__ uint32_t rot_up(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x12F, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t rot_down(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x121, 0xF, 0xF, false);
}

}  // namespace

// LDS word address of (n_a, n_b) within a sub-row region: the engine reads
// uint4 (it*2 + ks)*64 + lane holding n_a = 16 ks + 4 g + 0..3 and
// n_b = kmap32(it, x).
__device__ __forceinline__ int eng_addr(int na, int it, int x) {
    return (((it * 2 + (na >> 4)) * 64 + 16 * ((na >> 2) & 3) + x) << 2) + (na & 3);
}

template <int IO, int P>
__global__ void __launch_bounds__(32 * P, 2) wide_kernel(WideParams prm) {
    constexpr int Q = 1024, M = P * Q, HALF = P / 2, T = 32 * P;
    constexpr int CPT = Q / T;   // outer-stage columns per thread

    extern __shared__ uint4 s_lds[];
    uint4* s_f1b = s_lds;                              // [ks 2][jt 4][64]
    uint4* s_i1a = s_f1b + 8 * 64;                     // [mt 4][ks 2][64]
    uint32_t* s_two = (uint32_t*)(s_i1a + 8 * 64);     // [k1 - 1][thread][column]
    uint32_t* s_buf = s_two + HALF * Q;                // [P sub-rows][Q]
    uint32_t* s_scr = s_buf + M;                       // [39 k_b slots][16 x]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, x = lane & 15;
    const int total = prm.B * prm.H;
    // Rows are taken in channel-major order (index h * B + b).  At step t
    // the grid covers indices [t G, (t + 1) G), and the G / 8 workgroups
    // that share an XCD (consecutive dispatch ids go to consecutive XCDs)
    // take a contiguous block of them: the few channels in flight on an XCD
    // at a time keep their spectrum coefficients in that XCD's L2.
    const int G = gridDim.x;
    const int first = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
    if (first >= total) return;   // uniform over the workgroup

    for (int i = tid; i < 8 * 64; i += T) {
        s_f1b[i] = ((const uint4*)prm.f1b)[i];
        s_i1a[i] = ((const uint4*)prm.i1a)[i];
    }
    for (int i = tid; i < HALF * Q / 4; i += T) ((uint4*)s_two)[i] = ((const uint4*)prm.two)[i];
    uint4 f2a[4][2], i2b[2][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) f2a[mt][ks] = ((const uint4*)prm.f2a)[(mt * 2 + ks) * 64 + lane];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) i2b[ks][jt] = ((const uint4*)prm.i2b)[(ks * 4 + jt) * 64 + lane];
    uint32_t twf[2][2][4];
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) twf[it][kt][r] = prm.twf[lane * 16 + (it * 2 + kt) * 4 + r];

    // ---- outer-stage geometry: n_b = tid & 31, n_a = na0 + j (j < CPT)
    const int nb = tid & 31, na0 = CPT * (tid >> 5);
    const int it_o = nb < 16 ? 0 : 1, x_o = nb < 16 ? nb : (nb == 16 ? 0 : 32 - nb);
    const int oa0 = eng_addr(na0, it_o, x_o);   // consecutive words for j < min(CPT, 4)
    // outer twiddles w_k1[n'] (k1 = 1..HALF) of this thread's columns
    auto load_two = [&](uint32_t (&tw)[HALF][CPT]) {
#pragma unroll
        for (int k1 = 0; k1 < HALF; ++k1) {
            const uint32_t* s = s_two + (k1 * T + tid) * CPT;
            if constexpr (CPT == 2) {
                const uint2 v = *(const uint2*)s;
                tw[k1][0] = v.x;
                tw[k1][1] = v.y;
            } else {
#pragma unroll
                for (int q = 0; q < CPT / 4; ++q) {
                    const uint4 v = *(const uint4*)(s + 4 * q);
                    tw[k1][4 * q] = v.x;
                    tw[k1][4 * q + 1] = v.y;
                    tw[k1][4 * q + 2] = v.z;
                    tw[k1][4 * q + 3] = v.w;
                }
            }
        }
    };

    // word offset of this thread's first column; the rest are immediates
    // on a per-n1 scalar base
    const int lofs = 32 * na0 + nb;
    uint32_t uin[HALF][CPT];
    auto load_u = [&](int idx) {
        const int hh = idx / prm.B, bb = idx - hh * prm.B;
        const uint32_t* u = (const uint32_t*)prm.u + ((long long)bb * prm.H + hh) * (M / 2);
#pragma unroll
        for (int n1 = 0; n1 < HALF; ++n1) {
            const uint32_t* un = u + n1 * Q + lofs;
#pragma unroll
            for (int j = 0; j < CPT; ++j) uin[n1][j] = un[32 * j];
        }
    };
    load_u(first);
    __syncthreads();

    uint32_t* scr = s_scr + x;
    const int i1_base = (16 * (g >> 1) + x) * 4 + 2 * (g & 1);

    const int steps = (total - first - 1) / G + 1;
    for (int step = 0; step < steps; ++step) {
        const int idx = first + step * G;
        const int h = idx / prm.B, b = idx - h * prm.B;
        const long long mrow = (long long)b * prm.H + h;
        // next row of this workgroup (the last one re-reads its own row)
        const int inext = step + 1 < steps ? idx + G : idx;
        // ---------------- outer forward stage
        {
            typedef Outer<IO> O;
            typedef typename O::V C;
            uint32_t two[HALF][CPT];
            load_two(two);
            uint32_t V[P][CPT];
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                C xin[HALF], A[P];
#pragma unroll
                for (int n1 = 0; n1 < HALF; ++n1) xin[n1] = O::from_io(uin[n1][j]);
                dft_half_in<P>(xin, A);
                V[0][j] = O::to_h2(A[0]);
                V[1][j] = O::to_h2(O::mul(A[HALF], two[HALF - 1][j]));
#pragma unroll
                for (int k1 = 1; k1 < HALF; ++k1) {
                    V[2 * k1][j] = O::to_h2(O::mul(A[k1], two[k1 - 1][j]));
                    V[2 * k1 + 1][j] = O::to_h2(O::mul(cnj(A[P - k1]), two[k1 - 1][j]));
                }
            }
#pragma unroll
            for (int s = 0; s < P; ++s) {
                uint32_t* dst = s_buf + s * Q + oa0;
                if constexpr (CPT == 2) {
                    *(uint2*)dst = make_uint2(V[s][0], V[s][1]);
                } else {
#pragma unroll
                    for (int q = 0; q < CPT / 4; ++q)
                        *(uint4*)(dst + 64 * q) =
                            make_uint4(V[s][4 * q], V[s][4 * q + 1], V[s][4 * q + 2], V[s][4 * q + 3]);
                }
            }
        }
        __syncthreads();

        // ---------------- engine: sub-rows 2*wave and 2*wave + 1
        {
            // spectrum coefficients of this row's bins, in flight while the
            // forward transforms run
            const uint4* cf = (const uint4*)prm.kf + ((long long)h * HALF + wave) * 1024;
            uint4 cfr[2][2][4];   // [sub][kt][mt]; kt = 1 is issued after sub-row 0
#pragma unroll
            for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) cfr[sub][0][mt] = cf[(sub * 2) * 256 + mt * 64 + lane];
            uint32_t z[2][2][4][2];   // [sub][kt][mt][e] packed f16 bins
#pragma unroll
            for (int sub = 0; sub < 2; ++sub) {
                const uint4* src = (const uint4*)(s_buf + (2 * wave + sub) * Q);
                uint4 a[2][2];
#pragma unroll
                for (int it = 0; it < 2; ++it)
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) a[it][ks] = src[(it * 2 + ks) * 64 + lane];
                // F1: 32-point DFT over n_a (k_a to the lanes)
                rfloat4 c1[2][4];
#pragma unroll
                for (int it = 0; it < 2; ++it)
#pragma unroll
                    for (int jt = 0; jt < 4; ++jt) c1[it][jt] = rfloat4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int jt = 0; jt < 4; ++jt) {
                        const uint4 bt = s_f1b[(ks * 4 + jt) * 64 + lane];
#pragma unroll
                        for (int it = 0; it < 2; ++it) c1[it][jt] = mma_f16(a[it][ks], bt, c1[it][jt]);
                    }
                // twiddle W_1024^{k_a n_b}; F2's B operand
                uint4 b2[2][2];
#pragma unroll
                for (int it = 0; it < 2; ++it)
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt) {
                        uint32_t w[4];
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr)
                            w[rr] = as_u32(hmul(as_h2(pk2(c1[it][2 * kt][rr], c1[it][2 * kt + 1][rr])),
                                                as_h2(twf[it][kt][rr])));
                        b2[it][kt] = make_uint4(w[0], w[1], w[2], w[3]);
                    }
                // F2: 32-point DFT over n_b, k_b in-lane (mirror row order)
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) {
                        rfloat4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int ks = 0; ks < 2; ++ks) acc = mma_f16(f2a[mt][ks], b2[ks][kt], acc);
                        z[sub][kt][mt][0] = pk2(acc[0], acc[1]);
                        z[sub][kt][mt][1] = pk2(acc[2], acc[3]);
                    }
                if (sub == 0) {
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                        for (int mt = 0; mt < 4; ++mt) cfr[s2][1][mt] = cf[(s2 * 2 + 1) * 256 + mt * 64 + lane];
                }
                __builtin_amdgcn_sched_barrier(0);
            }

            // ---------------- spectrum product
            uint4 a2[2][2][2];   // [sub][kt][ks] I2 A operands
            if (wave != 0) {
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    uint32_t p0[4][2], p1[4][2];
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) {
                        const uint4 c0 = cfr[0][kt][mt];
                        const uint4 c1v = cfr[1][kt][mt];
#pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            const rhalf2 zx = as_h2(z[0][kt][mt][e]), zy = as_h2(z[1][kt][mt][e]);
                            const uint32_t al0 = e ? c0.z : c0.x, be0 = e ? c0.w : c0.y;
                            const uint32_t al1 = e ? c1v.z : c1v.x, be1 = e ? c1v.w : c1v.y;
                            p0[mt][e] = as_u32(hcmla(as_h2(al0), zx, as_h2(be0), zy));
                            p1[mt][e] = as_u32(hcmla(as_h2(al1), zy, as_h2(be1), zx));
                        }
                    }
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        a2[0][kt][ks] = make_uint4(p0[2 * ks][0], p0[2 * ks][1], p0[2 * ks + 1][0], p0[2 * ks + 1][1]);
                        a2[1][kt][ks] = make_uint4(p1[2 * ks][0], p1[2 * ks][1], p1[2 * ks + 1][0], p1[2 * ks + 1][1]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
                // sub-row 0: k_a = 0 column pairs k_b with -k_b (another lane
                // group): exchange through LDS
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int e = 0; e < 2; ++e) scr[16 * rmid_perm(8 * mt + 2 * g + e, 32)] = z[0][0][mt][e];
                // k_b = 0 also at slot 32 (slots 34..38 are padding), so the
                // partner slot 32 - k_b needs no wrap
                scr[16 * (32 + 2 * g)] = z[0][0][0][0];
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                uint32_t zq[4][2];
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const int kb = rmid_perm(8 * mt + 2 * g + e, 32);
                        zq[mt][e] = scr[16 * (32 - kb)];
                    }
                const bool l0 = (x == 0);
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    uint32_t p0[4][2], p1[4][2];
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) {
                        const int pm = (mt + 2) & 3;
                        const uint4 c0 = cfr[0][kt][mt];
                        const uint4 c1v = cfr[1][kt][mt];
#pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            // negation partner of sub-row 0
                            uint32_t pn;
                            if (kt == 0) pn = l0 ? zq[mt][e] : z[0][1][pm][e];
                            else pn = l0 ? z[0][1][pm][e] : z[0][0][pm][e];
                            // reversal partner of sub-row P/2: (31-k_a, 31-k_b)
                            const uint32_t pr = kt == 0 ? rot_up(z[1][1][pm][e]) : rot_down(z[1][0][pm][e]);
                            const uint32_t al0 = e ? c0.z : c0.x, be0 = e ? c0.w : c0.y;
                            const uint32_t al1 = e ? c1v.z : c1v.x, be1 = e ? c1v.w : c1v.y;
                            p0[mt][e] = as_u32(hpair(as_h2(al0), as_h2(z[0][kt][mt][e]), as_h2(be0), as_h2(pn)));
                            p1[mt][e] = as_u32(hpair(as_h2(al1), as_h2(z[1][kt][mt][e]), as_h2(be1), as_h2(pr)));
                        }
                    }
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        a2[0][kt][ks] = make_uint4(p0[2 * ks][0], p0[2 * ks][1], p0[2 * ks + 1][0], p0[2 * ks + 1][1]);
                        a2[1][kt][ks] = make_uint4(p1[2 * ks][0], p1[2 * ks][1], p1[2 * ks + 1][0], p1[2 * ks + 1][1]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }

            // next row's input: issued only now, because the load counter
            // retires in order and the coefficient loads above must not
            // wait behind it
            load_u(inext);

            // ---------------- inverse 1024-point DFT of both sub-rows
#pragma unroll
            for (int sub = 0; sub < 2; ++sub) {
                // I2: inverse 32-point DFT over k_b (data as A), then the
                // conjugate twiddle; I1's B operand
                uint4 b1v[2][2];
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        rfloat4 re = {0.f, 0.f, 0.f, 0.f}, im = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int ks = 0; ks < 2; ++ks) {
                            re = mma_f16(a2[sub][kt][ks], i2b[ks][2 * nt], re);
                            im = mma_f16(a2[sub][kt][ks], i2b[ks][2 * nt + 1], im);
                        }
                        uint32_t w[4];
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr)
                            w[rr] = as_u32(hmulc(as_h2(pk2(re[rr], im[rr])), as_h2(twf[kt][nt][rr])));
                        b1v[kt][nt] = make_uint4(w[0], w[1], w[2], w[3]);
                    }
                // I1: inverse 32-point DFT over k_a, all 32 n_a, to LDS
                uint32_t* dst = s_buf + (2 * wave + sub) * Q;
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    rfloat4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        const uint4 at = s_i1a[(mt * 2 + ks) * 64 + lane];
#pragma unroll
                        for (int nt = 0; nt < 2; ++nt) acc[nt] = mma_f16(at, b1v[ks][nt], acc[nt]);
                    }
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        // n_a = 8 mt + 2 g + e, n_b = kmap32(nt, x):
                        // eng_addr(8 mt + 2 g, nt, x)
                        *(uint2*)(dst + i1_base + ((nt * 2 + (mt >> 1)) * 64 + 32 * (mt & 1)) * 4) =
                            make_uint2(pk2(acc[nt][0], acc[nt][1]), pk2(acc[nt][2], acc[nt][3]));
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        __syncthreads();

        // ---------------- outer inverse stage and store
        {
            uint32_t R[P][CPT];
#pragma unroll
            for (int s = 0; s < P; ++s) {
                const uint32_t* src = s_buf + s * Q + oa0;
                if constexpr (CPT == 2) {
                    const uint2 v = *(const uint2*)src;
                    R[s][0] = v.x;
                    R[s][1] = v.y;
                } else {
#pragma unroll
                    for (int q = 0; q < CPT / 4; ++q) {
                        const uint4 v = *(const uint4*)(src + 64 * q);
                        R[s][4 * q] = v.x;
                        R[s][4 * q + 1] = v.y;
                        R[s][4 * q + 2] = v.z;
                        R[s][4 * q + 3] = v.w;
                    }
                }
            }
            uint32_t* yrow = (uint32_t*)prm.y + mrow * (M / 2);
            uint32_t two[HALF][CPT];
            load_two(two);
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                typedef Outer<IO> O;
                typedef typename O::V C;
                C Bv[P], zo[HALF];
                Bv[0] = O::from_h2(R[0][j]);
                Bv[HALF] = O::mulc(O::from_h2(R[1][j]), two[HALF - 1][j]);
#pragma unroll
                for (int k1 = 1; k1 < HALF; ++k1) {
                    Bv[k1] = O::mulc(O::from_h2(R[2 * k1][j]), two[k1 - 1][j]);
                    Bv[P - k1] = cnj(O::mulc(O::from_h2(R[2 * k1 + 1][j]), two[k1 - 1][j]));
                }
                idft_half_out<P>(Bv, zo);
#pragma unroll
                for (int n1 = 0; n1 < HALF; ++n1) yrow[n1 * Q + lofs + 32 * j] = O::to_io(zo[n1]);
            }
        }
    }
}

hipError_t launch_wide(int io, int P, const WideParams& p, int lds, hipStream_t s) {
    const dim3 grid((unsigned)p.grid), blk((unsigned)(32 * P));
#define FFTCONV_WIDE(IOT, PP)                                                              \
    do {                                                                                   \
        if (lds > 64 * 1024) {                                                             \
            hipError_t e_ = hipFuncSetAttribute((const void*)wide_kernel<IOT, PP>,         \
                                                hipFuncAttributeMaxDynamicSharedMemorySize, \
                                                lds);                                      \
            if (e_ != hipSuccess) return e_;                                               \
        }                                                                                  \
        hipLaunchKernelGGL((wide_kernel<IOT, PP>), grid, blk, lds, s, p);                  \
    } while (0)
    if (io == IO_BF16) {
        if (P == 4) FFTCONV_WIDE(IO_BF16, 4);
        else if (P == 8) FFTCONV_WIDE(IO_BF16, 8);
        else FFTCONV_WIDE(IO_BF16, 16);
    } else {
        if (P == 4) FFTCONV_WIDE(IO_F16, 4);
        else if (P == 8) FFTCONV_WIDE(IO_F16, 8);
        else FFTCONV_WIDE(IO_F16, 16);
    }
#undef FFTCONV_WIDE
    return hipGetLastError();
}

// Spectrum coefficients in the wide kernel's engine order:
// [h][unit j < P/2][sub 2][kt 2][mt 4][lane 64][e 2], each (alpha, beta) as
// packed f16.  Unit j > 0, sub 0 holds bin k = j + P k' (alpha_k, beta_k);
// sub 1 holds conj(alpha_{-k}), conj(beta_{-k}).  Unit 0: sub 0 is bin P k',
// sub 1 is bin P/2 + P k'.  k' = kmap32(kt, x) + 32 rmid_perm(8 mt + 2 g + e).
__global__ void wide_coef_kernel(WideCoefParams P) {
    const int HALF = P.P / 2;
    const long long per_ch = (long long)HALF * 2048;
    const long long total = (long long)P.hcount * per_ch;
    for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < total;
         i += (long long)gridDim.x * blockDim.x) {
        const long long hl = i / per_ch;
        int rem = (int)(i - hl * per_ch);
        const int e = rem & 1;
        const int lane = (rem >> 1) & 63;
        const int mt = (rem >> 7) & 3;
        const int kt = (rem >> 9) & 1;
        const int sub = (rem >> 10) & 1;
        const int j = rem >> 11;
        const int gg = lane >> 4, xx = lane & 15;
        const int ka = kmap32(kt, xx), kb = rmid_perm(8 * mt + 2 * gg + e, 32);
        const int kp = ka + 32 * kb;
        long long k;
        bool conj_out = false;
        if (j == 0) {
            k = sub == 0 ? (long long)P.P * kp : (long long)HALF + (long long)P.P * kp;
        } else {
            k = j + (long long)P.P * kp;
            if (sub == 1) {
                k = (P.M - k) % P.M;
                conj_out = true;
            }
        }
        const float2* X = P.X + hl * P.L;
        const float2 K1 = X[k], K2 = X[k + P.M];
        double sn, cs;
        sincospi(2.0 * (double)k / (double)P.L, &sn, &cs);
        const float s = (float)sn, c = (float)cs;
        float2 al = make_float2(0.5f * ((1.f - s) * K1.x + (1.f + s) * K2.x),
                                0.5f * ((1.f - s) * K1.y + (1.f + s) * K2.y));
        const float2 dlt = make_float2(K1.x - K2.x, K1.y - K2.y);
        float2 be = make_float2(-0.5f * c * dlt.y, 0.5f * c * dlt.x);
        if (conj_out) {
            al.y = -al.y;
            be.y = -be.y;
        }
        _Float16 hv[4] = {(_Float16)al.x, (_Float16)al.y, (_Float16)be.x, (_Float16)be.y};
        ((uint2*)P.kf)[(long long)(P.h0 + hl) * per_ch + rem] = *(const uint2*)hv;
    }
}

hipError_t launch_wide_coef(const WideCoefParams& p, hipStream_t s) {
    hipLaunchKernelGGL(wide_coef_kernel, dim3(2048), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace fftconv
