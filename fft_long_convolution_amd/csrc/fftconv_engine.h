// The 32 x 32 matrix-core engine shared by the fused wide kernel and the
// multi-pass inner kernel: the 1024-point DFT of one LDS region (stage over
// n_a, twiddle W_1024^{k_a n_b}, stage over n_b), the spectrum product of
// two regions, the inverse, and the small vector-ALU DFTs of the outer
// stages (page "FlashFFTConv: Efficient Convolutions for Long Sequences with
// Tensor Cores", section 3.4 and Algorithm 1).
//
// Engine layout of a region (1024 complex f16, one 32-bit word each): the
// uint4 (it*2 + ks)*64 + lane holds n_a = 16 ks + 4 g + 0..3 at
// n_b = kmap32(it, x) (lane = 16 g + x).  After the forward stages a lane
// holds bins k' = k_a + 32 k_b with k_a = kmap32(kt, x) and
// k_b = rmid_perm(8 mt + 2 g + e, 32) in z[kt][mt][e].
#pragma once

#include "fftconv_mfma.h"

#include <type_traits>

namespace fftconv {
namespace eng {


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

// In-place n-point DFT (n = 1..32), natural order in and out; INV uses
// W^-1.  Radix-2 decimation in time, indices and twiddles resolved at
// compile time.
template <int n, bool INV, class V>
__device__ __forceinline__ void dft_small(V (&v)[n]) {
    if constexpr (n == 1) {
        return;
    } else if constexpr (n == 2) {
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
    } else {
        V e[n / 2], o[n / 2];
#pragma unroll
        for (int m = 0; m < n / 2; ++m) {
            e[m] = v[2 * m];
            o[m] = v[2 * m + 1];
        }
        dft_small<n / 2, INV>(e);
        dft_small<n / 2, INV>(o);
#pragma unroll
        for (int k = 0; k < n / 2; ++k) {
            const V t = mulw_k(o[k], INV ? -(32 / n) * k : (32 / n) * k);   // W_n^{+-k}
            v[k] = e[k] + t;
            v[k + n / 2] = e[k] - t;
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
    // element-wise product with a packed pair of I/O values (a gate):
    // exact in fp32 for bf16, one rounding in packed f16 for f16
    static __device__ __forceinline__ V emul(V a, uint32_t g) {
        return a * from_io(g);
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


// Kernel gradient, 4 Z_g for one bin from its value and its mirror partner
// (not conjugated) of u and dy; W = exp(2 pi i k / M)
__device__ __forceinline__ rhalf2 kg_self(uint32_t a, uint32_t ap, uint32_t d, uint32_t dp, rhalf2 W) {
    const rhalf2 A = as_h2(a), Ap = as_h2(ap), Dv = as_h2(d), Dp = as_h2(dp);
    const rhalf2 cAp = {Ap.x, -Ap.y}, cDp = {Dp.x, -Dp.y};
    const rhalf2 E2 = A + cAp, O2 = A - cAp, Ed = Dv + cDp, Od = Dv - cDp;
    const rhalf2 T = Od - hmul(Ed, W);
    const rhalf2 two = {(_Float16)2.f, (_Float16)2.f};
    return __builtin_elementwise_fma(hmulc(Dv, E2), two, hmulc(T, O2));
}

// The same for an element-wise pair: a, d the bin's values of u and dy, c, e
// the conjugated mirror values held at the same position; returns 4 Z_g[k]
// and, in the conjugated form of the partner region, 4 conj Z_g[-k].
__device__ __forceinline__ void kg_pair(uint32_t a_, uint32_t c_, uint32_t d_, uint32_t e_, rhalf2 W,
                                        rhalf2& RX, rhalf2& RY) {
    const rhalf2 a = as_h2(a_), c = as_h2(c_), d = as_h2(d_), ee = as_h2(e_);
    const rhalf2 E2 = a + c, O2 = a - c, Ed = d + ee, Od = d - ee;
    const rhalf2 WE = hmul(Ed, W);
    const rhalf2 two = {(_Float16)2.f, (_Float16)2.f};
    RX = __builtin_elementwise_fma(hmulc(d, E2), two, hmulc(Od - WE, O2));
    RY = __builtin_elementwise_fma(hmulc(ee, E2), two, hmulc(Od + WE, O2));
}

// LDS word address of (n_a, n_b) within a sub-row region: the engine reads
// uint4 (it*2 + ks)*64 + lane holding n_a = 16 ks + 4 g + 0..3 and
// n_b = kmap32(it, x).
__device__ __forceinline__ int eng_addr(int na, int it, int x) {
    return (((it * 2 + (na >> 4)) * 64 + 16 * ((na >> 2) & 3) + x) << 2) + (na & 3);
}


// Dynamic distribution of rows (or units) over persistent workgroups.  The
// grid (G workgroups, a multiple of 8) splits into the 8 groups that share
// an XCD (consecutive dispatch ids go to consecutive XCDs).  Group x owns
// the indices whose position within each block of G falls in
// [x G/8, (x + 1) G/8) -- neighbouring indices share spectrum coefficients,
// which then stay in that XCD's L2 -- and its workgroups claim them in
// order from their own counter (ctr[32 x], a 128-byte line each).  A
// workgroup that the CU's arbitration favours simply claims more.
// With no counters (c == nullptr) the claims are static: the workgroup at
// position p of its group takes the group's indices p, p + G/8, p + 2 G/8,
// ... (the same order, without atomics or counters to clear).
struct XcdClaim {
    uint32_t* ctr;
    int G, gx, x;
    mutable uint32_t ks;   // static claims: the next one of this workgroup
    __device__ __forceinline__ XcdClaim(uint32_t* c, int grid, int bid)
        : ctr(c ? c + 32 * (bid & 7) : nullptr), G(grid), gx(grid >> 3), x(bid & 7),
          ks((uint32_t)(bid >> 3)) {}
    // next index of this group (monotonic; >= total means done)
    __device__ __forceinline__ long long next() const {
        uint32_t k;
        if (ctr) {
            k = atomicAdd(ctr, 1u);
        } else {
            k = ks;
            ks += (uint32_t)gx;
        }
        return (long long)(k / gx) * G + (long long)x * gx + (k % gx);
    }
};

// Stage tables the engine keeps in registers for the whole kernel.
struct Regs {
    uint4 f2a[4][2];        // stage over n_b, A tiles
    uint4 i2b[2][4];        // its inverse, B tiles
    uint32_t twf[2][2][4];  // W_1024^{k_a n_b} (conjugated for the inverse)
};

__device__ __forceinline__ void load_regs(Regs& E, const void* f2a, const void* i2b,
                                          const uint32_t* twf, int lane) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) E.f2a[mt][ks] = ((const uint4*)f2a)[(mt * 2 + ks) * 64 + lane];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) E.i2b[ks][jt] = ((const uint4*)i2b)[(ks * 4 + jt) * 64 + lane];
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) E.twf[it][kt][r] = twf[lane * 16 + (it * 2 + kt) * 4 + r];
}

// The same tables through buffer descriptors (scalar bases, one 32-bit lane
// offset): for kernels that reload them inside their row loop, where
// hoisted 64-bit per-lane addresses would stay live across the loop.
__device__ __forceinline__ void load_regs_buf(Regs& E, const void* f2a, const void* i2b,
                                              const uint32_t* twf, int lane);

// Forward 1024-point DFT of one region (engine layout) into z[kt][mt][e].
// SK (a band limit below M/4): the odd M-tiles of the second stage,
// k_b = 8..23, hold only bins the limit zeroes -- not computed (zero).
template <bool SK = false>
__device__ __forceinline__ void forward(const uint32_t* region, const uint4* s_f1b, const Regs& E,
                                        int lane, uint32_t (&z)[2][4][2]) {
    const uint4* src = (const uint4*)region;
    uint4 a[2][2];
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) a[it][ks] = src[(it * 2 + ks) * 64 + lane];
    // 32-point DFT over n_a (k_a to the lanes)
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
    // twiddle W_1024^{k_a n_b}; the next stage's B operand
    uint4 b2[2][2];
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            uint32_t w[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                w[rr] = as_u32(hmul(as_h2(pk2(c1[it][2 * kt][rr], c1[it][2 * kt + 1][rr])),
                                    as_h2(E.twf[it][kt][rr])));
            b2[it][kt] = make_uint4(w[0], w[1], w[2], w[3]);
        }
    // 32-point DFT over n_b, k_b in-lane (mirror row order)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            if (SK && (mt & 1)) {
                z[kt][mt][0] = z[kt][mt][1] = 0u;
                continue;
            }
            rfloat4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) acc = mma_f16(E.f2a[mt][ks], b2[ks][kt], acc);
            z[kt][mt][0] = pk2(acc[0], acc[1]);
            z[kt][mt][1] = pk2(acc[2], acc[3]);
        }
}

// Gather the spectrum-product results p[mt][e] of one column tile kt into
// the inverse stage's A operands: K-step ks holds M-tiles 2 ks and 2 ks + 1,
// or with SK ks and ks + 2 (K-step 1 is then all zero; the inverse table of
// a band-limited call is grouped the same way).
template <bool SK = false>
__device__ __forceinline__ void pack_a2(const uint32_t (&p)[4][2], uint4 (&a2)[2]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const int m0 = SK ? ks : 2 * ks, m1 = SK ? ks + 2 : 2 * ks + 1;
        a2[ks] = make_uint4(p[m0][0], p[m0][1], p[m1][0], p[m1][1]);
    }
}

// Element-wise spectrum product of a region pair whose second region holds
// conj(Z[-k]) where the first holds Z[k]:
//   X' = a0 X + b0 Y,  Y' = a1 Y + b1 X   (coefficients (a_e0, b_e0, a_e1, b_e1))
template <bool SK = false>
__device__ __forceinline__ void pair_elem(int kt, const uint32_t (&zX)[2][4][2],
                                          const uint32_t (&zY)[2][4][2], const uint4 (&cX)[4],
                                          const uint4 (&cY)[4], uint4 (&a2X)[2], uint4 (&a2Y)[2]) {
    uint32_t p0[4][2], p1[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            if (SK && (mt & 1)) {
                p0[mt][e] = p1[mt][e] = 0u;
                continue;
            }
            const rhalf2 zx = as_h2(zX[kt][mt][e]), zy = as_h2(zY[kt][mt][e]);
            const uint32_t al0 = e ? cX[mt].z : cX[mt].x, be0 = e ? cX[mt].w : cX[mt].y;
            const uint32_t al1 = e ? cY[mt].z : cY[mt].x, be1 = e ? cY[mt].w : cY[mt].y;
            p0[mt][e] = as_u32(hcmla(as_h2(al0), zx, as_h2(be0), zy));
            p1[mt][e] = as_u32(hcmla(as_h2(al1), zy, as_h2(be1), zx));
        }
    pack_a2<SK>(p0, a2X);
    pack_a2<SK>(p1, a2Y);
}

// Self pairing: region X pairs k' with -k' (negation, the k_a = 0 column
// through the LDS exchange scr), region Y pairs k' with 1023 - k' (reversal,
// one lane over).  Both with X' = a X + b conj(partner).
// First the exchange: every lane writes its k_a = 0 column bins.
__device__ __forceinline__ void self_exchange(const uint32_t (&zX)[2][4][2], uint32_t* scr, int g,
                                              uint32_t (&zq)[4][2]) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int e = 0; e < 2; ++e) scr[16 * rmid_perm(8 * mt + 2 * g + e, 32)] = zX[0][mt][e];
    // k_b = 0 also at slot 32 (slots 34..38 are padding), so the partner
    // slot 32 - k_b needs no wrap
    scr[16 * (32 + 2 * g)] = zX[0][0][0];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int kb = rmid_perm(8 * mt + 2 * g + e, 32);
            zq[mt][e] = scr[16 * (32 - kb)];
        }
}
template <bool SK = false>
__device__ __forceinline__ void pair_self(int kt, bool l0, const uint32_t (&zX)[2][4][2],
                                          const uint32_t (&zY)[2][4][2], const uint32_t (&zq)[4][2],
                                          const uint4 (&cX)[4], const uint4 (&cY)[4],
                                          uint4 (&a2X)[2], uint4 (&a2Y)[2]) {
    uint32_t p0[4][2], p1[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const int pm = (mt + 2) & 3;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            if (SK && (mt & 1)) {
                p0[mt][e] = p1[mt][e] = 0u;
                continue;
            }
            // negation partner of X
            uint32_t pn;
            if (kt == 0) pn = l0 ? zq[mt][e] : zX[1][pm][e];
            else pn = l0 ? zX[1][pm][e] : zX[0][pm][e];
            // reversal partner of Y: (31 - k_a, 31 - k_b)
            const uint32_t pr = kt == 0 ? rot_up(zY[1][pm][e]) : rot_down(zY[0][pm][e]);
            const uint32_t al0 = e ? cX[mt].z : cX[mt].x, be0 = e ? cX[mt].w : cX[mt].y;
            const uint32_t al1 = e ? cY[mt].z : cY[mt].x, be1 = e ? cY[mt].w : cY[mt].y;
            p0[mt][e] = as_u32(hpair(as_h2(al0), as_h2(zX[kt][mt][e]), as_h2(be0), as_h2(pn)));
            p1[mt][e] = as_u32(hpair(as_h2(al1), as_h2(zY[kt][mt][e]), as_h2(be1), as_h2(pr)));
        }
    }
    pack_a2<SK>(p0, a2X);
    pack_a2<SK>(p1, a2Y);
}

// Inverse 1024-point DFT of one region: A operands a2[kt][ks] -> region
// (engine layout).  i1_base = (16 (g >> 1) + x) * 4 + 2 (g & 1).
template <bool SK = false>
__device__ __forceinline__ void inverse(const uint4 (&a2)[2][2], const uint4* s_i1a, const Regs& E,
                                        int lane, int i1_base, uint32_t* region) {
    // inverse 32-point DFT over k_b (data as A), then the conjugate twiddle
    uint4 b1v[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            rfloat4 re = {0.f, 0.f, 0.f, 0.f}, im = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (SK && ks == 1) continue;
                re = mma_f16(a2[kt][ks], E.i2b[ks][2 * nt], re);
                im = mma_f16(a2[kt][ks], E.i2b[ks][2 * nt + 1], im);
            }
            uint32_t w[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                w[rr] = as_u32(hmulc(as_h2(pk2(re[rr], im[rr])), as_h2(E.twf[kt][nt][rr])));
            b1v[kt][nt] = make_uint4(w[0], w[1], w[2], w[3]);
        }
    // inverse 32-point DFT over k_a, all 32 n_a, to LDS
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
            // n_a = 8 mt + 2 g + e, n_b = kmap32(nt, x): eng_addr(8 mt + 2 g, nt, x)
            *(uint2*)(region + i1_base + ((nt * 2 + (mt >> 1)) * 64 + 32 * (mt & 1)) * 4) =
                make_uint2(pk2(acc[nt][0], acc[nt][1]), pk2(acc[nt][2], acc[nt][3]));
        }
    }
}

// Conversions and buffer-descriptor loads shared by the multi-pass kernels.
__device__ __forceinline__ rfloat2 f2_from_h2(uint32_t v) {
    const rhalf2 h = as_h2(v);
    const rfloat2 r = {(float)h.x, (float)h.y};
    return r;
}
template <int IO>
__device__ __forceinline__ rfloat2 f2_from_io(uint32_t v) {
    if constexpr (IO == IO_BF16) {
        const rfloat2 r = {__uint_as_float(v << 16), __uint_as_float(v & 0xffff0000u)};
        return r;
    } else {
        return f2_from_h2(v);
    }
}

// 16-byte load through a buffer descriptor (base in scalar registers, a
// per-lane byte offset, a scalar byte offset): the compiler keeps no 64-bit
// per-lane address to hoist out of a loop.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_ld16(__amdgpu_buffer_rsrc_t r, unsigned voff, int soff) {
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void load_regs_buf(Regs& E, const void* f2a, const void* i2b,
                                              const uint32_t* twf, int lane) {
    const __amdgpu_buffer_rsrc_t rf = buf_rsrc(f2a, 8 * 64 * 16);
    const __amdgpu_buffer_rsrc_t ri = buf_rsrc(i2b, 8 * 64 * 16);
    const __amdgpu_buffer_rsrc_t rt = buf_rsrc(twf, 64 * 16 * 4);
    const unsigned vo = (unsigned)lane * 16u;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) E.f2a[mt][ks] = buf_ld16(rf, vo, (mt * 2 + ks) * 64 * 16);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) E.i2b[ks][jt] = buf_ld16(ri, vo, (ks * 4 + jt) * 64 * 16);
    // twf: 16 consecutive words per lane, [it][kt][r]
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint4 v = buf_ld16(rt, vo * 4u, q * 16);
        E.twf[q >> 1][q & 1][0] = v.x;
        E.twf[q >> 1][q & 1][1] = v.y;
        E.twf[q >> 1][q & 1][2] = v.z;
        E.twf[q >> 1][q & 1][3] = v.w;
    }
}

}  // namespace eng
}  // namespace fftconv
