// gfx950 (CDNA4) kernels of the causal FFT long convolution.
//
// Every DFT stage is a small dense complex matrix product on the matrix
// cores (v_mfma_f32_16x16x32_f16 for 16-bit I/O plans, v_mfma_f32_16x16x4_f32
// for fp32 plans), the Monarch factorisation of the FFT described on the
// page "FlashFFTConv: Efficient Convolutions for Long Sequences with Tensor
// Cores", section 3.4 ("The Monarch FFT Decomposition", Algorithm 1 and its
// order-3/4 generalisations).  Data between stages lives in LDS as fp32
// complex; each stage rounds its operand to the matrix-core type once and
// accumulates in fp32.  Twiddles and the spectrum product are fp32 VALU work.
//
// Complex N-point DFTs are embedded as real 2N x 2N matrices
//     [re_out]   [ Re W  -Im W ] [re_in]
//     [im_out] = [ Im W   Re W ] [im_in]
// with re/im interleaved along both the rows and the contraction index, so a
// lane always holds the real and imaginary part of the same point.
//
// Matrix-core operand layouts used here (16x16 output tiles, 64 lanes,
// lane = 16*g + x):
//   A operand: lane (g, x) holds row x, contraction slots owned by group g
//   B operand: lane (g, x) holds column x, contraction slots owned by g
//   C result : lane (g, x) holds rows 4g..4g+3 of column x
// Which contraction index sits in which (g, slot) is a free choice as long
// as the matrix tables (built on the host) use the same one.
#include "fftconv_internal.h"

namespace fftconv {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
    return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}
// a * conj(b)
__device__ __forceinline__ float2 cmulc(float2 a, float2 b) {
    return make_float2(a.x * b.x + a.y * b.y, a.y * b.x - a.x * b.y);
}

// ---------------------------------------------------------------------------
// Matrix-core traits.
//  gather decode: K-step ks, lane group g, slot j <-> input digit nn, part d
//    f16: nn = 16 ks + 4 g + (j >> 1), d = j & 1     (8 halves per lane)
//    f32: nn = 2 ks + (g >> 1),        d = g & 1     (1 float per lane)
//  chain decode (operand taken straight from accumulators z[mt][e], which
//  hold output slot 8 mt + 2 g + e):
//    f16: K-step ks takes z[2ks + (j>>2)][(j>>1)&1], part j&1
//    f32: K-step ks takes z[ks>>2][(ks&3)>>1], part ks&1
// ---------------------------------------------------------------------------
struct MfF16 {
    typedef half8 AB;
    static constexpr int ksteps(int nin) { return nin <= 16 ? 1 : nin / 16; }
    static __device__ __forceinline__ floatx4 mma(const AB& a, const AB& b,
                                                  floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    template <class F>
    static __device__ __forceinline__ AB gather(int ks, int g, int nin,
                                                F&& get) {
        AB b;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int nn = 16 * ks + 4 * g + jj;
            float2 v = make_float2(0.f, 0.f);
            if (nn < nin) v = get(nn);
            b[2 * jj] = (_Float16)v.x;
            b[2 * jj + 1] = (_Float16)v.y;
        }
        return b;
    }
    template <int MT>
    static __device__ __forceinline__ AB chain(int ks,
                                               const float2 (&z)[MT][2]) {
        AB b;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float2 v = z[2 * ks + (j >> 2)][(j >> 1) & 1];
            b[j] = (_Float16)((j & 1) ? v.y : v.x);
        }
        return b;
    }
};

struct MfF32 {
    typedef float AB;
    static constexpr int ksteps(int nin) { return nin / 2; }
    static __device__ __forceinline__ floatx4 mma(const AB& a, const AB& b,
                                                  floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    template <class F>
    static __device__ __forceinline__ AB gather(int ks, int g, int nin,
                                                F&& get) {
        const int nn = 2 * ks + (g >> 1);
        float2 v = make_float2(0.f, 0.f);
        if (nn < nin) v = get(nn);
        return (g & 1) ? v.y : v.x;
    }
    template <int MT>
    static __device__ __forceinline__ AB chain(int ks,
                                               const float2 (&z)[MT][2]) {
        const float2 v = z[ks >> 2][(ks & 3) >> 1];
        return (ks & 1) ? v.y : v.x;
    }
};

// ---------------------------------------------------------------------------
// One regular Monarch stage over an LDS line (in place).
//  forward: gather digits nn (only the lower half when HALF: the causal zero
//           padding), DFT, multiply output digit k by W_{S}^{k c}, scatter.
//  inverse: gather digits k and multiply by conj(W_S^{k c}), inverse DFT,
//           scatter (only the lower half of the outputs when HALF).
// ---------------------------------------------------------------------------
template <class MF, int N, bool INV, bool HALF>
__device__ __forceinline__ void run_stage(float2* __restrict__ line,
                                          int line_len, const StageDev& d,
                                          int tw_off, int wave, int nwaves,
                                          int lane) {
    constexpr int NIN = (HALF && !INV) ? N / 2 : N;
    constexpr int NOUT = (HALF && INV) ? N / 2 : N;
    constexpr int KS = MF::ksteps(NIN);
    constexpr int MT = NOUT / 8 > 0 ? NOUT / 8 : 1;
    const int g = lane >> 4, x = lane & 15;
    const typename MF::AB* mat =
        (const typename MF::AB*)(INV ? d.mat_i : d.mat_f);
    typename MF::AB A[MT][KS];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) A[mt][ks] = mat[(mt * KS + ks) * 64 + lane];

    const int ntiles = (line_len / N) >> 4;
    const int cs = d.sb * d.Cb;
    const float2* __restrict__ tw = d.tw;
    for (int t = wave; t < ntiles; t += nwaves) {
        const int q = (t << 4) + x;
        const int cb = q % d.Cb;
        const int r1 = q / d.Cb;
        const int c = r1 % d.sb;
        const int b = r1 / d.sb;
        const int base = (b * d.Sb + c) * d.Cb + cb;
        const int twc = c * d.tw_mul + tw_off + cb;
        typename MF::AB B[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            B[ks] = MF::gather(ks, g, NIN, [&](int nn) {
                float2 v = line[base + nn * cs];
                if (INV) v = cmulc(v, tw[nn * d.tw_stride + twc]);
                return v;
            });
        }
        floatx4 acc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            acc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                acc[mt] = MF::mma(A[mt][ks], B[ks], acc[mt]);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int slot = 8 * mt + 2 * g + e;
                if (slot < NOUT) {
                    float2 v = make_float2(acc[mt][2 * e], acc[mt][2 * e + 1]);
                    if (!INV) v = cmul(v, tw[slot * d.tw_stride + twc]);
                    line[base + slot * cs] = v;
                }
            }
    }
}

template <class MF, bool INV>
__device__ __forceinline__ void dispatch_stage(bool half, const StageDev& d,
                                               float2* line, int line_len,
                                               int tw_off, int wave,
                                               int nwaves, int lane) {
    if (half) {
        if (d.n == 32) run_stage<MF, 32, INV, true>(line, line_len, d, tw_off, wave, nwaves, lane);
        else if (d.n == 16) run_stage<MF, 16, INV, true>(line, line_len, d, tw_off, wave, nwaves, lane);
        else run_stage<MF, 8, INV, true>(line, line_len, d, tw_off, wave, nwaves, lane);
    } else {
        if (d.n == 32) run_stage<MF, 32, INV, false>(line, line_len, d, tw_off, wave, nwaves, lane);
        else if (d.n == 16) run_stage<MF, 16, INV, false>(line, line_len, d, tw_off, wave, nwaves, lane);
        else run_stage<MF, 8, INV, false>(line, line_len, d, tw_off, wave, nwaves, lane);
    }
}

// ---------------------------------------------------------------------------
// Spectrum coefficients: one entry per packed bin = (alpha, beta).
// ---------------------------------------------------------------------------
template <int IO>
__device__ __forceinline__ void load_ab(const void* kf, long long idx,
                                        float2& a, float2& b) {
    if (IO == IO_F32) {
        const float4 v = ((const float4*)kf)[idx];
        a = make_float2(v.x, v.y);
        b = make_float2(v.z, v.w);
    } else {
        const uint2 w = ((const uint2*)kf)[idx];
        const _Float16* h = (const _Float16*)&w;
        a = make_float2((float)h[0], (float)h[1]);
        b = make_float2((float)h[2], (float)h[3]);
    }
}

// out = a*z + b*conj(p)
__device__ __forceinline__ float2 pair_combine(float2 a, float2 z, float2 b,
                                               float2 p) {
    return make_float2(a.x * z.x - a.y * z.y + b.x * p.x + b.y * p.y,
                       a.x * z.y + a.y * z.x + b.y * p.x - b.x * p.y);
}

// ---------------------------------------------------------------------------
// The innermost stage fused with the bin pairing and the first inverse
// stage (the forward DFT, the product with the kernel spectrum and the
// start of the inverse stay in registers, as in Algorithm 1 of the page).
//
// Bins of block b (lower part q) pair with bins of the block whose lower
// part is -q (mod Q); digit k pairs with n-1-k, except in the q = 0 block
// where it pairs with -k (mod n).  The forward matrix rows are permuted
// (slot s -> digit s for s < n/2, 3n/2-1-s otherwise) so that partner
// digits sit in the same lane, M-tile mt <-> mt + MT/2.  A lane processes a
// "lane slot": one block in column 0 of the MFMA tile and its partner in
// column 1.  Unit types:
//   0: one slab whose outer bin part is 0 (the only type for a fused row):
//      lane slot 0 = (q=0, q=Q/2), lane slot j = (j, Q-j)
//   1: one slab whose outer part is half the outer range: (j, Q-1-j)
//   2: two slabs with mirrored outer parts: (j in slab 0, Q-1-j in slab 1)
// ---------------------------------------------------------------------------
__device__ __forceinline__ int mid_perm(int slot, int n) {
    return slot < (n >> 1) ? slot : (3 * n / 2 - 1 - slot);
}

template <class MF, int IO, int N>
__device__ __forceinline__ void run_middle(float2* __restrict__ line,
                                           const MidDev& d, int utype,
                                           int sigA, int sigB,
                                           const void* kf, long long kfrow,
                                           int wave, int nwaves, int lane,
                                           float2* scratch) {
    constexpr int MT = N / 8;
    constexpr int KS = MF::ksteps(N);
    const int g = lane >> 4, x = lane & 15;
    typedef typename MF::AB AB;
    const AB* mf = (const AB*)d.mat_f;
    const AB* mi = (const AB*)d.mat_i;
    AB Af[MT][KS], Ai[MT][KS];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            Af[mt][ks] = mf[(mt * KS + ks) * 64 + lane];
            Ai[mt][ks] = mi[(mt * KS + ks) * 64 + lane];
        }
    const int Q = d.Q;
    const int LS = (utype == 2) ? Q : (Q >> 1);
    const int steps = (LS + 15) >> 4;
    for (int st = wave; st < steps; st += nwaves) {
        const int ls_raw = (st << 4) + x;
        const bool valid = ls_raw < LS;
        const int ls = valid ? ls_raw : LS - 1;
        const bool special = valid && utype == 0 && ls == 0;
        int qA = ls, qB, sA = 0, sB = 0;
        if (utype == 0) {
            qB = (ls == 0) ? (Q >> 1) : (Q - ls);
        } else {
            qB = Q - 1 - ls;
            if (utype == 2) sB = 1;
        }
        const int bA = d.digrev[qA], bB = d.digrev[qB];
        const int offA = sA * d.slab + bA * N;
        const int offB = sB * d.slab + bB * N;
        const long long pA = kfrow + (long long)sigA * d.slab + bA * N;
        const long long pB =
            kfrow + (long long)(sB ? sigB : sigA) * d.slab + bB * N;

        AB BA[KS], BB[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            BA[ks] = MF::gather(ks, g, N, [&](int nn) { return line[offA + nn]; });
            BB[ks] = MF::gather(ks, g, N, [&](int nn) { return line[offB + nn]; });
        }
        float2 za[MT][2], zb[MT][2];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            floatx4 ca = floatx4{0.f, 0.f, 0.f, 0.f};
            floatx4 cb = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                ca = MF::mma(Af[mt][ks], BA[ks], ca);
                cb = MF::mma(Af[mt][ks], BB[ks], cb);
            }
            za[mt][0] = make_float2(ca[0], ca[1]);
            za[mt][1] = make_float2(ca[2], ca[3]);
            zb[mt][0] = make_float2(cb[0], cb[1]);
            zb[mt][1] = make_float2(cb[2], cb[3]);
        }
        float2 ra[MT][2], rb[MT][2];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int slot = 8 * mt + 2 * g + e;
                const int k = mid_perm(slot, N);
                const int pm = (mt + MT / 2) % MT;
                float2 aa, ba, ab, bb;
                load_ab<IO>(kf, pA + k, aa, ba);
                load_ab<IO>(kf, pB + k, ab, bb);
                ra[mt][e] = pair_combine(aa, za[mt][e], ba, zb[pm][e]);
                rb[mt][e] = pair_combine(ab, zb[mt][e], bb, za[pm][e]);
                if (special) {
                    // column 1 holds q = Q/2, its own mirror block
                    rb[mt][e] = pair_combine(ab, zb[mt][e], bb, zb[pm][e]);
                }
            }
        if (special) {
            // column 0 holds q = 0: digit k pairs with -k (mod N), which
            // lives in another lane group; exchange through LDS.
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int e = 0; e < 2; ++e)
                    scratch[mid_perm(8 * mt + 2 * g + e, N)] = za[mt][e];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int k = mid_perm(8 * mt + 2 * g + e, N);
                    const float2 pz = scratch[(N - k) & (N - 1)];
                    float2 aa, ba;
                    load_ab<IO>(kf, pA + k, aa, ba);
                    ra[mt][e] = pair_combine(aa, za[mt][e], ba, pz);
                }
        }
        AB CA[KS], CB[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            CA[ks] = MF::template chain<MT>(ks, ra);
            CB[ks] = MF::template chain<MT>(ks, rb);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            floatx4 oa = floatx4{0.f, 0.f, 0.f, 0.f};
            floatx4 ob = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                oa = MF::mma(Ai[mt][ks], CA[ks], oa);
                ob = MF::mma(Ai[mt][ks], CB[ks], ob);
            }
            if (valid) {
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int slot = 8 * mt + 2 * g + e;
                    line[offA + slot] = make_float2(oa[2 * e], oa[2 * e + 1]);
                    line[offB + slot] = make_float2(ob[2 * e], ob[2 * e + 1]);
                }
            }
        }
    }
}

template <class MF, int IO>
__device__ __forceinline__ void dispatch_middle(const MidDev& d, float2* line,
                                                int utype, int sigA, int sigB,
                                                const void* kf,
                                                long long kfrow, int wave,
                                                int nwaves, int lane,
                                                float2* scratch) {
    if (d.n == 32)
        run_middle<MF, IO, 32>(line, d, utype, sigA, sigB, kf, kfrow, wave, nwaves, lane, scratch);
    else
        run_middle<MF, IO, 16>(line, d, utype, sigA, sigB, kf, kfrow, wave, nwaves, lane, scratch);
}

// ---------------------------------------------------------------------------
// I/O element conversions.  16-bit rows move as 16-byte vectors.
// ---------------------------------------------------------------------------
template <int IO>
__device__ __forceinline__ float io_to_f32(uint16_t v) {
    if (IO == IO_BF16) return __uint_as_float(((uint32_t)v) << 16);
    return (float)__builtin_bit_cast(_Float16, v);
}
template <int IO>
__device__ __forceinline__ uint16_t f32_to_io(float f) {
    if (IO == IO_BF16) return __builtin_bit_cast(uint16_t, (__bf16)f);
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Points move as 16-byte vectors: two fp32 points or four 16-bit ones.
template <int IO>
constexpr int pts_per_vec() { return IO == IO_F32 ? 2 : 4; }

// Vector j of a run of points: z[m] = u[2m] + i u[2m+1] from `src` (at
// u[2*m0]) into dst[pts_per_vec * j ...].  With a gate g (same layout as u,
// or null) the points are of u (.) g, each product formed in fp32 (exact
// for 16-bit inputs).
template <int IO>
__device__ __forceinline__ void load_vec(const void* src, const void* gsrc, float2* dst, int j) {
    if (IO == IO_F32) {
        float4 v = ((const float4*)src)[j];
        if (gsrc) {
            const float4 g = ((const float4*)gsrc)[j];
            v = make_float4(v.x * g.x, v.y * g.y, v.z * g.z, v.w * g.w);
        }
        dst[2 * j] = make_float2(v.x, v.y);
        dst[2 * j + 1] = make_float2(v.z, v.w);
    } else {
        const uint4 v = ((const uint4*)src)[j];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        float2 pt[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            pt[i] = make_float2(io_to_f32<IO>((uint16_t)(w[i] & 0xffffu)),
                                io_to_f32<IO>((uint16_t)(w[i] >> 16)));
        if (gsrc) {
            const uint4 gv = ((const uint4*)gsrc)[j];
            const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pt[i].x *= io_to_f32<IO>((uint16_t)(gw[i] & 0xffffu));
                pt[i].y *= io_to_f32<IO>((uint16_t)(gw[i] >> 16));
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[4 * j + i] = pt[i];
    }
}

// Vector j of a run of outputs: y[2m], y[2m+1] = Re, Im of src[m]; with a
// gate g (same layout as y, or null) each output is multiplied by g in fp32
// before the one rounding to the I/O type.
template <int IO>
__device__ __forceinline__ void store_vec(const float2* src, const void* gsrc, void* dst, int j) {
    if (IO == IO_F32) {
        const float2 a = src[2 * j], b = src[2 * j + 1];
        float4 r = make_float4(a.x, a.y, b.x, b.y);
        if (gsrc) {
            const float4 g = ((const float4*)gsrc)[j];
            r = make_float4(r.x * g.x, r.y * g.y, r.z * g.z, r.w * g.w);
        }
        ((float4*)dst)[j] = r;
    } else {
        float2 pt[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pt[i] = src[4 * j + i];
        if (gsrc) {
            const uint4 gv = ((const uint4*)gsrc)[j];
            const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pt[i].x *= io_to_f32<IO>((uint16_t)(gw[i] & 0xffffu));
                pt[i].y *= io_to_f32<IO>((uint16_t)(gw[i] >> 16));
            }
        }
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = (uint32_t)f32_to_io<IO>(pt[i].x) | ((uint32_t)f32_to_io<IO>(pt[i].y) << 16);
        ((uint4*)dst)[j] = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// A whole run of npts points with all threads of the workgroup.
template <int IO>
__device__ __forceinline__ void load_points(const void* src, const void* gsrc,
                                            float2* dst, int npts, int tid,
                                            int nthr) {
    for (int j = tid; j < npts / pts_per_vec<IO>(); j += nthr) load_vec<IO>(src, gsrc, dst, j);
}
template <int IO>
__device__ __forceinline__ void store_points(const float2* src, const void* gsrc,
                                             void* dst, int npts, int tid,
                                             int nthr) {
    for (int j = tid; j < npts / pts_per_vec<IO>(); j += nthr) store_vec<IO>(src, gsrc, dst, j);
}

template <int IO>
__device__ __forceinline__ const char* io_ptr(const void* base, long long elem) {
    return (const char*)base + elem * (IO == IO_F32 ? 4 : 2);
}
// the same for an optional gate (null stays null)
template <int IO>
__device__ __forceinline__ const char* gate_ptr(const void* base, long long elem) {
    return base ? io_ptr<IO>(base, elem) : nullptr;
}

// ---------------------------------------------------------------------------
// Fused path: one workgroup holds a whole row's M packed points in LDS.
// ---------------------------------------------------------------------------
template <class MF, int IO>
__global__ void __launch_bounds__(512) fused_kernel(FwdParams P) {
    extern __shared__ float2 smem[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
    float2* line = smem;
    float2* scratch = smem + P.M + wave * 32;
    for (long long row = blockIdx.x; row < P.rows; row += gridDim.x) {
        const int h = (int)(row % P.H);
        load_points<IO>(io_ptr<IO>(P.u, row * P.N), gate_ptr<IO>(P.w, row * P.N),
                        line, P.N >> 1, threadIdx.x, blockDim.x);
        __syncthreads();
        for (int i = 0; i < P.nst; ++i) {
            dispatch_stage<MF, false>(i == 0 && P.outer_half, P.st[i], line,
                                      P.M, 0, wave, nwaves, lane);
            __syncthreads();
        }
        dispatch_middle<MF, IO>(P.mid, line, 0, 0, 0, P.kf,
                                (long long)h * P.M, wave, nwaves, lane,
                                scratch);
        __syncthreads();
        for (int i = P.nst - 1; i >= 0; --i) {
            dispatch_stage<MF, true>(i == 0 && P.outer_half, P.st[i], line,
                                     P.M, 0, wave, nwaves, lane);
            __syncthreads();
        }
        store_points<IO>(line, gate_ptr<IO>(P.v, row * P.N),
                         (void*)io_ptr<IO>(P.y, row * P.N), P.N >> 1,
                         threadIdx.x, blockDim.x);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Multi-pass path (rows too long for one workgroup's LDS).
//  outer pass (forward): a tile of ct columns c2 of the [Qo][slab] view of
//    a row; the outer stages run over the Qo outer digits; result to the
//    fp32 workspace at the in-place positions.
//  inner pass: one unit (slab or mirrored slab pair) per workgroup; inner
//    stages, pairing with the spectrum, inverse inner stages; in place.
//  outer pass (inverse): inverse outer stages per column tile, then y.
// ---------------------------------------------------------------------------
template <class MF, int IO>
__global__ void __launch_bounds__(512) outer_fwd_kernel(FwdParams P) {
    extern __shared__ float2 smem[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
    const long long row = blockIdx.x;
    const int c0 = blockIdx.y * P.ct;
    const int slab = P.M / P.Qo;
    float2* line = smem;
    // the nonzero half of the outer digits: n_o < Qo/2 (all Qo digits for
    // a plan at FFT size N: no zero half), every thread over (digit,
    // vector) pairs -- a tile's run per digit is only ct points
    const int nload = P.outer_half ? (P.Qo >> 1) : P.Qo;
    {
        const int per = P.ct / pts_per_vec<IO>();
        for (int i = threadIdx.x; i < nload * per; i += blockDim.x) {
            const int no = i / per, j = i - no * per;
            const long long e0 = row * P.N + 2LL * ((long long)no * slab + c0);
            load_vec<IO>(io_ptr<IO>(P.u, e0), gate_ptr<IO>(P.w, e0), line + no * P.ct, j);
        }
    }
    __syncthreads();
    for (int i = 0; i < P.nst; ++i) {
        dispatch_stage<MF, false>(i == 0 && P.outer_half, P.st[i], line, P.Qo * P.ct, c0,
                                  wave, nwaves, lane);
        __syncthreads();
    }
    float2* ws = P.ws + row * (long long)P.M;
    const int per = P.ct >> 1;   // float4 (two points) per outer digit
    for (int j = threadIdx.x; j < P.Qo * per; j += blockDim.x) {
        const int no = j / per, c = (j - no * per) * 2;
        const float2 a = line[no * P.ct + c], b = line[no * P.ct + c + 1];
        *(float4*)(ws + (long long)no * slab + c0 + c) = make_float4(a.x, a.y, b.x, b.y);
    }
}

template <class MF, int IO>
__global__ void __launch_bounds__(512) inner_kernel(FwdParams P) {
    extern __shared__ float2 smem[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
    const long long row = blockIdx.x;
    const int unit = blockIdx.y;
    const int h = (int)(row % P.H);
    const int slab = P.M / P.Qo;
    const int utype = unit == 0 ? 0 : (unit == 1 ? 1 : 2);
    const int qoA = unit == 0 ? 0 : (unit == 1 ? (P.Qo >> 1) : unit - 1);
    const int sigA = P.digrev_o[qoA];
    const int sigB = utype == 2 ? P.digrev_o[P.Qo - qoA] : sigA;
    const int nslab = utype == 2 ? 2 : 1;
    float2* line = smem;
    float2* scratch = smem + 2 * slab + wave * 32;
    float2* ws = P.ws + row * (long long)P.M;
    for (int s = 0; s < nslab; ++s) {
        const float4* src = (const float4*)(ws + (long long)(s ? sigB : sigA) * slab);
        for (int j = threadIdx.x; j < (slab >> 1); j += blockDim.x) {
            const float4 v = src[j];
            line[s * slab + 2 * j] = make_float2(v.x, v.y);
            line[s * slab + 2 * j + 1] = make_float2(v.z, v.w);
        }
    }
    __syncthreads();
    const int len = nslab * slab;
    for (int i = 0; i < P.nst; ++i) {
        dispatch_stage<MF, false>(false, P.st[i], line, len, 0, wave, nwaves, lane);
        __syncthreads();
    }
    dispatch_middle<MF, IO>(P.mid, line, utype, sigA, sigB, P.kf,
                            (long long)h * P.M, wave, nwaves, lane, scratch);
    __syncthreads();
    for (int i = P.nst - 1; i >= 0; --i) {
        dispatch_stage<MF, true>(false, P.st[i], line, len, 0, wave, nwaves, lane);
        __syncthreads();
    }
    for (int s = 0; s < nslab; ++s) {
        float4* dst = (float4*)(ws + (long long)(s ? sigB : sigA) * slab);
        for (int j = threadIdx.x; j < (slab >> 1); j += blockDim.x) {
            const float2 a = line[s * slab + 2 * j], b = line[s * slab + 2 * j + 1];
            dst[j] = make_float4(a.x, a.y, b.x, b.y);
        }
    }
}

template <class MF, int IO>
__global__ void __launch_bounds__(512) outer_inv_kernel(FwdParams P) {
    extern __shared__ float2 smem[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
    const long long row = blockIdx.x;
    const int c0 = blockIdx.y * P.ct;
    const int slab = P.M / P.Qo;
    float2* line = smem;
    const float2* ws = P.ws + row * (long long)P.M;
    const int per = P.ct >> 1;
    for (int j = threadIdx.x; j < P.Qo * per; j += blockDim.x) {
        const int no = j / per, c = (j - no * per) * 2;
        const float4 v = *(const float4*)(ws + (long long)no * slab + c0 + c);
        line[no * P.ct + c] = make_float2(v.x, v.y);
        line[no * P.ct + c + 1] = make_float2(v.z, v.w);
    }
    __syncthreads();
    for (int i = P.nst - 1; i >= 0; --i) {
        dispatch_stage<MF, true>(i == 0 && P.outer_half, P.st[i], line, P.Qo * P.ct, c0,
                                 wave, nwaves, lane);
        __syncthreads();
    }
    {
        const int per = P.ct / pts_per_vec<IO>();
        const int nstore = P.outer_half ? (P.Qo >> 1) : P.Qo;
        for (int i = threadIdx.x; i < nstore * per; i += blockDim.x) {
            const int no = i / per, j = i - no * per;
            const long long e0 = row * P.N + 2LL * ((long long)no * slab + c0);
            store_vec<IO>(line + no * P.ct, gate_ptr<IO>(P.v, e0), (void*)io_ptr<IO>(P.y, e0), j);
        }
    }
}

// ---------------------------------------------------------------------------
// Kernel gradient of the causal convolution,
//   dk[h][j] = sum_b sum_{t>=j} dy[b,h,t] u[b,h,t-j],
// whose 2N-point spectrum is G = sum_b conj(U_b) . DY_b (page "FlashFFTConv:
// Efficient Convolutions for Long Sequences with Tensor Cores", section 3:
// the backward pass of an FFT convolution multiplies by conjugate spectra,
// and the input spectra are recomputed instead of stored).
// In the packed form (z = u_even + i u_odd, Z its M-point DFT), bins k and
// -k give E = (Z[k] + conj Z[-k]) / 2, O = (Z[k] - conj Z[-k]) / (2i) and
// U[k] = E + w O, U[k + M] = E - w O with w = W_2N^k; the real result's
// packed spectrum is Z_g[k] = (G[k] + G[k+M]) / 2 + i conj(w) (G[k] - G[k+M]) / 2.
// Z_g is linear in G, so it is accumulated over the batch directly, in the
// registers of the lane that owns the bin pair (the lane slots of the
// innermost stage, which already hold bins k and -k together), and then
// goes through the inverse stages like a product spectrum.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float2 kg_bin(float2 a, float2 ap, float2 d, float2 dp,
                                         float2 w) {
    const float2 c = make_float2(ap.x, -ap.y), f = make_float2(dp.x, -dp.y);
    // E = (Z + conj Z-) / 2, O = -i (Z - conj Z-) / 2
    const float2 eu = make_float2(0.5f * (a.x + c.x), 0.5f * (a.y + c.y));
    const float2 ou = make_float2(0.5f * (a.y - c.y), -0.5f * (a.x - c.x));
    const float2 ed = make_float2(0.5f * (d.x + f.x), 0.5f * (d.y + f.y));
    const float2 od = make_float2(0.5f * (d.y - f.y), -0.5f * (d.x - f.x));
    const float2 wu = cmul(w, ou), wd = cmul(w, od);
    const float2 up = make_float2(eu.x + wu.x, eu.y + wu.y);
    const float2 um = make_float2(eu.x - wu.x, eu.y - wu.y);
    const float2 dpl = make_float2(ed.x + wd.x, ed.y + wd.y);
    const float2 dmi = make_float2(ed.x - wd.x, ed.y - wd.y);
    // G+ = conj(U+) DY+, G- = conj(U-) DY-
    const float2 gp = cmulc(dpl, up), gm = cmulc(dmi, um);
    const float2 eg = make_float2(0.5f * (gp.x + gm.x), 0.5f * (gp.y + gm.y));
    const float2 og = cmulc(make_float2(0.5f * (gp.x - gm.x), 0.5f * (gp.y - gm.y)), w);
    return make_float2(eg.x - og.y, eg.y + og.x);
}

// W_2N^bin = exp(-i pi bin / M)
__device__ __forceinline__ float2 kg_w(int bin, int M) {
    float sn, cs;
    sincospif(-(float)bin / (float)M, &sn, &cs);
    return make_float2(cs, sn);
}

// Lane-slot geometry of the innermost stage (as in run_middle).
struct KgSlot {
    int ls, qA, qB, offA, offB;
    bool valid, special;
};
__device__ __forceinline__ KgSlot kg_slot(const MidDev& d, int utype, int st, int x) {
    const int Q = d.Q;
    const int LS = (utype == 2) ? Q : (Q >> 1);
    KgSlot k;
    const int ls_raw = (st << 4) + x;
    k.valid = ls_raw < LS;
    k.ls = k.valid ? ls_raw : LS - 1;
    k.special = k.valid && utype == 0 && k.ls == 0;
    k.qA = k.ls;
    int sB = 0;
    if (utype == 0) {
        k.qB = (k.ls == 0) ? (Q >> 1) : (Q - k.ls);
    } else {
        k.qB = Q - 1 - k.ls;
        if (utype == 2) sB = 1;
    }
    k.offA = d.digrev[k.qA] * d.n;
    k.offB = sB * d.slab + d.digrev[k.qB] * d.n;
    return k;
}

// Forward innermost stage of the u line and the dy line, and the
// accumulation of Z_g for every bin of this wave's lane slots.  Bins:
// k = ko + Qo (q + Q digit) (ko the outer part of the slab, Qo the number
// of slabs; 0 and 1 on a fused row).
template <class MF, int N, int SPW>
__device__ __forceinline__ void kgrad_middle(const float2* __restrict__ lu,
                                             const float2* __restrict__ ld,
                                             const MidDev& d, int utype, int koA,
                                             int koB, int Qo, int M, int wave,
                                             int nwaves, int lane, float2* scru,
                                             float2* scrd,
                                             float2 (&accA)[SPW][N / 8][2],
                                             float2 (&accB)[SPW][N / 8][2]) {
    constexpr int MT = N / 8;
    constexpr int KS = MF::ksteps(N);
    const int g = lane >> 4, x = lane & 15;
    typedef typename MF::AB AB;
    const AB* mf = (const AB*)d.mat_f;
    AB Af[MT][KS];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) Af[mt][ks] = mf[(mt * KS + ks) * 64 + lane];
    const int Q = d.Q;
    const int LS = (utype == 2) ? Q : (Q >> 1);
    const int steps = (LS + 15) >> 4;
#pragma unroll
    for (int sp = 0; sp < SPW; ++sp) {
        const int st = wave + sp * nwaves;
        if (st >= steps) break;
        const KgSlot ks_ = kg_slot(d, utype, st, x);
        float2 z[4][MT][2];   // u of A, u of B, dy of A, dy of B
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const float2* src = (v & 2) ? ld : lu;
            const int off = (v & 1) ? ks_.offB : ks_.offA;
            AB Bv[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                Bv[ks] = MF::gather(ks, g, N, [&](int nn) { return src[off + nn]; });
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                floatx4 c = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) c = MF::mma(Af[mt][ks], Bv[ks], c);
                z[v][mt][0] = make_float2(c[0], c[1]);
                z[v][mt][1] = make_float2(c[2], c[3]);
            }
        }
        if (ks_.special) {
            // block q = 0 pairs digit k with -k (mod N), held by another
            // lane group: exchange the u and dy values through LDS
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int k = mid_perm(8 * mt + 2 * g + e, N);
                    scru[k] = z[0][mt][e];
                    scrd[k] = z[2][mt][e];
                }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int k = mid_perm(8 * mt + 2 * g + e, N);
                const int pm = (mt + MT / 2) % MT;
                const float2 wA = kg_w(koA + Qo * (ks_.qA + Q * k), M);
                const float2 wB = kg_w(koB + Qo * (ks_.qB + Q * k), M);
                float2 cA, cB;
                if (ks_.special) {
                    const int km = (N - k) & (N - 1);
                    cA = kg_bin(z[0][mt][e], scru[km], z[2][mt][e], scrd[km], wA);
                    // block q = Q/2 is its own mirror block
                    cB = kg_bin(z[1][mt][e], z[1][pm][e], z[3][mt][e], z[3][pm][e], wB);
                } else {
                    cA = kg_bin(z[0][mt][e], z[1][pm][e], z[2][mt][e], z[3][pm][e], wA);
                    cB = kg_bin(z[1][mt][e], z[0][pm][e], z[3][mt][e], z[2][pm][e], wB);
                }
                accA[sp][mt][e].x += cA.x;
                accA[sp][mt][e].y += cA.y;
                accB[sp][mt][e].x += cB.x;
                accB[sp][mt][e].y += cB.y;
            }
    }
}

// Inverse innermost stage of the accumulated spectrum (times `pre`), into
// the line at the lane slots' positions.
template <class MF, int N, int SPW>
__device__ __forceinline__ void kgrad_final(float2* __restrict__ line, const MidDev& d,
                                            int utype, int wave, int nwaves, int lane,
                                            float pre, float2 (&accA)[SPW][N / 8][2],
                                            float2 (&accB)[SPW][N / 8][2]) {
    constexpr int MT = N / 8;
    constexpr int KS = MF::ksteps(N);
    const int g = lane >> 4, x = lane & 15;
    typedef typename MF::AB AB;
    const AB* mi = (const AB*)d.mat_i;
    const int Q = d.Q;
    const int LS = (utype == 2) ? Q : (Q >> 1);
    const int steps = (LS + 15) >> 4;
#pragma unroll
    for (int sp = 0; sp < SPW; ++sp) {
        const int st = wave + sp * nwaves;
        if (st >= steps) break;
        const KgSlot ks_ = kg_slot(d, utype, st, x);
        float2 ra[MT][2], rb[MT][2];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                ra[mt][e] = make_float2(accA[sp][mt][e].x * pre, accA[sp][mt][e].y * pre);
                rb[mt][e] = make_float2(accB[sp][mt][e].x * pre, accB[sp][mt][e].y * pre);
            }
        AB CA[KS], CB[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            CA[ks] = MF::template chain<MT>(ks, ra);
            CB[ks] = MF::template chain<MT>(ks, rb);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            floatx4 oa = floatx4{0.f, 0.f, 0.f, 0.f};
            floatx4 ob = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const AB a = mi[(mt * KS + ks) * 64 + lane];
                oa = MF::mma(a, CA[ks], oa);
                ob = MF::mma(a, CB[ks], ob);
            }
            if (ks_.valid) {
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int slot = 8 * mt + 2 * g + e;
                    line[ks_.offA + slot] = make_float2(oa[2 * e], oa[2 * e + 1]);
                    line[ks_.offB + slot] = make_float2(ob[2 * e], ob[2 * e + 1]);
                }
            }
        }
    }
}

// lane-slot steps per wave (checked by the host): two for 16-point
// innermost stages, one for 32-point ones (registers)
constexpr int kg_spw(int nm) { return nm == 32 ? 1 : 2; }

// Fused: one workgroup per (channel, slice of the batch), looping over its
// rows; two lines (u and dy) in LDS.  Writes `post` x the inverse of the
// accumulated spectrum to dk (one slice) or to the slice's partial row
// (several slices, summed by kgrad_reduce_kernel: the inverse is linear).
template <class MF, int IO, int NM>
__global__ void __launch_bounds__(512) kgrad_fused_kernel(KgradParams P) {
    extern __shared__ float2 smem[];
    const FwdParams& F = P.f;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
    float2* la = smem;
    float2* lb = smem + F.M;
    float2* scr = smem + 2 * F.M + wave * 64;
    const int h = blockIdx.x;
    const int b0 = (int)(((long long)P.B * blockIdx.y) / gridDim.y);
    const int b1 = (int)(((long long)P.B * (blockIdx.y + 1)) / gridDim.y);
    constexpr int SPW = kg_spw(NM);
    float2 accA[SPW][NM / 8][2], accB[SPW][NM / 8][2];
#pragma unroll
    for (int sp = 0; sp < SPW; ++sp)
#pragma unroll
        for (int mt = 0; mt < NM / 8; ++mt)
#pragma unroll
            for (int e = 0; e < 2; ++e) accA[sp][mt][e] = accB[sp][mt][e] = make_float2(0.f, 0.f);
    for (int b = b0; b < b1; ++b) {
        const long long row = (long long)b * P.H + h;
        load_points<IO>(io_ptr<IO>(P.u, row * F.N), nullptr, la, F.N >> 1, threadIdx.x, blockDim.x);
        load_points<IO>(io_ptr<IO>(P.dy, row * F.N), nullptr, lb, F.N >> 1, threadIdx.x, blockDim.x);
        __syncthreads();
        for (int i = 0; i < F.nst; ++i) {
            dispatch_stage<MF, false>(i == 0 && F.outer_half, F.st[i], la, F.M, 0, wave, nwaves, lane);
            dispatch_stage<MF, false>(i == 0 && F.outer_half, F.st[i], lb, F.M, 0, wave, nwaves, lane);
            __syncthreads();
        }
        kgrad_middle<MF, NM, SPW>(la, lb, F.mid, 0, 0, 0, 1, F.M, wave, nwaves, lane, scr,
                                     scr + 32, accA, accB);
        __syncthreads();
    }
    const float pre = rsqrtf((float)F.M);
    kgrad_final<MF, NM, SPW>(la, F.mid, 0, wave, nwaves, lane, pre, accA, accB);
    __syncthreads();
    for (int i = F.nst - 1; i >= 0; --i) {
        dispatch_stage<MF, true>(i == 0 && F.outer_half, F.st[i], la, F.M, 0, wave, nwaves, lane);
        __syncthreads();
    }
    const float post = P.scale;
    float* dst = gridDim.y > 1 ? (float*)P.wsg + (long long)blockIdx.y * P.H * F.N : P.dk;
    float2* o = (float2*)(dst + (long long)h * F.N);
    for (int j = threadIdx.x; j < (F.N >> 1); j += blockDim.x)
        o[j] = make_float2(la[j].x * post, la[j].y * post);
}

// dk = the sum of the slices' partial rows, [nsplit][H * N] -> [H * N]
__global__ void kgrad_reduce_kernel(const float4* __restrict__ part, float4* __restrict__ dk,
                                    long long n4, int nsplit) {
    for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n4;
         i += (long long)gridDim.x * blockDim.x) {
        float4 a = part[i];
        for (int sidx = 1; sidx < nsplit; ++sidx) {
            const float4 b = part[(long long)sidx * n4 + i];
            a.x += b.x;
            a.y += b.y;
            a.z += b.z;
            a.w += b.w;
        }
        dk[i] = a;
    }
}

// Multi-pass inner pass: one workgroup per (channel, unit of slabs), looping
// over the batch; the outer-transformed rows of u and dy come from the
// workspace, the result (inverse inner stages done) goes to the channel's
// workspace row for the outer inverse pass.
template <class MF, int IO, int NM>
__global__ void __launch_bounds__(512) kgrad_inner_kernel(KgradParams P) {
    extern __shared__ float2 smem[];
    const FwdParams& F = P.f;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
    const int h = blockIdx.x, unit = blockIdx.y;
    const int slab = F.M / F.Qo;
    const int utype = unit == 0 ? 0 : (unit == 1 ? 1 : 2);
    const int qoA = unit == 0 ? 0 : (unit == 1 ? (F.Qo >> 1) : unit - 1);
    const int sigA = F.digrev_o[qoA];
    const int sigB = utype == 2 ? F.digrev_o[F.Qo - qoA] : sigA;
    const int nslab = utype == 2 ? 2 : 1;
    const int koA = qoA, koB = utype == 2 ? F.Qo - qoA : qoA;
    const int len = nslab * slab;
    float2* la = smem;
    float2* lb = smem + 2 * slab;
    float2* scr = smem + 4 * slab + wave * 64;
    constexpr int SPW = kg_spw(NM);
    float2 accA[SPW][NM / 8][2], accB[SPW][NM / 8][2];
#pragma unroll
    for (int sp = 0; sp < SPW; ++sp)
#pragma unroll
        for (int mt = 0; mt < NM / 8; ++mt)
#pragma unroll
            for (int e = 0; e < 2; ++e) accA[sp][mt][e] = accB[sp][mt][e] = make_float2(0.f, 0.f);
    for (int b = 0; b < P.B; ++b) {
        const long long row = (long long)b * P.H + h;
        for (int sl = 0; sl < nslab; ++sl) {
            const long long off = row * (long long)F.M + (long long)(sl ? sigB : sigA) * slab;
            const float4* su = (const float4*)(P.wsu + off);
            const float4* sd = (const float4*)(P.wsd + off);
            for (int j = threadIdx.x; j < (slab >> 1); j += blockDim.x) {
                const float4 a = su[j], c = sd[j];
                la[sl * slab + 2 * j] = make_float2(a.x, a.y);
                la[sl * slab + 2 * j + 1] = make_float2(a.z, a.w);
                lb[sl * slab + 2 * j] = make_float2(c.x, c.y);
                lb[sl * slab + 2 * j + 1] = make_float2(c.z, c.w);
            }
        }
        __syncthreads();
        for (int i = 0; i < F.nst; ++i) {
            dispatch_stage<MF, false>(false, F.st[i], la, len, 0, wave, nwaves, lane);
            dispatch_stage<MF, false>(false, F.st[i], lb, len, 0, wave, nwaves, lane);
            __syncthreads();
        }
        kgrad_middle<MF, NM, SPW>(la, lb, F.mid, utype, koA, koB, F.Qo, F.M, wave, nwaves,
                                     lane, scr, scr + 32, accA, accB);
        __syncthreads();
    }
    const float pre = rsqrtf((float)F.M);
    kgrad_final<MF, NM, SPW>(la, F.mid, utype, wave, nwaves, lane, pre, accA, accB);
    __syncthreads();
    for (int i = F.nst - 1; i >= 0; --i) {
        dispatch_stage<MF, true>(false, F.st[i], la, len, 0, wave, nwaves, lane);
        __syncthreads();
    }
    for (int sl = 0; sl < nslab; ++sl) {
        float4* dst = (float4*)(P.wsg + (long long)h * F.M + (long long)(sl ? sigB : sigA) * slab);
        for (int j = threadIdx.x; j < (slab >> 1); j += blockDim.x) {
            const float2 a = la[sl * slab + 2 * j], c = la[sl * slab + 2 * j + 1];
            dst[j] = make_float4(a.x, a.y, c.x, c.y);
        }
    }
}

// x *= a; a = 0 writes zeros (whatever x held)
__global__ void scale_f32_kernel(float* x, long long n, float a) {
    for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n;
         i += (long long)gridDim.x * blockDim.x)
        x[i] = a == 0.f ? 0.f : x[i] * a;
}

// ---------------------------------------------------------------------------
// Kernel spectrum (untimed, once per channel): an accurate fp32 radix-2
// Stockham FFT of the zero-padded kernel, then alpha/beta per packed bin.
// ---------------------------------------------------------------------------
// The 2N-periodic kernel c whose circular convolution with the zero-padded
// input gives the operator of `kind` on outputs t < N:
//   0 causal            c[t] = k[t] (t < N), 0 above
//   1 causal adjoint    c[0] = k[0], c[2N - j] = k[j] (0 < j < N), 0 else
//                       (y[s] = sum_{t>=s} u[t] k[t-s])
//   2 circular          c[t] = k[t mod N]  (y[t] = sum_s u[s] k[(t-s) mod N])
//   3 circular adjoint  c[t] = k[(-t) mod N]
// L = 2N: the 2N-periodic kernel of each operator kind (the causal
// transform size); L = N: the N-periodic kernel of the circular kinds
// (k itself, or k reversed: k[-t mod N]) for plans at FFT size N.
__global__ void kpad_kernel(const float* __restrict__ k, float2* __restrict__ X,
                            int hcount, int N, int L, int kind) {
    const long long total = (long long)hcount * L;
    for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < total;
         i += (long long)gridDim.x * blockDim.x) {
        const long long h = i / L;
        const int t = (int)(i - h * L);
        const float* kr = k + h * N;
        float v = 0.f;
        if (L == N) {
            v = kr[kind == 2 ? t : ((N - t) & (N - 1))];
        } else if (kind == 0) {
            if (t < N) v = kr[t];
        } else if (kind == 1) {
            if (t == 0) v = kr[0];
            else if (t > N) v = kr[2 * N - t];
        } else if (kind == 2) {
            v = kr[t & (N - 1)];
        } else {
            const int m = t & (N - 1);
            v = kr[m == 0 ? 0 : N - m];
        }
        X[i] = make_float2(v, 0.f);
    }
}

// Band limit of kernel spectra: X[h][f] = 0 where min(f, L - f) > F.
__global__ void band_limit_kernel(float2* __restrict__ X, int hcount, int L, int F) {
    const long long total = (long long)hcount * L;
    for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < total;
         i += (long long)gridDim.x * blockDim.x) {
        const int f = (int)(i % L);
        const int dist = f < L - f ? f : L - f;
        if (dist > F) X[i] = make_float2(0.f, 0.f);
    }
}

// One radix-2 Stockham pass: sub-transforms of length Ns are combined into
// length 2Ns; natural-order output after log2(L) passes.
__global__ void stockham_kernel(const float2* __restrict__ in,
                                float2* __restrict__ out, int hcount, int L,
                                int Ns) {
    const long long half = L >> 1;
    const long long total = hcount * half;
    for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < total;
         i += (long long)gridDim.x * blockDim.x) {
        const long long h = i / half, j = i - h * half;
        const float2* a = in + h * L;
        float2* o = out + h * L;
        const int k = (int)(j % Ns);
        double sn, cs;
        sincospi(-(double)k / (double)Ns, &sn, &cs);
        const float2 u0 = a[j];
        const float2 u1 = cmul(a[j + half], make_float2((float)cs, (float)sn));
        const long long dst = (j / Ns) * 2 * Ns + k;
        o[dst] = make_float2(u0.x + u1.x, u0.y + u1.y);
        o[dst + Ns] = make_float2(u0.x - u1.x, u0.y - u1.y);
    }
}

// alpha_k = ((1 - s) K[k] + (1 + s) K[k+M]) / 2,  beta_k = i c (K[k] - K[k+M]) / 2
// with s + i c = e^{i(pi/2 - 2 pi k/L)}... i.e. s = sin(2 pi k/L), c = cos(2 pi k/L);
// stored at the in-place position of bin k.
template <int IO>
__global__ void alphabeta_kernel(SpecParams P) {
    const long long total = (long long)P.hcount * P.M;
    for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < total;
         i += (long long)gridDim.x * blockDim.x) {
        const long long hl = i / P.M;
        const int pos = (int)(i - hl * P.M);
        // bin of position: digits k_1..k_p, most significant first
        int rem = pos, S = P.M, mul = 1, kb = 0;
        for (int f = 0; f < P.p; ++f) {
            const int n = P.factors[f];
            const int s = S / n;
            const int dgt = rem / s;
            rem -= dgt * s;
            kb += dgt * mul;
            mul *= n;
            S = s;
        }
        const float2* X = P.X + hl * P.L;
        const float2 K1 = X[kb], K2 = X[kb + P.M];
        double sn, cs;
        sincospi(2.0 * (double)kb / (double)P.L, &sn, &cs);
        const float s = (float)sn, c = (float)cs;
        const float2 al = make_float2(0.5f * ((1.f - s) * K1.x + (1.f + s) * K2.x),
                                      0.5f * ((1.f - s) * K1.y + (1.f + s) * K2.y));
        const float2 dlt = make_float2(K1.x - K2.x, K1.y - K2.y);
        const float2 be = make_float2(-0.5f * c * dlt.y, 0.5f * c * dlt.x);
        const long long o = (long long)(P.h0 + hl) * P.M + pos;
        if (IO == IO_F32) {
            ((float4*)P.kf)[o] = make_float4(al.x, al.y, be.x, be.y);
        } else {
            _Float16 hv[4] = {(_Float16)al.x, (_Float16)al.y, (_Float16)be.x, (_Float16)be.y};
            ((uint2*)P.kf)[o] = *(const uint2*)hv;
        }
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <class K>
static hipError_t set_lds(K kern, int bytes) {
    if (bytes <= 64 * 1024) return hipSuccess;
    return hipFuncSetAttribute((const void*)kern,
                               hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

#define FFTCONV_LAUNCH(KERNEL, GRID)                                          \
    do {                                                                      \
        hipError_t e_;                                                        \
        const dim3 blk(p.threads);                                            \
        switch (io) {                                                         \
        case IO_F32:                                                          \
            e_ = set_lds(KERNEL<MfF32, IO_F32>, lds);                         \
            if (e_ != hipSuccess) return e_;                                  \
            hipLaunchKernelGGL((KERNEL<MfF32, IO_F32>), GRID, blk, lds, s, p); \
            break;                                                            \
        case IO_F16:                                                          \
            e_ = set_lds(KERNEL<MfF16, IO_F16>, lds);                         \
            if (e_ != hipSuccess) return e_;                                  \
            hipLaunchKernelGGL((KERNEL<MfF16, IO_F16>), GRID, blk, lds, s, p); \
            break;                                                            \
        default:                                                              \
            e_ = set_lds(KERNEL<MfF16, IO_BF16>, lds);                        \
            if (e_ != hipSuccess) return e_;                                  \
            hipLaunchKernelGGL((KERNEL<MfF16, IO_BF16>), GRID, blk, lds, s, p); \
            break;                                                            \
        }                                                                     \
        return hipGetLastError();                                             \
    } while (0)

hipError_t launch_fused(int io, const FwdParams& p, int lds, hipStream_t s) {
    FFTCONV_LAUNCH(fused_kernel, dim3((unsigned)p.rows));
}

hipError_t launch_outer_fwd(int io, const FwdParams& p, int lds, hipStream_t s) {
    const int slab = p.M / p.Qo;
    FFTCONV_LAUNCH(outer_fwd_kernel, dim3((unsigned)p.rows, slab / p.ct));
}

hipError_t launch_inner(int io, const FwdParams& p, int lds, hipStream_t s) {
    FFTCONV_LAUNCH(inner_kernel, dim3((unsigned)p.rows, p.nunits));
}

hipError_t launch_outer_inv(int io, const FwdParams& p, int lds, hipStream_t s) {
    const int slab = p.M / p.Qo;
    FFTCONV_LAUNCH(outer_inv_kernel, dim3((unsigned)p.rows, slab / p.ct));
}

hipError_t launch_kpad(const float* k, float2* X, int hcount, int N, int L, int kind,
                       hipStream_t s) {
    if (L != N && L != 2 * N) return hipErrorInvalidValue;
    if (L == N && kind != 2 && kind != 3) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kpad_kernel, dim3(1024), dim3(256), 0, s, k, X, hcount, N, L, kind);
    return hipGetLastError();
}

__device__ __forceinline__ bool block_zero(long long k, int M, int P, int a, int d) {
    const long long kin = k / P;
    const int kout = (int)(k - kin * P);
    const int kb = (int)((kin * 32 * P) / M);
    if (kb >= 16 - a / 2 && kb < 16 + a / 2) return true;
    // 0 < |kout - P/2| <= d/2, or kout = P/2 when d is odd
    const int twice = 2 * kout - P;
    const int dist2 = twice < 0 ? -twice : twice;
    if (dist2 > 0 && dist2 <= 2 * (d / 2)) return true;
    return (d & 1) && dist2 == 0;
}

__global__ void block_mask_kernel(float2* __restrict__ X, int hcount, int L, int M, int P,
                                  int a, int d) {
    const long long total = (long long)hcount * L;
    for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < total;
         i += (long long)gridDim.x * blockDim.x) {
        const long long f = i % L;
        const long long k = f % M, km = (M - k) % M;
        if (block_zero(k, M, P, a, d) || block_zero(km, M, P, a, d)) X[i] = make_float2(0.f, 0.f);
    }
}

hipError_t launch_block_mask(float2* X, int hcount, int L, int M, int P, int a, int d,
                             hipStream_t s) {
    hipLaunchKernelGGL(block_mask_kernel, dim3(1024), dim3(256), 0, s, X, hcount, L, M, P, a, d);
    return hipGetLastError();
}

// Multi-pass workspace rows hold, per outer digit k_o, a slab of 4096 f16
// complex words at slab position sigma(k_o) (the column passes' digit
// order); zero the slabs of the units q >= q_from.
__global__ void mp_zero_units_kernel(uint4* __restrict__ ws, long long rows, int M, int Po,
                                     int P1, int P2, int q_from) {
    const int per_slab = 4096 / 4;   // uint4 per slab
    const int nq = Po / 2 - q_from;
    const long long total = rows * (long long)nq * 2 * per_slab;
    for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < total;
         i += (long long)gridDim.x * blockDim.x) {
        const int w = (int)(i % per_slab);
        long long rest = i / per_slab;
        const int side = (int)(rest & 1);
        rest >>= 1;
        const int q = q_from + (int)(rest % nq);
        const long long r = rest / nq;
        const int ko = side ? Po - q : q;
        const int slab = (ko % P1) * P2 + ko / P1;
        ws[(r * M + (long long)slab * 4096) / 4 + w] = make_uint4(0u, 0u, 0u, 0u);
    }
}

hipError_t launch_mp_zero_units(void* ws, long long rows, int M, int Po, int P1, int P2,
                                int q_from, hipStream_t s) {
    if (q_from >= Po / 2) return hipSuccess;
    hipLaunchKernelGGL(mp_zero_units_kernel, dim3(2048), dim3(256), 0, s, (uint4*)ws, rows, M,
                       Po, P1, P2, q_from);
    return hipGetLastError();
}

hipError_t launch_band_limit(float2* X, int hcount, int L, int F, hipStream_t s) {
    hipLaunchKernelGGL(band_limit_kernel, dim3(1024), dim3(256), 0, s, X, hcount, L, F);
    return hipGetLastError();
}

hipError_t launch_stockham(const float2* in, float2* out, int hcount, int L,
                           int Ns, hipStream_t s) {
    hipLaunchKernelGGL(stockham_kernel, dim3(2048), dim3(256), 0, s, in, out,
                       hcount, L, Ns);
    return hipGetLastError();
}

hipError_t launch_alphabeta(int io, const SpecParams& p, hipStream_t s) {
    if (io == IO_F32)
        hipLaunchKernelGGL(alphabeta_kernel<IO_F32>, dim3(2048), dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL(alphabeta_kernel<IO_F16>, dim3(2048), dim3(256), 0, s, p);
    return hipGetLastError();
}


#define FFTCONV_KG_LAUNCH(KERNEL, GRID)                                                  \
    do {                                                                                 \
        const dim3 blk(p.f.threads), grid = (GRID);                                      \
        hipError_t e_;                                                                   \
        if (p.f.mid.n != 16 && p.f.mid.n != 32) return hipErrorInvalidValue;           \
        switch (io * 2 + (p.f.mid.n == 32 ? 1 : 0)) {                                    \
        case IO_F32 * 2:                                                                 \
            e_ = set_lds(KERNEL<MfF32, IO_F32, 16>, lds);                                \
            if (e_ != hipSuccess) return e_;                                             \
            hipLaunchKernelGGL((KERNEL<MfF32, IO_F32, 16>), grid, blk, lds, s, p);       \
            break;                                                                       \
        case IO_F32 * 2 + 1:                                                             \
            e_ = set_lds(KERNEL<MfF32, IO_F32, 32>, lds);                                \
            if (e_ != hipSuccess) return e_;                                             \
            hipLaunchKernelGGL((KERNEL<MfF32, IO_F32, 32>), grid, blk, lds, s, p);       \
            break;                                                                       \
        case IO_F16 * 2:                                                                 \
            e_ = set_lds(KERNEL<MfF16, IO_F16, 16>, lds);                                \
            if (e_ != hipSuccess) return e_;                                             \
            hipLaunchKernelGGL((KERNEL<MfF16, IO_F16, 16>), grid, blk, lds, s, p);       \
            break;                                                                       \
        case IO_F16 * 2 + 1:                                                             \
            e_ = set_lds(KERNEL<MfF16, IO_F16, 32>, lds);                                \
            if (e_ != hipSuccess) return e_;                                             \
            hipLaunchKernelGGL((KERNEL<MfF16, IO_F16, 32>), grid, blk, lds, s, p);       \
            break;                                                                       \
        case IO_BF16 * 2:                                                                \
            e_ = set_lds(KERNEL<MfF16, IO_BF16, 16>, lds);                               \
            if (e_ != hipSuccess) return e_;                                             \
            hipLaunchKernelGGL((KERNEL<MfF16, IO_BF16, 16>), grid, blk, lds, s, p);      \
            break;                                                                       \
        default:                                                                         \
            e_ = set_lds(KERNEL<MfF16, IO_BF16, 32>, lds);                               \
            if (e_ != hipSuccess) return e_;                                             \
            hipLaunchKernelGGL((KERNEL<MfF16, IO_BF16, 32>), grid, blk, lds, s, p);      \
            break;                                                                       \
        }                                                                                \
        return hipGetLastError();                                                        \
    } while (0)

hipError_t launch_kgrad_fused(int io, const KgradParams& p, int nsplit, int lds, hipStream_t s) {
    FFTCONV_KG_LAUNCH(kgrad_fused_kernel, dim3((unsigned)p.H, (unsigned)nsplit));
}

hipError_t launch_kgrad_reduce(const float* part, float* dk, long long n, int nsplit,
                               hipStream_t s) {
    if (n % 4) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kgrad_reduce_kernel, dim3(2048), dim3(256), 0, s, (const float4*)part,
                       (float4*)dk, n / 4, nsplit);
    return hipGetLastError();
}

hipError_t launch_kgrad_inner(int io, const KgradParams& p, int lds, hipStream_t s) {
    FFTCONV_KG_LAUNCH(kgrad_inner_kernel, dim3((unsigned)p.H, (unsigned)p.f.nunits));
}

hipError_t launch_outer_inv_f32out(int io, const FwdParams& p, int lds, hipStream_t s) {
    const int slab = p.M / p.Qo;
    const dim3 grid((unsigned)p.rows, slab / p.ct), blk(p.threads);
    hipError_t e;
    if (io == IO_F32) {
        e = set_lds(outer_inv_kernel<MfF32, IO_F32>, lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((outer_inv_kernel<MfF32, IO_F32>), grid, blk, lds, s, p);
    } else {
        e = set_lds(outer_inv_kernel<MfF16, IO_F32>, lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((outer_inv_kernel<MfF16, IO_F32>), grid, blk, lds, s, p);
    }
    return hipGetLastError();
}

// Streaming copy through 16-byte non-temporal loads and stores: each
// workgroup moves contiguous chunks of 4 x 256 x 16 bytes, four loads in
// flight per thread before the stores.  Its rate is the one a pure
// read+write stream reaches on the part (the practical HBM roof), and its
// byte counters are the reference for kernels that stream the same way.
typedef unsigned int stream_v4 __attribute__((ext_vector_type(4)));
__global__ void __launch_bounds__(256) stream_copy_kernel(const stream_v4* __restrict__ src,
                                                          stream_v4* __restrict__ dst,
                                                          long long n16) {
    constexpr long long PER = 4 * 256;
    for (long long base = (long long)blockIdx.x * PER; base < n16;
         base += (long long)gridDim.x * PER) {
        const long long i0 = base + threadIdx.x;
        stream_v4 r[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (i0 + k * 256 < n16) r[k] = __builtin_nontemporal_load(&src[i0 + k * 256]);
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (i0 + k * 256 < n16) __builtin_nontemporal_store(r[k], &dst[i0 + k * 256]);
    }
}

hipError_t launch_stream_copy(const void* src, void* dst, long long n16, int num_cu, hipStream_t s) {
    hipLaunchKernelGGL(stream_copy_kernel, dim3((unsigned)(32 * num_cu)), dim3(256), 0, s,
                       (const stream_v4*)src, (stream_v4*)dst, n16);
    return hipGetLastError();
}

hipError_t launch_scale_f32(float* x, long long n, float a, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(scale_f32_kernel, dim3(1024), dim3(256), 0, s, x, n, a);
    return hipGetLastError();
}

}  // namespace fftconv
