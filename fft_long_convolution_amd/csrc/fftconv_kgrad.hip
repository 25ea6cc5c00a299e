// Kernel gradient of the causal convolution on the register-resident
// 32 x 32 engine (N = 1024, 16-bit I/O):
//   dk[h][j] = sum_b sum_{t>=j} dy[b,h,t] u[b,h,t-j],
// the inverse transform of G = sum_b conj(U_b) DY_b (page "FlashFFTConv:
// Efficient Convolutions for Long Sequences with Tensor Cores", section 3:
// the gradients of an FFT convolution multiply by conjugate spectra, and the
// input spectra are recomputed in the backward pass instead of kept).
//
// kgrad_row_kernel: one wavefront per (channel, slice of the batch).  Each
// row of u and of dy goes through the forward half of the row kernel (whole
// 128-byte line loads, F1 with the twiddle, F2), which leaves bin
// k = k_a + 32 k_b and its mirror -k in the same lane (the k_a = 0 column
// through an LDS exchange).  With a = Z_u[k], c = conj Z_u[-k], d = Z_dy[k],
// e = conj Z_dy[-k], E2 = a + c, O' = a - c, Ed2 = d + e, Od' = d - e and
// w = W_2N^k, the packed spectrum of the real result is
//   4 Z_g[k] = 2 conj(E2) d + conj(O') (Od' - conj(w)^2 Ed2):
// the real-FFT unpack of both spectra, the products conj(U) DY at k and
// k + M, and the repack, folded into three complex products (packed f16,
// like the forward pairing).  The wave accumulates it
// over its rows in fp32 registers and writes the lane's 16 bins to a
// partial row.
// kgrad_row_inv: one wavefront per channel sums the partial rows and runs
// the inverse half of the engine (I2, twiddle, I1) into fp32 dk.
#include "fftconv_engine.h"

namespace fftconv {

constexpr int kKgWaves = 8;

// The channel's accumulated spectrum (times 4; s4[kt * 4 + mt] holds bins
// (kt, mt, e = 0, 1) of the lane) through I2, the conjugate twiddle and I1
// into fp32 dk, as the row kernel's inverse; `pre` scales the f16 operands
// so that they stay in range however concentrated the spectrum is.
__device__ __forceinline__ void kg_row_inverse(const float4 (&s4)[8], const uint4* s_i2b,
                                               const uint4* s_i1a, const uint32_t (&twf)[2][2][4],
                                               const KgRowParams& P, int h, int lane) {
    constexpr int NB = 32, MT2 = 4, KS2 = 2, NT = 2;
    const int g = lane >> 4, x = lane & 15;
    uint4 a2[2][KS2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
        uint32_t zp[MT2][2];
#pragma unroll
        for (int mt = 0; mt < MT2; ++mt) {
            const float4 v = s4[kt * MT2 + mt];
            zp[mt][0] = pk2(v.x * P.pre, v.y * P.pre);
            zp[mt][1] = pk2(v.z * P.pre, v.w * P.pre);
        }
#pragma unroll
        for (int ks = 0; ks < KS2; ++ks)
            a2[kt][ks] = make_uint4(zp[2 * ks][0], zp[2 * ks][1], zp[2 * ks + 1][0], zp[2 * ks + 1][1]);
    }
    // I2 and the conjugate twiddle, as the row kernel
    uint4 b1v[2][NT];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            rfloat4 re = {0.f, 0.f, 0.f, 0.f}, im = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS2; ++ks) {
                re = mma_f16(a2[kt][ks], s_i2b[(ks * 2 * NT + 2 * nt) * 64 + lane], re);
                im = mma_f16(a2[kt][ks], s_i2b[(ks * 2 * NT + 2 * nt + 1) * 64 + lane], im);
            }
            uint32_t w[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) w[r] = as_u32(hmulc(as_h2(pk2(re[r], im[r])), as_h2(twf[kt][nt][r])));
            b1v[kt][nt] = make_uint4(w[0], w[1], w[2], w[3]);
        }
    // I1 into fp32 points (t even, t odd), whole lines as the row kernel
    float2* dk = (float2*)(P.dk + (long long)h * (32 * NB));
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        float2 o[NT][2];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            rfloat4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) acc = mma_f16(s_i1a[(mt * 2 + ks) * 64 + lane], b1v[ks][nt], acc);
#pragma unroll
            for (int e = 0; e < 2; ++e) o[nt][e] = make_float2(acc[2 * e] * P.post, acc[2 * e + 1] * P.post);
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            uint32_t ax = __float_as_uint(o[0][e].x), bx = __float_as_uint(o[1][e].x);
            uint32_t ay = __float_as_uint(o[0][e].y), by = __float_as_uint(o[1][e].y);
            swap16(ax, bx);
            swap16(ay, by);
            const int na = 8 * mt + 4 * (g >> 1) + e, w = (g & 1) ? kmap32(1, x) : x;
            dk[NB * na + w] = make_float2(__uint_as_float(ax), __uint_as_float(ay));
            dk[NB * (na + 2) + w] = make_float2(__uint_as_float(bx), __uint_as_float(by));
        }
    }
}

// FUSE (S = kKgWaves: a workgroup's waves are the slices of one channel):
// the slices' sums meet in LDS and wave 0 runs the inverse into dk, with no
// partial rows in memory and no second kernel.
template <int IO, bool FUSE>
__global__ void __launch_bounds__(64 * kKgWaves, 1) kgrad_row_kernel(KgRowParams P) {
    constexpr int NB = 32, IT = 2, MT2 = 4, KS2 = 2, M = 1024;
    constexpr bool BF = (IO == IO_BF16);
    constexpr int F1T = BF ? 8 : 4;
    extern __shared__ uint4 s_lds[];
    uint4* s_f1b = s_lds;                                   // [F1T][64]
    uint4* s_f2a = s_f1b + F1T * 64;                        // [MT2][KS2][64]
    uint32_t* s_scr = (uint32_t*)(s_f2a + MT2 * KS2 * 64);  // [waves][2][NB][16]
    uint4* s_i2b = (uint4*)(s_scr + kKgWaves * 2 * NB * 16);  // FUSE: [KS2][4][64]
    uint4* s_i1a = s_i2b + 8 * 64;                             // FUSE: [4][64]
    float4* s_red = (float4*)(s_i1a + 4 * 64);                 // FUSE: [waves][64][8]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, x = lane & 15;
    constexpr int TH = 64 * kKgWaves;
    for (int i = tid; i < F1T * 64; i += TH) s_f1b[i] = ((const uint4*)P.f1b)[i];
    for (int i = tid; i < MT2 * KS2 * 64; i += TH) s_f2a[i] = ((const uint4*)P.f2a)[i];
    if constexpr (FUSE) {
        for (int i = tid; i < 8 * 64; i += TH) s_i2b[i] = ((const uint4*)P.i2b)[i];
        for (int i = tid; i < 4 * 64; i += TH) s_i1a[i] = ((const uint4*)P.i1a)[i];
    }
    uint32_t twf[IT][2][4];
#pragma unroll
    for (int it = 0; it < IT; ++it)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) twf[it][kt][r] = P.twf[lane * (IT * 8) + (it * 2 + kt) * 4 + r];
    __syncthreads();
    // without FUSE no workgroup barrier follows: a wave without a task may
    // leave; with FUSE every wave has one (the grid is one workgroup per
    // channel) and an idle one would still reach the barrier
    const int task = blockIdx.x * kKgWaves + wave;
    const bool has_task = task < P.H * P.S;
    if (!FUSE && !has_task) return;
    const int h = task / P.S, sl = task - h * P.S;
    const int b0 = has_task ? (int)((long long)P.B * sl / P.S) : 0;
    const int b1 = has_task ? (int)((long long)P.B * (sl + 1) / P.S) : 0;

    // conj(W_2N^k)^2 = exp(2 pi i k / M) of the lane's bins, packed f16
    uint32_t wc[2][MT2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int mt = 0; mt < MT2; ++mt)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int k = kmap32(kt, x) + 32 * rmid_perm(8 * mt + 2 * g + e, NB);
                float sn, cs;
                sincospif(2.f * (float)k / (float)M, &sn, &cs);
                wc[kt][mt][e] = pk2(cs, sn);
            }

    auto load_row = [&](uint32_t (&dst)[IT][4], const void* base, int b) {
        const uint32_t* r = (const uint32_t*)base + ((long long)b * P.H + h) * (M / 2);
#pragma unroll
        for (int q = 0; q < 8; ++q)
            dst[q >> 2][q & 3] =
                __builtin_nontemporal_load(&r[NB * (8 * (g >> 1) + q) + ((g & 1) ? kmap32(1, x) : x)]);
    };
    // F1 (with the twiddle) and F2 of one row: bins (kt, mt, e) as packed f16
    auto forward = [&](uint32_t (&cur)[IT][4], uint32_t (&z)[2][MT2][2]) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) swap16(cur[0][jj], cur[1][jj]);
        uint4 b2[KS2][2];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const uint4 a = make_uint4(cur[it][0], cur[it][1], cur[it][2], cur[it][3]);
            rfloat4 c1[4];
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) {
                rfloat4 acc = {0.f, 0.f, 0.f, 0.f};
                if (BF) {
                    acc = mma_bf16(a, s_f1b[jt * 64 + lane], acc);
                    acc = mma_bf16(a, s_f1b[(4 + jt) * 64 + lane], acc);
                } else {
                    acc = mma_f16(a, s_f1b[jt * 64 + lane], acc);
                }
                c1[jt] = acc;
            }
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                uint32_t w[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    w[r] = as_u32(hmul(as_h2(pk2(c1[2 * kt][r], c1[2 * kt + 1][r])), as_h2(twf[it][kt][r])));
                b2[it][kt] = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int mt = 0; mt < MT2; ++mt) {
                rfloat4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS2; ++ks) acc = mma_f16(s_f2a[(mt * KS2 + ks) * 64 + lane], b2[ks][kt], acc);
                z[kt][mt][0] = pk2(acc[0], acc[1]);
                z[kt][mt][1] = pk2(acc[2], acc[3]);
            }
    };
    // bin -k_b of the k_a = 0 column, from the lane group that holds it
    uint32_t* scr_u = s_scr + (wave * 2) * 16 * NB + x;
    uint32_t* scr_d = scr_u + 16 * NB;
    auto mirror0 = [&](const uint32_t (&z)[2][MT2][2], uint32_t* scr, uint32_t (&zq)[MT2][2]) {
#pragma unroll
        for (int mt = 0; mt < MT2; ++mt)
#pragma unroll
            for (int e = 0; e < 2; ++e) scr[16 * rmid_perm(8 * mt + 2 * g + e, NB)] = z[0][mt][e];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int mt = 0; mt < MT2; ++mt)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int kb = rmid_perm(8 * mt + 2 * g + e, NB);
                zq[mt][e] = scr[16 * ((NB - kb) & (NB - 1))];
            }
    };

    float2 acc[2][MT2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int mt = 0; mt < MT2; ++mt)
#pragma unroll
            for (int e = 0; e < 2; ++e) acc[kt][mt][e] = make_float2(0.f, 0.f);

    const bool l0 = (x == 0);
    uint32_t nu[IT][4], nd[IT][4];   // next row, in flight
    if (b0 < b1) {
        load_row(nu, P.u, b0);
        load_row(nd, P.dy, b0);
    }
    for (int b = b0; b < b1; ++b) {
        uint32_t cu[IT][4], cd[IT][4];
#pragma unroll
        for (int it = 0; it < IT; ++it)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                cu[it][jj] = nu[it][jj];
                cd[it][jj] = nd[it][jj];
            }
        // the next row (past the end: this row again, so every iteration
        // issues the same loads)
        const int bn = b + 1 < b1 ? b + 1 : b;
        load_row(nu, P.u, bn);
        load_row(nd, P.dy, bn);
        uint32_t zu[2][MT2][2], zd[2][MT2][2], qu[MT2][2], qd[MT2][2];
        forward(cu, zu);
        forward(cd, zd);
        mirror0(zu, scr_u, qu);
        mirror0(zd, scr_d, qd);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int mt = 0; mt < MT2; ++mt)
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int pm = (mt + MT2 / 2) % MT2;
                    uint32_t pu, pd;
                    if (kt == 0) {
                        pu = l0 ? qu[mt][e] : zu[1][pm][e];
                        pd = l0 ? qd[mt][e] : zd[1][pm][e];
                    } else {
                        pu = l0 ? zu[1][pm][e] : zu[0][pm][e];
                        pd = l0 ? zd[1][pm][e] : zd[0][pm][e];
                    }
                    const rhalf2 A = as_h2(zu[kt][mt][e]), Ap = as_h2(pu);
                    const rhalf2 Dv = as_h2(zd[kt][mt][e]), Dp = as_h2(pd);
                    const rhalf2 cAp = {Ap.x, -Ap.y}, cDp = {Dp.x, -Dp.y};
                    const rhalf2 E2 = A + cAp, O2 = A - cAp;
                    const rhalf2 Ed = Dv + cDp, Od = Dv - cDp;
                    const rhalf2 T = Od - hmul(Ed, as_h2(wc[kt][mt][e]));
                    const rhalf2 two = {(_Float16)2.f, (_Float16)2.f};
                    const rhalf2 R = __builtin_elementwise_fma(hmulc(Dv, E2), two, hmulc(T, O2));
                    acc[kt][mt][e].x += (float)R.x;
                    acc[kt][mt][e].y += (float)R.y;
                }
    }
    float4* o = FUSE ? s_red + (wave * 64 + lane) * 8
                     : (float4*)P.part + ((long long)(sl * P.H + h) * 64 + lane) * 8;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int mt = 0; mt < MT2; ++mt)
            o[kt * MT2 + mt] = make_float4(acc[kt][mt][0].x, acc[kt][mt][0].y, acc[kt][mt][1].x,
                                           acc[kt][mt][1].y);
    if constexpr (FUSE) {
        __syncthreads();
        if (wave == 0 && has_task) {
            float4 s4[2 * MT2];
#pragma unroll
            for (int i = 0; i < 2 * MT2; ++i) s4[i] = make_float4(0.f, 0.f, 0.f, 0.f);
            for (int w = 0; w < kKgWaves; ++w) {
#pragma unroll
                for (int i = 0; i < 2 * MT2; ++i) {
                    const float4 v = s_red[(w * 64 + lane) * 8 + i];
                    s4[i].x += v.x;
                    s4[i].y += v.y;
                    s4[i].z += v.z;
                    s4[i].w += v.w;
                }
            }
            kg_row_inverse(s4, s_i2b, s_i1a, twf, P, h, lane);
        }
    }
}

template <int IO>
__global__ void __launch_bounds__(64 * kKgWaves, 1) kgrad_row_inv_kernel(KgRowParams P) {
    constexpr int MT2 = 4, KS2 = 2, NT = 2, IT = 2;
    extern __shared__ uint4 s_lds[];
    uint4* s_i2b = s_lds;                       // [KS2][2 NT][64]
    uint4* s_i1a = s_i2b + KS2 * 2 * NT * 64;   // [4][64]
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    constexpr int TH = 64 * kKgWaves;
    for (int i = tid; i < KS2 * 2 * NT * 64; i += TH) s_i2b[i] = ((const uint4*)P.i2b)[i];
    for (int i = tid; i < 4 * 64; i += TH) s_i1a[i] = ((const uint4*)P.i1a)[i];
    uint32_t twf[IT][2][4];
#pragma unroll
    for (int it = 0; it < IT; ++it)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) twf[it][kt][r] = P.twf[lane * (IT * 8) + (it * 2 + kt) * 4 + r];
    __syncthreads();
    const int h = blockIdx.x * kKgWaves + wave;
    if (h >= P.H) return;
    // the channel's accumulated spectrum (times 4), scaled by `pre` so that
    // the f16 operands stay in range however concentrated it is
    float4 s4[2 * MT2];
#pragma unroll
    for (int i = 0; i < 2 * MT2; ++i) s4[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int sl = 0; sl < P.S; ++sl) {
        const float4* p = (const float4*)P.part + ((long long)(sl * P.H + h) * 64 + lane) * 8;
#pragma unroll
        for (int i = 0; i < 2 * MT2; ++i) {
            const float4 v = p[i];
            s4[i].x += v.x;
            s4[i].y += v.y;
            s4[i].z += v.z;
            s4[i].w += v.w;
        }
    }
    kg_row_inverse(s4, s_i2b, s_i1a, twf, P, h, lane);
}

int kgrad_row_lds(int io) { return ((io == IO_BF16 ? 8 : 4) + 8) * 64 * 16 + kKgWaves * 2 * 32 * 16 * 4; }
// with FUSE: the inverse's tables and the slices' sums
int kgrad_row_fused_lds(int io) { return kgrad_row_lds(io) + (8 + 4) * 64 * 16 + kKgWaves * 64 * 8 * 16; }

template <int IO>
static hipError_t kgrad_row_fused_t(const KgRowParams& p, hipStream_t s) {
    const int lds = kgrad_row_fused_lds(IO);
    const hipError_t e = hipFuncSetAttribute((const void*)kgrad_row_kernel<IO, true>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((kgrad_row_kernel<IO, true>), dim3((unsigned)p.H), dim3(64 * kKgWaves), lds, s, p);
    return hipGetLastError();
}

hipError_t launch_kgrad_row(int io, const KgRowParams& p, hipStream_t s) {
    if (p.H <= 0 || p.S <= 0) return hipSuccess;
    if (p.S == kKgWaves)
        return io == IO_BF16 ? kgrad_row_fused_t<IO_BF16>(p, s) : kgrad_row_fused_t<IO_F16>(p, s);
    const unsigned tasks = (unsigned)(p.H * p.S);
    const dim3 grid((tasks + kKgWaves - 1) / kKgWaves), blk(64 * kKgWaves);
    const int lds = kgrad_row_lds(io);
    if (io == IO_BF16) hipLaunchKernelGGL((kgrad_row_kernel<IO_BF16, false>), grid, blk, lds, s, p);
    else hipLaunchKernelGGL((kgrad_row_kernel<IO_F16, false>), grid, blk, lds, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 grid2((unsigned)((p.H + kKgWaves - 1) / kKgWaves));
    const int lds2 = (2 * 2 * 2 + 4) * 64 * 16;
    if (io == IO_BF16) hipLaunchKernelGGL(kgrad_row_inv_kernel<IO_BF16>, grid2, blk, lds2, s, p);
    else hipLaunchKernelGGL(kgrad_row_inv_kernel<IO_F16>, grid2, blk, lds2, s, p);
    return hipGetLastError();
}


// ---------------------------------------------------------------------------
// The same on the one-workgroup-per-row engine (N = P x 1024, P = 4, 8, 16,
// 16-bit I/O): a workgroup of P/2 waves per (channel, batch slice).  Each
// row of u and of dy goes through the wide kernel's outer forward stage into
// LDS and the engine's forward transform of the wave's two sub-rows.  For
// waves w >= 1 the second sub-row holds conj(Z[-k]) where the first holds
// Z[k] (k = w + P k'), so both contributions are element-wise:
//   4 Z_g[k]        = 2 conj(E2) d + conj(O') (Od' - W Ed2)
//   4 conj Z_g[-k]  = 2 conj(E2) e + conj(O') (Od' + W Ed2)
// with a, c, d, e the two sub-rows of u and dy, E2 = a + c, O' = a - c,
// Ed2 = d + e, Od' = d - e and W = exp(2 pi i k / M) -- the second one in the
// conjugated form the inverse expects of that sub-row.  Wave 0's sub-rows
// (k = P k' and P/2 + P k') pair within themselves as in the wide kernel.
// kgrad_wide_inv_kernel sums the slices per channel, runs the engine's
// inverse and the outer inverse stage, and writes fp32 dk.
// ---------------------------------------------------------------------------
using namespace eng;

template <int IO, int P>
__global__ void __launch_bounds__(32 * P, 2) kgrad_wide_kernel(KgWideParams K) {
    constexpr int Q = 1024, M = P * Q, HALF = P / 2, T = 32 * P;
    constexpr int CPT = Q / T;
    extern __shared__ uint4 s_lds[];
    uint4* s_f1b = s_lds;                              // [ks 2][jt 4][64]
    uint32_t* s_two = (uint32_t*)(s_f1b + 8 * 64);     // [k1 - 1][thread][column]
    uint32_t* s_buf = s_two + HALF * Q;                // [P sub-rows][Q]
    uint32_t* s_scr = s_buf + M;                       // [u, dy][39 k_b slots][16 x]
    uint32_t* s_wb = s_scr + 2 * 39 * 16;              // [kt][mt][e][lane] exp(2 pi i k'/1024)

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, x = lane & 15;
    for (int i = tid; i < 8 * 64; i += T) s_f1b[i] = ((const uint4*)K.f1b)[i];
    for (int i = tid; i < HALF * Q / 4; i += T) ((uint4*)s_two)[i] = ((const uint4*)K.two)[i];
    Regs E;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) E.f2a[mt][ks] = ((const uint4*)K.f2a)[(mt * 2 + ks) * 64 + lane];
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) E.twf[it][kt][r] = K.twf[lane * 16 + (it * 2 + kt) * 4 + r];
    __syncthreads();

    const int h = blockIdx.x / K.S, sl = blockIdx.x - h * K.S;
    const int b0 = (int)((long long)K.B * sl / K.S), b1 = (int)((long long)K.B * (sl + 1) / K.S);

    // W = exp(2 pi i k / M) = exp(2 pi i k1 / M) exp(2 pi i k' / 1024): the
    // lane's engine bins k' times a factor of the sub-row
    if (wave == 0) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int kp = kmap32(kt, x) + 32 * rmid_perm(8 * mt + 2 * g + e, 32);
                    float sn, cs;
                    sincospif(2.f * (float)kp / (float)Q, &sn, &cs);
                    s_wb[((kt * 4 + mt) * 2 + e) * 64 + lane] = pk2(cs, sn);
                }
    }
    __syncthreads();
    // sub-row factors: wave w >= 1: k1 = w for both; wave 0: 1 and P/2
    uint32_t wsub[2];
    {
        float sn, cs;
        sincospif(2.f * (float)(wave == 0 ? HALF : wave) / (float)M, &sn, &cs);
        const uint32_t f = pk2(cs, sn);
        wsub[0] = wave == 0 ? pk2(1.f, 0.f) : f;
        wsub[1] = f;
    }

    // ---- outer forward stage geometry (as the wide kernel)
    const int nb = tid & 31, na0 = CPT * (tid >> 5);
    const int it_o = nb < 16 ? 0 : 1, x_o = nb < 16 ? nb : (nb == 16 ? 0 : 32 - nb);
    const int oa0 = eng_addr(na0, it_o, x_o);
    const int lofs = 32 * na0 + nb;
    auto load_in = [&](uint32_t (&dst)[HALF][CPT], const void* base, int b) {
        const uint32_t* r = (const uint32_t*)base + ((long long)b * K.H + h) * (M / 2);
#pragma unroll
        for (int n1 = 0; n1 < HALF; ++n1)
#pragma unroll
            for (int j = 0; j < CPT; ++j) dst[n1][j] = __builtin_nontemporal_load(&r[n1 * Q + lofs + 32 * j]);
    };
    auto outer_fwd = [&](const uint32_t (&in)[HALF][CPT]) {
        typedef Outer<IO> O;
        typedef typename O::V C;
        uint32_t V[P][CPT];
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            C xin[HALF], A[P];
#pragma unroll
            for (int n1 = 0; n1 < HALF; ++n1) xin[n1] = O::from_io(in[n1][j]);
            dft_half_in<P>(xin, A);
            const uint32_t* tw = s_two + tid * CPT + j;
            V[0][j] = O::to_h2(A[0]);
            V[1][j] = O::to_h2(O::mul(A[HALF], tw[(HALF - 1) * T * CPT]));
#pragma unroll
            for (int k1 = 1; k1 < HALF; ++k1) {
                const uint32_t t = tw[(k1 - 1) * T * CPT];
                V[2 * k1][j] = O::to_h2(O::mul(A[k1], t));
                V[2 * k1 + 1][j] = O::to_h2(O::mul(cnj(A[P - k1]), t));
            }
        }
#pragma unroll
        for (int sidx = 0; sidx < P; ++sidx) {
            uint32_t* dst = s_buf + sidx * Q + oa0;
            if constexpr (CPT == 2) {
                *(uint2*)dst = make_uint2(V[sidx][0], V[sidx][1]);
            } else {
#pragma unroll
                for (int q = 0; q < CPT / 4; ++q)
                    *(uint4*)(dst + 64 * q) =
                        make_uint4(V[sidx][4 * q], V[sidx][4 * q + 1], V[sidx][4 * q + 2], V[sidx][4 * q + 3]);
            }
        }
    };

    float2 acc[2][2][4][2];   // [sub][kt][mt][e]
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int e = 0; e < 2; ++e) acc[sb][kt][mt][e] = make_float2(0.f, 0.f);

    uint32_t* scr_u = s_scr + x;
    uint32_t* scr_d = s_scr + 39 * 16 + x;
    for (int b = b0; b < b1; ++b) {
        uint32_t zu[2][2][4][2], zd[2][2][4][2];   // [sub][kt][mt][e]
        {
            uint32_t in_u[HALF][CPT];
            load_in(in_u, K.u, b);
            outer_fwd(in_u);
        }
        __syncthreads();
        forward(s_buf + (2 * wave) * Q, s_f1b, E, lane, zu[0]);
        forward(s_buf + (2 * wave + 1) * Q, s_f1b, E, lane, zu[1]);
        __syncthreads();
        {
            uint32_t in_d[HALF][CPT];
            load_in(in_d, K.dy, b);
            outer_fwd(in_d);
        }
        __syncthreads();
        forward(s_buf + (2 * wave) * Q, s_f1b, E, lane, zd[0]);
        forward(s_buf + (2 * wave + 1) * Q, s_f1b, E, lane, zd[1]);
        if (wave != 0) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const rhalf2 a = as_h2(zu[0][kt][mt][e]), c = as_h2(zu[1][kt][mt][e]);
                        const rhalf2 d = as_h2(zd[0][kt][mt][e]), ee = as_h2(zd[1][kt][mt][e]);
                        const rhalf2 W = hmul(as_h2(s_wb[((kt * 4 + mt) * 2 + e) * 64 + lane]), as_h2(wsub[0]));
                        const rhalf2 E2 = a + c, O2 = a - c, Ed = d + ee, Od = d - ee;
                        const rhalf2 WE = hmul(Ed, W);
                        const rhalf2 two = {(_Float16)2.f, (_Float16)2.f};
                        const rhalf2 RX = __builtin_elementwise_fma(hmulc(d, E2), two, hmulc(Od - WE, O2));
                        const rhalf2 RY = __builtin_elementwise_fma(hmulc(ee, E2), two, hmulc(Od + WE, O2));
                        acc[0][kt][mt][e].x += (float)RX.x;
                        acc[0][kt][mt][e].y += (float)RX.y;
                        acc[1][kt][mt][e].x += (float)RY.x;
                        acc[1][kt][mt][e].y += (float)RY.y;
                    }
        } else {
            // sub-row 0 pairs k' with -k' (the k_a = 0 column through LDS),
            // sub-row 1 pairs k' with 1023 - k' (one lane over)
            uint32_t qu[4][2], qd[4][2];
            self_exchange(zu[0], scr_u, g, qu);
            self_exchange(zd[0], scr_d, g, qd);
            const bool l0 = (x == 0);
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    const int pm = (mt + 2) & 3;
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        uint32_t nu, nd;
                        if (kt == 0) {
                            nu = l0 ? qu[mt][e] : zu[0][1][pm][e];
                            nd = l0 ? qd[mt][e] : zd[0][1][pm][e];
                        } else {
                            nu = l0 ? zu[0][1][pm][e] : zu[0][0][pm][e];
                            nd = l0 ? zd[0][1][pm][e] : zd[0][0][pm][e];
                        }
                        const uint32_t ru = kt == 0 ? rot_up(zu[1][1][pm][e]) : rot_down(zu[1][0][pm][e]);
                        const uint32_t rd = kt == 0 ? rot_up(zd[1][1][pm][e]) : rot_down(zd[1][0][pm][e]);
                        const rhalf2 W0 = as_h2(s_wb[((kt * 4 + mt) * 2 + e) * 64 + lane]);
                        const rhalf2 W1 = hmul(W0, as_h2(wsub[1]));
                        const rhalf2 R0 = kg_self(zu[0][kt][mt][e], nu, zd[0][kt][mt][e], nd, W0);
                        const rhalf2 R1 = kg_self(zu[1][kt][mt][e], ru, zd[1][kt][mt][e], rd, W1);
                        acc[0][kt][mt][e].x += (float)R0.x;
                        acc[0][kt][mt][e].y += (float)R0.y;
                        acc[1][kt][mt][e].x += (float)R1.x;
                        acc[1][kt][mt][e].y += (float)R1.y;
                    }
                }
        }
        __syncthreads();
    }
    float4* o = (float4*)K.part + (((long long)(sl * K.H + h) * HALF + wave) * 64 + lane) * 16;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                o[(sb * 2 + kt) * 4 + mt] = make_float4(acc[sb][kt][mt][0].x, acc[sb][kt][mt][0].y,
                                                        acc[sb][kt][mt][1].x, acc[sb][kt][mt][1].y);
}

template <int IO, int P>
__global__ void __launch_bounds__(32 * P, 2) kgrad_wide_inv_kernel(KgWideParams K) {
    constexpr int Q = 1024, M = P * Q, HALF = P / 2, T = 32 * P;
    constexpr int CPT = Q / T;
    extern __shared__ uint4 s_lds[];
    uint4* s_i1a = s_lds;                              // [mt 4][ks 2][64]
    uint32_t* s_two = (uint32_t*)(s_i1a + 8 * 64);
    uint32_t* s_buf = s_two + HALF * Q;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, x = lane & 15;
    for (int i = tid; i < 8 * 64; i += T) s_i1a[i] = ((const uint4*)K.i1a)[i];
    for (int i = tid; i < HALF * Q / 4; i += T) ((uint4*)s_two)[i] = ((const uint4*)K.two)[i];
    Regs E;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) E.i2b[ks][jt] = ((const uint4*)K.i2b)[(ks * 4 + jt) * 64 + lane];
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) E.twf[it][kt][r] = K.twf[lane * 16 + (it * 2 + kt) * 4 + r];
    const int h = blockIdx.x;
    // the channel's accumulated spectra of this wave's sub-rows
    float4 s4[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) s4[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int sl = 0; sl < K.S; ++sl) {
        const float4* pp = (const float4*)K.part + (((long long)(sl * K.H + h) * HALF + wave) * 64 + lane) * 16;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float4 v = pp[i];
            s4[i].x += v.x;
            s4[i].y += v.y;
            s4[i].z += v.z;
            s4[i].w += v.w;
        }
    }
    uint4 a2[2][2][2];   // [sub][kt][ks]
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            uint32_t pz[4][2];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const float4 v = s4[(sb * 2 + kt) * 4 + mt];
                pz[mt][0] = pk2(v.x * K.pre, v.y * K.pre);
                pz[mt][1] = pk2(v.z * K.pre, v.w * K.pre);
            }
            pack_a2(pz, a2[sb][kt]);
        }
    __syncthreads();   // tables in LDS
    const int i1_base = (16 * (g >> 1) + x) * 4 + 2 * (g & 1);
    inverse(a2[0], s_i1a, E, lane, i1_base, s_buf + (2 * wave) * Q);
    inverse(a2[1], s_i1a, E, lane, i1_base, s_buf + (2 * wave + 1) * Q);
    __syncthreads();
    // outer inverse stage, fp32 output
    const int nb = tid & 31, na0 = CPT * (tid >> 5);
    const int it_o = nb < 16 ? 0 : 1, x_o = nb < 16 ? nb : (nb == 16 ? 0 : 32 - nb);
    const int oa0 = eng_addr(na0, it_o, x_o);
    const int lofs = 32 * na0 + nb;
    typedef Outer<IO> O;
    typedef typename O::V C;
    uint32_t R[P][CPT];
#pragma unroll
    for (int sidx = 0; sidx < P; ++sidx) {
        const uint32_t* src = s_buf + sidx * Q + oa0;
        if constexpr (CPT == 2) {
            const uint2 v = *(const uint2*)src;
            R[sidx][0] = v.x;
            R[sidx][1] = v.y;
        } else {
#pragma unroll
            for (int q = 0; q < CPT / 4; ++q) {
                const uint4 v = *(const uint4*)(src + 64 * q);
                R[sidx][4 * q] = v.x;
                R[sidx][4 * q + 1] = v.y;
                R[sidx][4 * q + 2] = v.z;
                R[sidx][4 * q + 3] = v.w;
            }
        }
    }
    float2* dk = (float2*)(K.dk + (long long)h * M);   // N = M reals per row
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const uint32_t* tw = s_two + tid * CPT + j;
        C Bv[P], zo[HALF];
        Bv[0] = O::from_h2(R[0][j]);
        Bv[HALF] = O::mulc(O::from_h2(R[1][j]), tw[(HALF - 1) * T * CPT]);
#pragma unroll
        for (int k1 = 1; k1 < HALF; ++k1) {
            const uint32_t t = tw[(k1 - 1) * T * CPT];
            Bv[k1] = O::mulc(O::from_h2(R[2 * k1][j]), t);
            Bv[P - k1] = cnj(O::mulc(O::from_h2(R[2 * k1 + 1][j]), t));
        }
        idft_half_out<P>(Bv, zo);
#pragma unroll
        for (int n1 = 0; n1 < HALF; ++n1)
            dk[n1 * Q + lofs + 32 * j] = make_float2((float)zo[n1].x * K.post, (float)zo[n1].y * K.post);
    }
}

int kgrad_wide_lds(int P) {
    return 8 * 64 * 16 + (P / 2) * 1024 * 4 + P * 1024 * 4 + 2 * 39 * 16 * 4 + 16 * 64 * 4;
}
int kgrad_wide_inv_lds(int P) { return 8 * 64 * 16 + (P / 2) * 1024 * 4 + P * 1024 * 4; }

template <int IO, int P>
static hipError_t kgrad_wide_t(const KgWideParams& p, hipStream_t s) {
    const int l1 = kgrad_wide_lds(P), l2 = kgrad_wide_inv_lds(P);
    hipError_t e = hipFuncSetAttribute((const void*)kgrad_wide_kernel<IO, P>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, l1);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void*)kgrad_wide_inv_kernel<IO, P>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, l2);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((kgrad_wide_kernel<IO, P>), dim3((unsigned)(p.H * p.S)), dim3(32 * P), l1, s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((kgrad_wide_inv_kernel<IO, P>), dim3((unsigned)p.H), dim3(32 * P), l2, s, p);
    return hipGetLastError();
}

hipError_t launch_kgrad_wide(int io, int P, const KgWideParams& p, hipStream_t s) {
    if (p.H <= 0 || p.S <= 0) return hipSuccess;
    if (io == IO_BF16) {
        if (P == 4) return kgrad_wide_t<IO_BF16, 4>(p, s);
        if (P == 8) return kgrad_wide_t<IO_BF16, 8>(p, s);
        if (P == 16) return kgrad_wide_t<IO_BF16, 16>(p, s);
    } else {
        if (P == 4) return kgrad_wide_t<IO_F16, 4>(p, s);
        if (P == 8) return kgrad_wide_t<IO_F16, 8>(p, s);
        if (P == 16) return kgrad_wide_t<IO_F16, 16>(p, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace fftconv
