// Fused kernel for rows of N = P * 1024 (P = 4, 8, 16, 32) with 16-bit I/O:
// one workgroup per row (P/2 wavefronts, at most eight), the whole 2N-point
// transform held in LDS and registers (page "FlashFFTConv: Efficient Convolutions for Long
// Sequences with Tensor Cores", section 3.4 and Algorithm 1: an order-3
// Monarch decomposition P x 32 x 32, with the real-input packing and the
// implicit zero padding of section 3.4, "Implicit zero-padding for causal
// convolutions").
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
// Input and output rows are touched once and go through non-temporal
// loads and stores, which keeps L2 for the spectrum coefficients.
//
// Gated rows (y = v (.) ((u (.) w) * k)): the input gate is prefetched with
// u and multiplies it in the outer forward stage; the output gate is
// fetched as the outer inverse stage starts and multiplies its results
// before the store (fp32 for bf16 rows, packed f16 for f16 rows, as the
// stage itself computes).
//
// FULL (the circular operators at FFT size 2M, P <= 16): no zero half; the
// outer stage takes all P sub-rows of the row (a whole P-point DFT) and the
// outer inverse stores all P.
//
// Mirror pairing.  Bin k pairs with -k.  For 0 < k1 < P/2 the partner bins
// live in sub-row P - k1.  That sub-row is pushed through the engine as
// w_k1 * conj(A_{P-k1}) -- the same twiddle as sub-row k1 -- which returns
// conj(Z[-k]) in exactly the register that holds Z[k]: the spectrum product
// of a pair becomes element-wise, and the partner's inverse result is the
// conjugate of the engine output.  Sub-row 0 pairs within itself by
// negation (as in the row kernel) and sub-row P/2 by reversal
// k' <-> 1023 - k', whose partner sits one lane over (a DPP rotation).
#include "fftconv_engine.h"

namespace fftconv {

using namespace eng;

// Waves per workgroup: one per mirror pair of sub-rows up to P = 16; at
// P = 32 the 16 pairs go to 8 waves, two each in turn (the row's 32 sub-rows
// fill 128 KB of LDS, which leaves no room for the outer twiddles: those are
// read through L2 instead).
template <int P>
struct WideShape {
    static constexpr int HALF = P / 2;
    static constexpr int WAVES = HALF < 8 ? HALF : 8;
    static constexpr int T = 64 * WAVES;
    static constexpr int PPW = HALF / WAVES;     // mirror pairs per wave
    static constexpr bool TWG = P > 16;          // outer twiddles from memory
};

template <int IO, int P, bool G, bool SK, bool FULL>
__global__ void __launch_bounds__(WideShape<P>::T, 2) wide_kernel(WideParams prm) {
    typedef WideShape<P> WS;
    constexpr int Q = 1024, M = P * Q, HALF = P / 2, T = WS::T;
    constexpr int NIN = FULL ? P : HALF;      // sub-rows loaded and stored
    constexpr int ROWW = NIN * Q;             // 32-bit words per I/O row
    constexpr int WAVES = WS::WAVES, PPW = WS::PPW;
    constexpr bool TWG = WS::TWG;
    constexpr int CPT = Q / T;   // outer-stage columns per thread
    static_assert(!(FULL && TWG), "FFT-size rows on the P <= 16 kernels only");

    extern __shared__ uint4 s_lds[];
    uint4* s_f1b = s_lds;                              // [ks 2][jt 4][64]
    uint4* s_i1a = s_f1b + 8 * 64;                     // [mt 4][ks 2][64]
    uint32_t* s_two = (uint32_t*)(s_i1a + 8 * 64);     // [k1 - 1][thread][column]
    uint32_t* s_buf = s_two + (TWG ? 0 : HALF * Q);    // [P sub-rows][Q]
    uint32_t* s_scr = s_buf + M;                       // [39 k_b slots][16 x]
    int* s_claim = (int*)(s_scr + 39 * 16);            // [2] claimed row indices

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, x = lane & 15;
    const int total = prm.B * prm.H;
    // Rows are taken in channel-major order (index h * B + b), in the order
    // of this workgroup's XCD group (with counters: claimed from them; the
    // library passes none: each workgroup takes its fixed share), one row
    // ahead by thread 0 and published through LDS at the row's barriers.
    const XcdClaim claimer(prm.ctr, gridDim.x, blockIdx.x);

    for (int i = tid; i < 8 * 64; i += T) {
        s_f1b[i] = ((const uint4*)prm.f1b)[i];
        s_i1a[i] = ((const uint4*)prm.i1a)[i];
    }
    if constexpr (!TWG)
        for (int i = tid; i < HALF * Q / 4; i += T) ((uint4*)s_two)[i] = ((const uint4*)prm.two)[i];
    if (tid == 0) {
        const long long c0 = claimer.next(), c1 = claimer.next();
        s_claim[0] = (int)(c0 < total ? c0 : total);
        s_claim[1] = (int)(c1 < total ? c1 : total);
    }
    // engine tables in registers: for the whole kernel up to P = 16; at
    // P = 32 they are reloaded (from L2) for each row's engine phase, so
    // that they are not live across the larger outer stages
    Regs E;
    if constexpr (!TWG) load_regs(E, prm.f2a, SK ? prm.i2bs : prm.i2b, prm.twf, lane);
    // outer twiddles read from memory (P = 32): [k1 - 1][thread][column]
    const __amdgpu_buffer_rsrc_t rtwo = buf_rsrc(prm.two, HALF * T * CPT * 4);

    // ---- outer-stage geometry: n_b = tid & 31, n_a = na0 + j (j < CPT)
    const int nb = tid & 31, na0 = CPT * (tid >> 5);
    const int it_o = nb < 16 ? 0 : 1, x_o = nb < 16 ? nb : (nb == 16 ? 0 : 32 - nb);
    const int oa0 = eng_addr(na0, it_o, x_o);   // consecutive words for j < min(CPT, 4)
    // outer twiddles w_k1[n'] (k1 = 1..HALF) of this thread's columns
    auto load_two = [&](uint32_t (&tw)[HALF][CPT]) {
#pragma unroll
        for (int k1 = 0; k1 < HALF; ++k1) {
            if constexpr (TWG) {
                static_assert(CPT == 2, "memory twiddles are read as pairs");
                const uint2 v = *(const uint2*)(prm.two + (k1 * T + tid) * CPT);
                tw[k1][0] = v.x;
                tw[k1][1] = v.y;
                continue;
            }
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
    uint32_t uin[NIN][CPT];
    uint32_t win[G ? NIN : 1][CPT];   // input gate (gated only)
    auto load_u = [&](int idx) {
        const int hh = idx / prm.B, bb = idx - hh * prm.B;
        const long long off = ((long long)bb * prm.H + hh) * ROWW;
        const uint32_t* u = (const uint32_t*)prm.u + off;
#pragma unroll
        for (int n1 = 0; n1 < NIN; ++n1) {
            const uint32_t* un = u + n1 * Q + lofs;
#pragma unroll
            for (int j = 0; j < CPT; ++j) uin[n1][j] = __builtin_nontemporal_load(&un[32 * j]);
        }
        if constexpr (G) {
            const uint32_t* w = (const uint32_t*)prm.w + off;
#pragma unroll
            for (int n1 = 0; n1 < NIN; ++n1) {
                const uint32_t* wn = w + n1 * Q + lofs;
#pragma unroll
                for (int j = 0; j < CPT; ++j) win[n1][j] = __builtin_nontemporal_load(&wn[32 * j]);
            }
        }
    };
    __syncthreads();
    int cur = s_claim[0], nxt = s_claim[1];
    if (cur >= total) return;   // uniform over the workgroup
    load_u(cur);

    uint32_t* scr = s_scr + x;
    const int i1_base = (16 * (g >> 1) + x) * 4 + 2 * (g & 1);

    while (cur < total) {
        const int h = cur / prm.B, b = cur - h * prm.B;
        const long long mrow = (long long)b * prm.H + h;
        // next row of this workgroup (past the end: re-read this row)
        const int inext = nxt < total ? nxt : cur;
        // ---------------- outer forward stage
        if constexpr (TWG) {
            // one column at a time, its twiddles read as it starts and its
            // P outputs stored to LDS as they come
            typedef Outer<IO> O;
            typedef typename O::V C;
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                uint32_t tw[HALF];
#pragma unroll
                for (int k1 = 0; k1 < HALF; ++k1)
                    tw[k1] = __builtin_amdgcn_raw_buffer_load_b32(rtwo, (unsigned)(tid * CPT + j) * 4u,
                                                                  k1 * T * CPT * 4, 0);
                C xin[HALF], A[P];
#pragma unroll
                for (int n1 = 0; n1 < HALF; ++n1) {
                    xin[n1] = O::from_io(uin[n1][j]);
                    if constexpr (G) xin[n1] = O::emul(xin[n1], win[n1][j]);
                }
                dft_half_in<P>(xin, A);
                uint32_t* dst = s_buf + oa0 + j;
                dst[0] = O::to_h2(A[0]);
                dst[Q] = O::to_h2(O::mul(A[HALF], tw[HALF - 1]));
#pragma unroll
                for (int k1 = 1; k1 < HALF; ++k1) {
                    dst[(2 * k1) * Q] = O::to_h2(O::mul(A[k1], tw[k1 - 1]));
                    dst[(2 * k1 + 1) * Q] = O::to_h2(O::mul(cnj(A[P - k1]), tw[k1 - 1]));
                }
                // the columns one after the other (interleaved, their
                // transforms would not fit the registers together)
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            typedef Outer<IO> O;
            typedef typename O::V C;
            uint32_t two[HALF][CPT];
            load_two(two);
            uint32_t V[P][CPT];
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                C xin[NIN], A[P];
#pragma unroll
                for (int n1 = 0; n1 < NIN; ++n1) {
                    xin[n1] = O::from_io(uin[n1][j]);
                    if constexpr (G) xin[n1] = O::emul(xin[n1], win[n1][j]);
                }
                if constexpr (FULL) {
#pragma unroll
                    for (int n1 = 0; n1 < P; ++n1) A[n1] = xin[n1];
                    dft_small<P, false>(A);
                } else {
                    dft_half_in<P>(xin, A);
                }
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
        // claim the row after next now: the atomic returns long before the
        // value is published, and it is older than the loads it must not
        // delay
        long long c2 = 0;
        if (tid == 0) c2 = claimer.next();
        __syncthreads();
        if constexpr (TWG) load_regs_buf(E, prm.f2a, SK ? prm.i2bs : prm.i2b, prm.twf, lane);

        // ---------------- engine: mirror pair j = wave + q * WAVES (q < PPW),
        // sub-rows 2 j and 2 j + 1
#pragma unroll
        for (int q = 0; q < PPW; ++q) {
            const int pr = wave + q * WAVES;
            if (pr >= prm.pairs) {
                // a frequency-sparse call whose pair holds only zeroed bins:
                // its sub-rows are zero
                if (q == PPW - 1) {
                    if (tid == 0) s_claim[0] = (int)(c2 < total ? c2 : total);
                    load_u(inext);
                }
                uint4* z0 = (uint4*)(s_buf + (2 * pr) * Q);
#pragma unroll
                for (int i = 0; i < 8; ++i) z0[i * 64 + lane] = make_uint4(0u, 0u, 0u, 0u);
                continue;
            }
            // spectrum coefficients of this row's bins, in flight while the
            // forward transforms run; kt = 1 is issued after sub-row 0
            const uint4* cf = (const uint4*)prm.kf + ((long long)h * HALF + pr) * 1024;
            uint4 cfr[2][2][4];   // [sub][kt][mt]
#pragma unroll
            for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) cfr[sub][0][mt] = cf[(sub * 2) * 256 + mt * 64 + lane];
            uint32_t z[2][2][4][2];   // [sub][kt][mt][e] packed f16 bins
            forward<SK>(s_buf + (2 * pr) * Q, s_f1b, E, lane, z[0]);
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) cfr[s2][1][mt] = cf[(s2 * 2 + 1) * 256 + mt * 64 + lane];
            __builtin_amdgcn_sched_barrier(0);
            forward<SK>(s_buf + (2 * pr + 1) * Q, s_f1b, E, lane, z[1]);
            __builtin_amdgcn_sched_barrier(0);

            // ---------------- spectrum product
            uint4 a2[2][2][2];   // [sub][kt][ks] inverse A operands
            if (pr != 0) {
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    pair_elem<SK>(kt, z[0], z[1], cfr[0][kt], cfr[1][kt], a2[0][kt], a2[1][kt]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
                // sub-row 0 pairs by negation, sub-row P/2 by reversal
                uint32_t zq[4][2];
                self_exchange(z[0], scr, g, zq);
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    pair_self<SK>(kt, x == 0, z[0], z[1], zq, cfr[0][kt], cfr[1][kt], a2[0][kt], a2[1][kt]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            if (q == PPW - 1) {
                // publish the row after next; then the next row's input,
                // issued only now because the load counter retires in order
                // and the coefficient loads above must not wait behind it
                if (tid == 0) s_claim[0] = (int)(c2 < total ? c2 : total);
                load_u(inext);
            }

            // ---------------- inverse 1024-point DFT of both sub-rows
            inverse<SK>(a2[0], s_i1a, E, lane, i1_base, s_buf + (2 * pr) * Q);
            __builtin_amdgcn_sched_barrier(0);
            inverse<SK>(a2[1], s_i1a, E, lane, i1_base, s_buf + (2 * pr + 1) * Q);
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
        const int nn = s_claim[0];
        // ---------------- outer inverse stage and store
        if constexpr (TWG) {
            // one column at a time (as the forward stage)
            typedef Outer<IO> O;
            typedef typename O::V C;
            uint32_t* yrow = (uint32_t*)prm.y + mrow * (M / 2);
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                uint32_t vin[G ? HALF : 1];   // output gate (gated only)
                if constexpr (G) {
                    const uint32_t* vr = (const uint32_t*)prm.v + mrow * (M / 2);
#pragma unroll
                    for (int n1 = 0; n1 < HALF; ++n1)
                        vin[n1] = __builtin_nontemporal_load(&vr[n1 * Q + lofs + 32 * j]);
                }
                uint32_t tw[HALF];
#pragma unroll
                for (int k1 = 0; k1 < HALF; ++k1)
                    tw[k1] = __builtin_amdgcn_raw_buffer_load_b32(rtwo, (unsigned)(tid * CPT + j) * 4u,
                                                                  k1 * T * CPT * 4, 0);
                const uint32_t* src = s_buf + oa0 + j;
                C Bv[P], zo[HALF];
                Bv[0] = O::from_h2(src[0]);
                Bv[HALF] = O::mulc(O::from_h2(src[Q]), tw[HALF - 1]);
#pragma unroll
                for (int k1 = 1; k1 < HALF; ++k1) {
                    Bv[k1] = O::mulc(O::from_h2(src[(2 * k1) * Q]), tw[k1 - 1]);
                    Bv[P - k1] = cnj(O::mulc(O::from_h2(src[(2 * k1 + 1) * Q]), tw[k1 - 1]));
                }
                idft_half_out<P>(Bv, zo);
#pragma unroll
                for (int n1 = 0; n1 < HALF; ++n1) {
                    if constexpr (G) zo[n1] = O::emul(zo[n1], vin[n1]);
                    __builtin_nontemporal_store(O::to_io(zo[n1]), &yrow[n1 * Q + lofs + 32 * j]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            uint32_t vin[G ? NIN : 1][CPT];   // output gate (gated only)
            if constexpr (G) {
                const uint32_t* vr = (const uint32_t*)prm.v + mrow * ROWW;
#pragma unroll
                for (int n1 = 0; n1 < NIN; ++n1)
#pragma unroll
                    for (int j = 0; j < CPT; ++j)
                        vin[n1][j] = __builtin_nontemporal_load(&vr[n1 * Q + lofs + 32 * j]);
            }
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
            uint32_t* yrow = (uint32_t*)prm.y + mrow * ROWW;
            uint32_t two[HALF][CPT];
            load_two(two);
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                typedef Outer<IO> O;
                typedef typename O::V C;
                C Bv[P], zo[NIN];
                Bv[0] = O::from_h2(R[0][j]);
                Bv[HALF] = O::mulc(O::from_h2(R[1][j]), two[HALF - 1][j]);
#pragma unroll
                for (int k1 = 1; k1 < HALF; ++k1) {
                    Bv[k1] = O::mulc(O::from_h2(R[2 * k1][j]), two[k1 - 1][j]);
                    Bv[P - k1] = cnj(O::mulc(O::from_h2(R[2 * k1 + 1][j]), two[k1 - 1][j]));
                }
                if constexpr (FULL) {
                    dft_small<P, true>(Bv);
#pragma unroll
                    for (int n1 = 0; n1 < P; ++n1) zo[n1] = Bv[n1];
                } else {
                    idft_half_out<P>(Bv, zo);
                }
#pragma unroll
                for (int n1 = 0; n1 < NIN; ++n1) {
                    if constexpr (G) zo[n1] = O::emul(zo[n1], vin[n1][j]);
                    __builtin_nontemporal_store(O::to_io(zo[n1]), &yrow[n1 * Q + lofs + 32 * j]);
                }
            }
        }
        cur = nxt;
        nxt = nn;
    }
}

template <bool G, bool SK, bool FULL>
static hipError_t launch_wide_g(int io, int P, const WideParams& p, int lds, hipStream_t s) {
    const dim3 grid((unsigned)p.grid), blk((unsigned)(P >= 16 ? 512 : 32 * P));
#define FFTCONV_WIDE(IOT, PP)                                                                  \
    do {                                                                                       \
        if (lds > 64 * 1024) {                                                                 \
            hipError_t e_ = hipFuncSetAttribute((const void*)wide_kernel<IOT, PP, G, SK, FULL>, \
                                                hipFuncAttributeMaxDynamicSharedMemorySize,     \
                                                lds);                                          \
            if (e_ != hipSuccess) return e_;                                                   \
        }                                                                                      \
        hipLaunchKernelGGL((wide_kernel<IOT, PP, G, SK, FULL>), grid, blk, lds, s, p);         \
    } while (0)
    if (io == IO_BF16) {
        if (P == 4) FFTCONV_WIDE(IO_BF16, 4);
        else if (P == 8) FFTCONV_WIDE(IO_BF16, 8);
        else if (P == 16) FFTCONV_WIDE(IO_BF16, 16);
        else if (P == 32 && !FULL) FFTCONV_WIDE(IO_BF16, 32 - 16 * FULL);
        else return hipErrorInvalidValue;
    } else {
        if (P == 4) FFTCONV_WIDE(IO_F16, 4);
        else if (P == 8) FFTCONV_WIDE(IO_F16, 8);
        else if (P == 16) FFTCONV_WIDE(IO_F16, 16);
        else if (P == 32 && !FULL) FFTCONV_WIDE(IO_F16, 32 - 16 * FULL);
        else return hipErrorInvalidValue;
    }
#undef FFTCONV_WIDE
    return hipGetLastError();
}

hipError_t launch_wide(int io, int P, const WideParams& p, int lds, hipStream_t s) {
    if (p.full) {
        // FFT-size rows: P <= 16, no band limit or digit blocks
        if (p.skip_hi || P > 16 || p.pairs != P / 2) return hipErrorInvalidValue;
        return p.w ? launch_wide_g<true, false, true>(io, P, p, lds, s)
                   : launch_wide_g<false, false, true>(io, P, p, lds, s);
    }
    if (p.w) return launch_wide_g<true, false, false>(io, P, p, lds, s);
    if (p.skip_hi) return launch_wide_g<false, true, false>(io, P, p, lds, s);
    return launch_wide_g<false, false, false>(io, P, p, lds, s);
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
