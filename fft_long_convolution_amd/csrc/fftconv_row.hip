// Register-resident fused kernel for rows of N = 32 * NB (NB = 16 or 32):
// the whole row -- load, four Monarch DFT stages, twiddles, the spectrum
// product with mirror-bin pairing, store -- stays in one wavefront's
// registers (page "FlashFFTConv: Efficient Convolutions for Long Sequences
// with Tensor Cores", section 3.4, Algorithm 1: matrix products with the
// twiddle and kernel multiplies done in the accumulators, register reuse of
// appendix A.2).
//
// Packed row z[m] = u[2m] + i u[2m+1], m = NB*n_a + n_b (n_a < 16 nonzero:
// the causal zero half is never touched).  Bins k = k_a + 32 k_b.
// FULL (the circular operators at FFT size 2M = 64 NB, no padding): all 32
// n_a are loaded, F1 contracts them in two K-steps and I1 produces all 32.
//
// The four matrix-core products alternate the role of the data so that the
// index the next stage contracts is always the one held inside a lane:
//   F1  C[n_b][(c,k_a)] = data(A: rows n_b, K n_a) x F32       (k_a -> lanes)
//   F2  C[(k_b,c)][k_a] = F_NB x data(B: K n_b, cols k_a)      (k_b in-lane)
//   I2  C[k_a][(c,n_b)] = data(A: rows k_a, K k_b) x F_NB^-1   (k_a in-lane)
//   I1  C[(n_a,c)][n_b] = F32^-1 x data(B: K k_a, cols n_b)    (n_a < 16;
//                                                               all: FULL)
// Real and imaginary parts of a point always sit in the same lane (the
// complex index goes to rows, or to separate column tiles).  Lane x holds
// k_a = x and its mirror 32-x (lane 0: 0 and 16), and the F_NB row order
// keeps k_b and NB-1-k_b in one lane group, so bin k and bin -k meet in the
// same lane; only the k_a = 0 column needs an LDS exchange.
#include "fftconv_mfma.h"

namespace fftconv {

// Schedule: rows are taken in channel-major order (index = h*B + b) and each
// workgroup (one per CU, sixteen waves: four per SIMD, so that one wave's
// matrix products overlap another's vector arithmetic) owns one contiguous slice
// of that order.  The spectrum coefficients of every channel the slice
// touches are staged in LDS once at the start (lane-major, so every lane
// reads its own consecutive entries); after that the row loop has no
// barriers.  Waves claim rows of the slice one at a time from an LDS
// counter, DEPTH claims ahead of the row being computed: a wave that the
// SIMD's arbitration favours simply takes more rows, so the waves of a CU
// finish together.  Refills are unconditional (a claim past the end re-reads
// the last row), so every row issues the same memory operations and the wait
// counts stay exact.  The twiddles stay in registers for the whole kernel;
// the four stage tables are read from LDS at each use (keeping them in
// registers would halve the waves per SIMD).  Input and output rows are touched once: non-temporal loads and
// stores keep them from displacing the spectra in L2.
//
// Gated rows (y = v (.) ((u (.) w) * k)): the input gate rides in a second
// ring beside u and multiplies it as the row is consumed; the product feeds
// the first stage as f16 (for bf16 rows too: rounding it to bf16 would cost
// as much as the whole error budget).  The output gate is fetched at the
// start of the row, with the stores' addresses, and multiplies the fp32
// accumulators before the one rounding to the I/O type.  The extra registers
// take the workgroup down to twelve waves.
constexpr int kRowDepth = 2;
// Rows of 32 n_a at NB = 32 (FULL) hold twice the input registers: twelve
// waves, like gated rows; gated FULL rows also prefetch one row less.
//
// Plain rows of N = 1024 (NB = 32, no gate, band limit or FULL) run two per
// wave instead, stage by stage: each stage table read from LDS and each
// twiddle register then serves both rows, and the compiler interleaves the
// two rows' independent matrix products and vector arithmetic.  A wave
// claims two consecutive rows at once, finds their coordinates once per
// claim, and fetches the next pair as soon as the first stage has consumed
// the current one.  The doubled working set takes the workgroup to twelve
// waves; measured on MI355X at B = 64, H = 768 against the one-row loop:
// bf16 -5.2 %, f16 -5.6 % per call, bit-identical outputs.
template <bool G, bool SK, bool FULL, int NB>
constexpr bool row_pairs() { return NB == 32 && !G && !SK && !FULL; }
template <bool G, bool FULL, int NB, bool SK = false>
constexpr int row_waves() {
    return (G || (FULL && NB == 32) || row_pairs<G, SK, FULL, NB>()) ? kRowWavesGated : kRowWaves;
}

template <int IO, int NB, bool G, bool SK, bool FULL>
__global__ void __launch_bounds__((64 * row_waves<G, FULL, NB, SK>()), 1)
row_kernel(RowParams P) {
    constexpr int WAVES = row_waves<G, FULL, NB, SK>();
    constexpr bool PAIR = row_pairs<G, SK, FULL, NB>();
    constexpr int M = 32 * NB;
    constexpr int NH = FULL ? 2 : 1;      // halves of n_a loaded (16 each)
    constexpr int ROWW = NH * M / 2;      // 32-bit words per I/O row
    constexpr int MTO = 2 * NH;           // I1 output tiles (8 n_a each)
    constexpr int IT = NB / 16;    // n_b tiles
    constexpr int MT2 = NB / 8;    // k_b slot tiles
    constexpr int KS2 = NB / 16;   // K-steps over n_b / k_b
    constexpr int NT = NB / 16;    // n_b tiles of the inverse
    constexpr bool BF = (IO == IO_BF16);
    constexpr int F1R = BF ? 8 : 4;       // first-stage region (plan layout)
    constexpr bool BFA = BF && !G;        // bf16 first-stage operands
    constexpr int F1T = BFA ? 8 : 4;      // first-stage tiles used
    constexpr int D = (G && FULL && NB == 32) ? 1 : kRowDepth;

    extern __shared__ uint4 s_lds[];
    uint4* s_f1b = s_lds;                            // [NH][F1R][64]
    uint4* s_i1a = s_f1b + NH * F1R * 64;            // [MTO][2][64]
    uint4* s_f2a = s_i1a + MTO * 2 * 64;             // [MT2][KS2][64]
    uint4* s_i2b = s_f2a + MT2 * KS2 * 64;           // [KS2][2 NT][64]
    uint32_t* s_ctr = (uint32_t*)(s_i2b + KS2 * 2 * NT * 64);   // row claim counter (16 B)
    uint32_t* s_scr = s_ctr + 4;                     // [waves][NB][16]
    uint2* s_ab = (uint2*)(s_scr + kRowWaves * NB * 16);   // [channels][bins per lane][64]

    const int tid = threadIdx.x, lane = tid & 63;
    // wave index as a scalar: branches on it stay uniform (scalar branches)
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // band limit below M/4: the M-tiles of k_b = 8..23 are all zero
    constexpr bool skip_hi = SK && NB == 32;
    const int g = lane >> 4, x = lane & 15;
    const long long total = (long long)P.B * P.H;
    const long long r0 = (long long)blockIdx.x * P.rows_per_wg;
    const long long r1 = min(total, r0 + P.rows_per_wg);
    const int h_lo = (int)(r0 / P.B);

    constexpr int TH = 64 * WAVES;
    const uint4* f1src = (const uint4*)(G ? P.f1h : P.f1b);
    // the table holds F1T tiles per half; the LDS region F1R per half
    for (int i = tid; i < NH * F1T * 64; i += TH) {
        const int hf = i / (F1T * 64);
        s_f1b[hf * F1R * 64 + (i - hf * F1T * 64)] = f1src[i];
    }
    for (int i = tid; i < MTO * 2 * 64; i += TH) s_i1a[i] = ((const uint4*)P.i1a)[i];
    for (int i = tid; i < MT2 * KS2 * 64; i += TH) s_f2a[i] = ((const uint4*)P.f2a)[i];
    const uint4* i2src = (const uint4*)(skip_hi ? P.i2bs : P.i2b);
    for (int i = tid; i < KS2 * 2 * NT * 64; i += TH) s_i2b[i] = i2src[i];
    if (tid == 0) s_ctr[0] = 0;
    constexpr bool SYM = (NB == 32);
    uint32_t twf[IT][2][4], twi[SYM ? 1 : 2][SYM ? 1 : NT][4];
#pragma unroll
    for (int it = 0; it < IT; ++it)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                twf[it][kt][r] = P.twf[lane * (IT * 8) + (it * 2 + kt) * 4 + r];
    if (!SYM) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    twi[SYM ? 0 : kt][SYM ? 0 : nt][r] = P.twi[lane * (NT * 8) + (kt * NT + nt) * 4 + r];
    }

    // ---- spectrum coefficients of every channel of this slice -> LDS
    if (r0 < r1) {
        const int h_hi = (int)((r1 - 1) / P.B);
        const int nch = h_hi - h_lo + 1;
        for (int i = tid; i < nch * M; i += TH) {
            const int c = i / M, pos = i - c * M;
            // bin (k_a, k_b) at position NB*k_a + k_b -> its lane and slot
            const int ka = pos / NB, kb = pos - ka * NB;
            const int kt = ka < 16 ? 0 : 1;
            const int xx = ka < 16 ? ka : (ka == 16 ? 0 : 32 - ka);
            const int sl = kb < NB / 2 ? kb : (3 * NB / 2 - 1 - kb);
            const int mt = sl >> 3, gg = (sl >> 1) & 3, e = sl & 1;
            s_ab[(long long)c * M + ((kt * MT2 + mt) * 2 + e) * 64 + gg * 16 + xx] =
                ((const uint2*)P.kf)[(long long)(h_lo + c) * M + pos];
        }
    }
    __syncthreads();

    // rows of the slice are claimed one at a time (slice position c)
    const int nslice = (int)(r1 - r0);
    const int b_lo = (int)(r0 - (long long)h_lo * P.B);
    if constexpr (PAIR) {
        // ---- plain rows of N = 1024, two per wave, stage by stage: every
        // stage table read from LDS and every twiddle register serves both
        // rows, and the two rows' independent matrix products and vector
        // arithmetic interleave.  Claims take two consecutive slice
        // positions at once; their (channel, batch) coordinates are found
        // once per claim (positions past the end repeat the last row, whose
        // repeat is computed but not stored).
        constexpr int Q = 2;
        uint32_t ring[Q][IT][4];
        int cl0 = 0, hr[Q], br[Q];
        auto take = [&]() {
            uint32_t c = 0;
            if (lane == 0) c = atomicAdd(s_ctr, (uint32_t)Q);
            cl0 = (int)__builtin_amdgcn_readfirstlane(c);
            int off = b_lo + (cl0 < nslice ? cl0 : nslice - 1), hh = h_lo;
            while (off >= P.B) {
                off -= P.B;
                ++hh;
            }
            hr[0] = hh;
            br[0] = off;
#pragma unroll
            for (int q = 1; q < Q; ++q) {
                hr[q] = hr[q - 1];
                br[q] = br[q - 1];
                if (cl0 + q < nslice && ++br[q] >= P.B) {
                    br[q] = 0;
                    ++hr[q];
                }
            }
            // whole 128-byte rows per load, as the single-row path
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const uint32_t* uh = (const uint32_t*)P.u + ((long long)br[q] * P.H + hr[q]) * ROWW;
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    ring[q][j >> 2][j & 3] = __builtin_nontemporal_load(
                        &uh[NB * (8 * (g >> 1) + j) + ((g & 1) ? kmap32(1, x) : x)]);
            }
        };
        if (nslice > 0) take();
        uint32_t* scr = s_scr + wave * 16 * NB + x;
        const bool l0 = (x == 0);
        while (nslice > 0 && cl0 < nslice) {
            const int m0 = cl0;
            int hc[Q], bc[Q];
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                hc[q] = hr[q];
                bc[q] = br[q];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) swap16(ring[q][0][jj], ring[q][1][jj]);
            }
            // ---- F1 (as the single-row path) and its twiddle
            uint4 b2[Q][KS2][2];
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                rfloat4 c1[Q][4];
#pragma unroll
                for (int jt = 0; jt < 4; ++jt) {
                    const uint4 t0 = s_f1b[jt * 64 + lane];
                    const uint4 t1 = BFA ? s_f1b[(4 + jt) * 64 + lane] : t0;
#pragma unroll
                    for (int q = 0; q < Q; ++q) {
                        const uint4 a = make_uint4(ring[q][it][0], ring[q][it][1], ring[q][it][2],
                                                   ring[q][it][3]);
                        rfloat4 acc = {0.f, 0.f, 0.f, 0.f};
                        if (BFA) {
                            acc = mma_bf16(a, t0, acc);
                            acc = mma_bf16(a, t1, acc);
                        } else {
                            acc = mma_f16(a, t0, acc);
                        }
                        c1[q][jt] = acc;
                    }
                }
#pragma unroll
                for (int q = 0; q < Q; ++q)
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt) {
                        uint32_t w[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            w[r] = as_u32(hmul(as_h2(pk2(c1[q][2 * kt][r], c1[q][2 * kt + 1][r])),
                                               as_h2(twf[it][kt][r])));
                        b2[q][it][kt] = make_uint4(w[0], w[1], w[2], w[3]);
                    }
            }
            // the inputs are consumed: claim and fetch the next rows now, so
            // that the loads fly during the rest of the transform
            take();
            // ---- F2
            uint32_t z[Q][2][MT2][2];
#pragma unroll
            for (int mt = 0; mt < MT2; ++mt) {
                uint4 ta[KS2];
#pragma unroll
                for (int ks = 0; ks < KS2; ++ks) ta[ks] = s_f2a[(mt * KS2 + ks) * 64 + lane];
#pragma unroll
                for (int q = 0; q < Q; ++q)
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt) {
                        rfloat4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int ks = 0; ks < KS2; ++ks) acc = mma_f16(ta[ks], b2[q][ks][kt], acc);
                        z[q][kt][mt][0] = pk2(acc[0], acc[1]);
                        z[q][kt][mt][1] = pk2(acc[2], acc[3]);
                    }
            }
            // ---- mirror exchange of column 0, one row after the other
            // through the wave's LDS scratch
            uint32_t zq[Q][MT2][2];
#pragma unroll
            for (int q = 0; q < Q; ++q) {
#pragma unroll
                for (int mt = 0; mt < MT2; ++mt)
#pragma unroll
                    for (int e = 0; e < 2; ++e)
                        scr[16 * rmid_perm(8 * mt + 2 * g + e, NB)] = z[q][0][mt][e];
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
                for (int mt = 0; mt < MT2; ++mt)
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const int kb = rmid_perm(8 * mt + 2 * g + e, NB);
                        zq[q][mt][e] = scr[16 * ((NB - kb) & (NB - 1))];
                    }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            }
            // ---- spectrum product with the mirror partners (as the
            // single-row path)
            uint4 a2[Q][2][KS2];
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const int abbase = (hc[q] - h_lo) * M;
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    uint32_t zp[MT2][2];
#pragma unroll
                    for (int mt = 0; mt < MT2; ++mt)
#pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            const int pm = (mt + MT2 / 2) % MT2;
                            const uint2 ab = s_ab[abbase + ((kt * MT2 + mt) * 2 + e) * 64 + lane];
                            uint32_t p;
                            if (kt == 0) p = l0 ? zq[q][mt][e] : z[q][1][pm][e];
                            else p = l0 ? z[q][1][pm][e] : z[q][0][pm][e];
                            zp[mt][e] = as_u32(hpair(as_h2(ab.x), as_h2(z[q][kt][mt][e]),
                                                     as_h2(ab.y), as_h2(p)));
                        }
#pragma unroll
                    for (int ks = 0; ks < KS2; ++ks)
                        a2[q][kt][ks] = make_uint4(zp[2 * ks][0], zp[2 * ks][1], zp[2 * ks + 1][0],
                                                   zp[2 * ks + 1][1]);
                }
            }
            // ---- I2 and the conjugate twiddle
            uint4 b1v[Q][2][NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                uint4 tr[KS2], ti[KS2];
#pragma unroll
                for (int ks = 0; ks < KS2; ++ks) {
                    tr[ks] = s_i2b[(ks * 2 * NT + 2 * nt) * 64 + lane];
                    ti[ks] = s_i2b[(ks * 2 * NT + 2 * nt + 1) * 64 + lane];
                }
#pragma unroll
                for (int q = 0; q < Q; ++q)
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt) {
                        rfloat4 re = {0.f, 0.f, 0.f, 0.f}, im = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int ks = 0; ks < KS2; ++ks) {
                            re = mma_f16(a2[q][kt][ks], tr[ks], re);
                            im = mma_f16(a2[q][kt][ks], ti[ks], im);
                        }
                        uint32_t w[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            w[r] = as_u32(hmulc(as_h2(pk2(re[r], im[r])), as_h2(twf[kt][nt][r])));
                        b1v[q][kt][nt] = make_uint4(w[0], w[1], w[2], w[3]);
                    }
            }
            // ---- I1 (n_a < 16) and whole-line stores
#pragma unroll
            for (int mt = 0; mt < MTO; ++mt) {
                uint4 ti[2];
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) ti[ks] = s_i1a[(mt * 2 + ks) * 64 + lane];
#pragma unroll
                for (int q = 0; q < Q; ++q) {
                    if (q > 0 && m0 + q >= nslice) continue;
                    uint32_t* yrow = (uint32_t*)P.y + ((long long)bc[q] * P.H + hc[q]) * (long long)ROWW;
                    uint32_t o[NT][2];
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        rfloat4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int ks = 0; ks < 2; ++ks) acc = mma_f16(ti[ks], b1v[q][ks][nt], acc);
#pragma unroll
                        for (int e = 0; e < 2; ++e) o[nt][e] = pk2io<IO>(acc[2 * e], acc[2 * e + 1]);
                    }
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        swap16(o[0][e], o[1][e]);
                        const int na = 8 * mt + 4 * (g >> 1) + e, w = (g & 1) ? kmap32(1, x) : x;
                        __builtin_nontemporal_store(o[0][e], &yrow[NB * na + w]);
                        __builtin_nontemporal_store(o[1][e], &yrow[NB * (na + 2) + w]);
                    }
                }
            }
        }
    } else {
        auto claim = [&]() {
            uint32_t c = 0;
            if (lane == 0) c = atomicAdd(s_ctr, 1u);
            return (int)__builtin_amdgcn_readfirstlane(c);
        };
        // slice position -> (channel, batch) by stepping from the slice's first
        // row: a slice spans only the few channels whose spectra fit the LDS, so
        // this takes a handful of scalar steps where a 64-bit division would take
        // over a hundred
        auto row_of = [&](int c, int& h, int& b) {
            int off = b_lo + (c < nslice ? c : nslice - 1);
            int hh = h_lo;
            while (off >= P.B) {
                off -= P.B;
                ++hh;
            }
            h = hh;
            b = off;
        };
        auto load_row = [&](uint32_t (&dst)[NH][IT][4], const void* base, int c) {
            int h, b;
            row_of(c, h, b);
            const uint32_t* u =
                (const uint32_t*)base + ((long long)b * P.H + h) * ROWW;
    #pragma unroll
            for (int hf = 0; hf < NH; ++hf) {
                const uint32_t* uh = u + hf * 16 * NB;
                if constexpr (NB == 32) {
                    // whole 128-byte rows per load: lane groups g and g + 1 take
                    // the two halves of rows 8 (g / 2) + q; the exchange into the
                    // operand layout happens where the row is consumed
    #pragma unroll
                    for (int q = 0; q < 8; ++q)
                        dst[hf][q >> 2][q & 3] = __builtin_nontemporal_load(
                            &uh[NB * (8 * (g >> 1) + q) + ((g & 1) ? kmap32(1, x) : x)]);
                } else {
    #pragma unroll
                    for (int it = 0; it < IT; ++it)
    #pragma unroll
                        for (int jj = 0; jj < 4; ++jj)
                            dst[hf][it][jj] = __builtin_nontemporal_load(&uh[NB * (4 * g + jj) + nbmap<NB>(it, x)]);
                }
            }
        };

        uint32_t ring[D][NH][IT][4];
        uint32_t wring[G ? D : 1][NH][IT][4];   // input gate rows (gated only)
        int cl[D];
        if (nslice > 0) {
    #pragma unroll
            for (int k = 0; k < D; ++k) {
                cl[k] = claim();
                load_row(ring[k], P.u, cl[k]);
                if constexpr (G) load_row(wring[k], P.w, cl[k]);
            }
        }
        // mirror exchange of the k_a = 0 column: every lane writes its column-0
        // bins and reads back bin -k_b of the same column (used by lanes x = 0)
        uint32_t* scr = s_scr + wave * 16 * NB + x;

        {
            auto row_body = [&](uint32_t (&cur)[NH][IT][4], uint32_t (&wcur)[NH][IT][4], const int m) {
                int h, b;
                row_of(m, h, b);
                const long long row = (long long)b * P.H + h;
                const int abbase = (h - h_lo) * M;
                // output gate at the stores' addresses: [mt][nt][e] is the word
                // stored from o[nt][e] of tile mt (for NB = 32 after the
                // exchange, which is undone below)
                uint32_t vg[G ? MTO : 1][NT][2];
                if constexpr (G) {
                    const uint32_t* vrow = (const uint32_t*)P.v + row * (long long)ROWW;
    #pragma unroll
                    for (int mt = 0; mt < MTO; ++mt)
    #pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            if constexpr (NB == 32) {
                                const int na = 8 * mt + 4 * (g >> 1) + e, w = (g & 1) ? kmap32(1, x) : x;
                                vg[mt][0][e] = __builtin_nontemporal_load(&vrow[NB * na + w]);
                                vg[mt][1][e] = __builtin_nontemporal_load(&vrow[NB * (na + 2) + w]);
                            } else {
    #pragma unroll
                                for (int nt = 0; nt < NT; ++nt)
                                    vg[mt][nt][e] = __builtin_nontemporal_load(
                                        &vrow[NB * (8 * mt + 2 * g + e) + nbmap<NB>(nt, x)]);
                            }
                        }
                }
    #pragma unroll
                for (int hf = 0; hf < NH; ++hf) {
                    if constexpr (NB == 32) {
    #pragma unroll
                        for (int jj = 0; jj < 4; ++jj) {
                            swap16(cur[hf][0][jj], cur[hf][1][jj]);
                            if constexpr (G) swap16(wcur[hf][0][jj], wcur[hf][1][jj]);
                        }
                    }
                    if constexpr (G) {
    #pragma unroll
                        for (int it = 0; it < IT; ++it)
    #pragma unroll
                            for (int jj = 0; jj < 4; ++jj)
                                cur[hf][it][jj] = gate_in<IO>(cur[hf][it][jj], wcur[hf][it][jj]);
                    }
                }
                // ---- F1: 32-point DFT over n_a (16 nonzero; all 32 in two
                // K-steps when FULL), k_a to the lanes
                uint4 b2[KS2][2];
    #pragma unroll
                for (int it = 0; it < IT; ++it) {
                    rfloat4 c1[4];
    #pragma unroll
                    for (int jt = 0; jt < 4; ++jt) {
                        rfloat4 acc = {0.f, 0.f, 0.f, 0.f};
    #pragma unroll
                        for (int hf = 0; hf < NH; ++hf) {
                            const uint4 a = make_uint4(cur[hf][it][0], cur[hf][it][1], cur[hf][it][2],
                                                       cur[hf][it][3]);
                            const uint4* tb = s_f1b + hf * F1R * 64;
                            if (BFA) {
                                acc = mma_bf16(a, tb[jt * 64 + lane], acc);
                                acc = mma_bf16(a, tb[(4 + jt) * 64 + lane], acc);
                            } else {
                                acc = mma_f16(a, tb[jt * 64 + lane], acc);
                            }
                        }
                        c1[jt] = acc;
                    }
                    // twiddle W_M^{k_a n_b} (packed f16); F2's B operand (K = n_b)
    #pragma unroll
                    for (int kt = 0; kt < 2; ++kt) {
                        uint32_t w[4];
    #pragma unroll
                        for (int r = 0; r < 4; ++r)
                            w[r] = as_u32(hmul(as_h2(pk2(c1[2 * kt][r], c1[2 * kt + 1][r])),
                                               as_h2(twf[it][kt][r])));
                        b2[it][kt] = make_uint4(w[0], w[1], w[2], w[3]);
                    }
                }
                // ---- F2: NB-point DFT over n_b, k_b in-lane (rows permuted)
                // (under a band limit below M/4 the odd M-tiles -- k_b 8..23, the
                // highest frequencies -- hold only zeroed bins: not computed)
                uint32_t z[2][MT2][2];
    #pragma unroll
                for (int kt = 0; kt < 2; ++kt)
    #pragma unroll
                    for (int mt = 0; mt < MT2; ++mt) {
                        if (skip_hi && (mt & 1)) {
                            z[kt][mt][0] = z[kt][mt][1] = 0u;
                            continue;
                        }
                        rfloat4 acc = {0.f, 0.f, 0.f, 0.f};
    #pragma unroll
                        for (int ks = 0; ks < KS2; ++ks) acc = mma_f16(s_f2a[(mt * KS2 + ks) * 64 + lane], b2[ks][kt], acc);
                        z[kt][mt][0] = pk2(acc[0], acc[1]);
                        z[kt][mt][1] = pk2(acc[2], acc[3]);
                    }
                // ---- mirror partner of every bin
                // column 0 (k_a = 0, lane x = 0) pairs k_b with -k_b (mod NB),
                // which another lane group holds: exchange through LDS
    #pragma unroll
                for (int mt = 0; mt < MT2; ++mt)
    #pragma unroll
                    for (int e = 0; e < 2; ++e)
                        scr[16 * rmid_perm(8 * mt + 2 * g + e, NB)] = z[0][mt][e];
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                uint32_t zq[MT2][2];
    #pragma unroll
                for (int mt = 0; mt < MT2; ++mt)
    #pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const int kb = rmid_perm(8 * mt + 2 * g + e, NB);
                        zq[mt][e] = scr[16 * ((NB - kb) & (NB - 1))];
                    }
                // ---- spectrum product: Z'[k] = alpha Z[k] + beta conj(Z[-k])
                // partner of (k_a, k_b) for k_a != 0: (-k_a, NB-1-k_b), i.e. the
                // other column tile and M-tile mt +- MT2/2; lane 0's second
                // column (k_a = 16) is its own mirror
                const bool l0 = (x == 0);
                uint4 a2[2][KS2];
    #pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    uint32_t zp[MT2][2];
    #pragma unroll
                    for (int mt = 0; mt < MT2; ++mt)
    #pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            if (skip_hi && (mt & 1)) {
                                zp[mt][e] = 0u;
                                continue;
                            }
                            const int pm = (mt + MT2 / 2) % MT2;
                            const uint2 ab = s_ab[abbase + ((kt * MT2 + mt) * 2 + e) * 64 + lane];
                            uint32_t p;
                            if (kt == 0) {
                                p = l0 ? zq[mt][e] : z[1][pm][e];
                            } else {
                                p = l0 ? z[1][pm][e] : z[0][pm][e];
                            }
                            zp[mt][e] = as_u32(hpair(as_h2(ab.x), as_h2(z[kt][mt][e]),
                                                     as_h2(ab.y), as_h2(p)));
                        }
                    // I2's A operand (K = k_b in accumulator order): K-step ks
                    // holds M-tiles 2 ks and 2 ks + 1, or, band-limited, ks and
                    // ks + KS2 (then K-step 1 is all zero)
    #pragma unroll
                    for (int ks = 0; ks < KS2; ++ks) {
                        const int m0 = skip_hi ? ks : 2 * ks, m1 = skip_hi ? ks + KS2 : 2 * ks + 1;
                        a2[kt][ks] = make_uint4(zp[m0][0], zp[m0][1], zp[m1][0], zp[m1][1]);
                    }
                }
                // ---- I2: inverse NB-point DFT over k_b (data as A), k_a in-lane
                uint4 b1v[2][NT];
    #pragma unroll
                for (int kt = 0; kt < 2; ++kt)
    #pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        rfloat4 re = {0.f, 0.f, 0.f, 0.f}, im = {0.f, 0.f, 0.f, 0.f};
    #pragma unroll
                        for (int ks = 0; ks < KS2; ++ks) {
                            if (skip_hi && ks == 1) continue;
                            re = mma_f16(a2[kt][ks], s_i2b[(ks * 2 * NT + 2 * nt) * 64 + lane], re);
                            im = mma_f16(a2[kt][ks], s_i2b[(ks * 2 * NT + 2 * nt + 1) * 64 + lane], im);
                        }
                        // conj twiddle W_M^{-k_a n_b}; pack as I1's B operand
                        uint32_t w[4];
    #pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const rhalf2 v = as_h2(pk2(re[r], im[r]));
                            w[r] = SYM ? as_u32(hmulc(v, as_h2(twf[kt][nt][r])))
                                       : as_u32(hmul(v, as_h2(twi[SYM ? 0 : kt][SYM ? 0 : nt][r])));
                        }
                        b1v[kt][nt] = make_uint4(w[0], w[1], w[2], w[3]);
                    }
                // ---- I1: inverse 32-point DFT over k_a, only n_a < 16 (t < N;
                // all 32 when FULL)
                uint32_t* yrow = (uint32_t*)P.y + row * (long long)ROWW;
    #pragma unroll
                for (int mt = 0; mt < MTO; ++mt) {
                    uint32_t o[NT][2];
                    if constexpr (G && NB == 32) {
    #pragma unroll
                        for (int e = 0; e < 2; ++e) swap16(vg[mt][0][e], vg[mt][1][e]);
                    }
    #pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        rfloat4 acc = {0.f, 0.f, 0.f, 0.f};
    #pragma unroll
                        for (int ks = 0; ks < 2; ++ks)
                            acc = mma_f16(s_i1a[(mt * 2 + ks) * 64 + lane], b1v[ks][nt], acc);
    #pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            if constexpr (G)
                                o[nt][e] = pk2io<IO>(acc[2 * e] * io_lo<IO>(vg[mt][nt][e]),
                                                     acc[2 * e + 1] * io_hi<IO>(vg[mt][nt][e]));
                            else
                                o[nt][e] = pk2io<IO>(acc[2 * e], acc[2 * e + 1]);
                        }
                    }
                    if constexpr (NB == 32) {
                        // rows n_a = 8 mt + 4 (g / 2) + e (+ 2): whole lines
    #pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            swap16(o[0][e], o[1][e]);
                            const int na = 8 * mt + 4 * (g >> 1) + e, w = (g & 1) ? kmap32(1, x) : x;
                            __builtin_nontemporal_store(o[0][e], &yrow[NB * na + w]);
                            __builtin_nontemporal_store(o[1][e], &yrow[NB * (na + 2) + w]);
                        }
                    } else {
    #pragma unroll
                        for (int nt = 0; nt < NT; ++nt)
    #pragma unroll
                            for (int e = 0; e < 2; ++e)
                                __builtin_nontemporal_store(o[nt][e], &yrow[NB * (8 * mt + 2 * g + e) + nbmap<NB>(nt, x)]);
                    }
                }
            };
            // claims grow monotonically and the ring is consumed in claim
            // order, so the first claim past the end ends the wave's work
            bool more = nslice > 0;
            while (more) {
    #pragma unroll
                for (int k = 0; k < D; ++k) {
                    if (more && cl[k] < nslice) {
                        row_body(ring[k], wring[G ? k : 0], cl[k]);
                        cl[k] = claim();
                        load_row(ring[k], P.u, cl[k]);
                        if constexpr (G) load_row(wring[k], P.w, cl[k]);
                    } else {
                        more = false;
                    }
                }
            }
        }
    }
}

template <int IO, int NB, bool G, bool SK, bool FULL>
static hipError_t launch_row_t(const RowParams& p, int lds, hipStream_t s) {
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute((const void*)row_kernel<IO, NB, G, SK, FULL>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((row_kernel<IO, NB, G, SK, FULL>), dim3((unsigned)p.grid),
                       dim3(64 * row_waves<G, FULL, NB, SK>()), lds, s, p);
    return hipGetLastError();
}

template <bool G, bool FULL>
static hipError_t launch_row_g(int io, int nb, const RowParams& p, int lds, hipStream_t s) {
    if (io == IO_BF16)
        return nb == 32 ? launch_row_t<IO_BF16, 32, G, false, FULL>(p, lds, s)
                        : launch_row_t<IO_BF16, 16, G, false, FULL>(p, lds, s);
    return nb == 32 ? launch_row_t<IO_F16, 32, G, false, FULL>(p, lds, s)
                    : launch_row_t<IO_F16, 16, G, false, FULL>(p, lds, s);
}

hipError_t launch_row(int io, int nb, const RowParams& p, int lds, hipStream_t s) {
    if (p.full) {
        if (p.skip_hi) return hipErrorInvalidValue;
        return p.w ? launch_row_g<true, true>(io, nb, p, lds, s)
                   : launch_row_g<false, true>(io, nb, p, lds, s);
    }
    if (p.w) return launch_row_g<true, false>(io, nb, p, lds, s);
    if (p.skip_hi) {
        // band-limited rows (N = 1024 only)
        if (nb != 32) return hipErrorInvalidValue;
        return io == IO_BF16 ? launch_row_t<IO_BF16, 32, false, true, false>(p, lds, s)
                             : launch_row_t<IO_F16, 32, false, true, false>(p, lds, s);
    }
    return launch_row_g<false, false>(io, nb, p, lds, s);
}

}  // namespace fftconv
