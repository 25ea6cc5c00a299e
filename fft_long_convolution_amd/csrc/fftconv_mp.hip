// Multi-pass path for N >= 32K with 16-bit I/O (page "FlashFFTConv:
// Efficient Convolutions for Long Sequences with Tensor Cores", sections
// 3.2 and 3.4: beyond what one workgroup holds, the outer Monarch factors
// are applied in passes through HBM and the inner factors stay fused).
//
// M = P_o * 4096 with P_o = P1 (one outer level) or P1 * P2 (two levels),
// an f16 complex workspace [row][M]:
//   column pass, level 1: P1-point DFT over points spaced M/P1 apart (half
//     of them zero: the causal padding), twiddle W_M^{c k1}, u -> workspace;
//   column pass, level 2: P2-point DFT over points spaced 4096 apart inside
//     each level-1 block, twiddle W_{M/P1}^{c k2}, in place;
//   inner pass: slabs of 4096 points (outer bin k_o at slab
//     sigma(k_o) = (k_o mod P1) P2 + k_o / P1) go through the 4 x 32 x 32
//     engine in units of two slabs: the slab of k_o and the slab of its
//     mirror P_o - k_o, or slabs 0 and P_o/2 together;
//   inverse column passes in the opposite order, the last one writing y.
// Column passes compute in fp32 and store f16.  Streams (input, workspace,
// output) use non-temporal loads and stores; L2 keeps the coefficients.  Each outer stage carries
// 1/sqrt(P) so the workspace stays O(|u|).
//
// Mirror pairing across slabs.  With S_B the slab of P_o - k_o, the data
// conj(S_B[c]) W_4096^c transforms to conj(Z[-k]) at the position where the
// slab of k_o has Z[k]; in the inner outer stage that is the 4-point DFT of
// conj(S_B) taken at output (j + 1) mod 4 with twiddle W_4096^{n'(j + 1)}.
// Slab P_o/2 pairs with itself the same way (its conjugated copy fills
// sub-rows 2 and 3 of the pairing), slab 0 pairs like a fused row.
#include "fftconv_engine.h"

namespace fftconv {

using namespace eng;


// ---------------------------------------------------------------------------
// Column passes.  One thread per column c of a block: MODE 0 reads u (first
// level, P/2 nonzero inputs) and writes the workspace; MODE 1 is a forward
// level in place; MODE 2 an inverse level in place; MODE 3 the last inverse
// level, writing the P/2 outputs t < N to y.  FULL (modes 0 and 3; the
// circular operators at FFT size 2M): all P inputs and outputs, rows of M
// 32-bit words.
template <int IO, int P, int MODE, bool FULL = false>
__global__ void __launch_bounds__(256) mp_col_kernel(MpColParams prm) {
    constexpr int NIN = FULL ? P : P / 2;     // first-level points in u / y
    const long long roww = FULL ? (long long)prm.M : (long long)(prm.M / 2);
    // the first pass of a chunk clears the inner pass's claim counters
    if (MODE == 0 && blockIdx.x == 0 && threadIdx.x < kClaimWords) prm.ctr[threadIdx.x] = 0u;
    // M / P columns per row and S are powers of two and M / P is a multiple
    // of the block size, so the row is uniform over the block: shifts, and
    // one 32-bit division per block, instead of per-thread 64-bit divisions
    const int lg_row = __builtin_ctz((unsigned)prm.M) - __builtin_ctz((unsigned)P);
    const int lg_s = __builtin_ctz((unsigned)prm.S);
    const unsigned i0 = blockIdx.x * 256u;
    const long long row = (long long)(i0 >> lg_row);
    if (row >= prm.rows) return;
    const int rem = (int)(i0 & ((1u << lg_row) - 1u)) + (int)threadIdx.x;
    const int blk = rem >> lg_s, c = rem & (prm.S - 1);
    // input/output row in memory: batch row / hc, channel h0 + row % hc
    const unsigned bq = (unsigned)row / (unsigned)prm.hc;
    const long long mrow = (long long)bq * prm.H + prm.h0 + ((unsigned)row - bq * (unsigned)prm.hc);
    const float sc = rsqrtf((float)P);
    const float2 tt = prm.tw[c];   // W_{P S}^c
    const rfloat2 t1 = {tt.x, tt.y};

    rfloat2 v[P];
    uint32_t* ws = (uint32_t*)prm.ws + row * (long long)prm.M + (long long)blk * P * prm.S + c;
    if constexpr (MODE == 0) {
        const uint32_t* u = (const uint32_t*)prm.u + mrow * roww + c;
        rfloat2 xin[NIN];
#pragma unroll
        for (int n = 0; n < NIN; ++n)
            xin[n] = f2_from_io<IO>(__builtin_nontemporal_load(&u[(long long)n * prm.S])) * sc;
        if (prm.w) {
            // input gate: u (.) w, exact in fp32
            const uint32_t* w = (const uint32_t*)prm.w + mrow * roww + c;
#pragma unroll
            for (int n = 0; n < NIN; ++n)
                xin[n] = xin[n] * f2_from_io<IO>(__builtin_nontemporal_load(&w[(long long)n * prm.S]));
        }
        if constexpr (FULL) {
#pragma unroll
            for (int n = 0; n < P; ++n) v[n] = xin[n];
            dft_small<P, false>(v);
        } else {
            dft_half_in<P>(xin, v);
        }
    } else if constexpr (MODE == 1) {
#pragma unroll
        for (int n = 0; n < P; ++n) v[n] = f2_from_h2(__builtin_nontemporal_load(&ws[(long long)n * prm.S])) * sc;
        dft_small<P, false>(v);
    } else {
        // conjugate twiddles, then the inverse DFT
        rfloat2 w = {1.f, 0.f};
#pragma unroll
        for (int k = 0; k < P; ++k) {
            const rfloat2 a = f2_from_h2(__builtin_nontemporal_load(&ws[(long long)k * prm.S])) * sc;
            v[k] = k == 0 ? a : fmulc(a, w);
            w = fmul(w, t1);
        }
    }
    if constexpr (MODE <= 1) {
        rfloat2 w = {1.f, 0.f};
#pragma unroll
        for (int k = 0; k < P; ++k) {
            const rfloat2 a = k == 0 ? v[k] : fmul(v[k], w);
            __builtin_nontemporal_store(pk2(a.x, a.y), &ws[(long long)k * prm.S]);
            w = fmul(w, t1);
        }
    } else if constexpr (MODE == 2) {
        dft_small<P, true>(v);
#pragma unroll
        for (int n = 0; n < P; ++n) __builtin_nontemporal_store(pk2(v[n].x, v[n].y), &ws[(long long)n * prm.S]);
    } else {
        rfloat2 z[NIN];
        if constexpr (FULL) {
            dft_small<P, true>(v);
#pragma unroll
            for (int n = 0; n < P; ++n) z[n] = v[n];
        } else {
            idft_half_out<P>(v, z);
        }
        if (prm.v) {
            // output gate, in fp32 before the one rounding to the I/O type
            const uint32_t* g = (const uint32_t*)prm.v + mrow * roww + c;
#pragma unroll
            for (int n = 0; n < NIN; ++n)
                z[n] = z[n] * f2_from_io<IO>(__builtin_nontemporal_load(&g[(long long)n * prm.S]));
        }
        if constexpr (MODE >= 4) {
            // fp32 rows (the kernel gradient): t = 2m, 2m + 1 as one float2;
            // mode 5 adds to them (batch chunks after the first)
            float2* y = (float2*)prm.y + mrow * (long long)(prm.M / 2) + c;
#pragma unroll
            for (int n = 0; n < P / 2; ++n) {
                float2 o = make_float2(z[n].x * prm.post, z[n].y * prm.post);
                if constexpr (MODE == 5) {
                    const float2 p = y[(long long)n * prm.S];
                    o.x += p.x;
                    o.y += p.y;
                }
                y[(long long)n * prm.S] = o;
            }
        } else {
            uint32_t* y = (uint32_t*)prm.y + mrow * roww + c;
#pragma unroll
            for (int n = 0; n < NIN; ++n)
                __builtin_nontemporal_store(pk2io<IO>(z[n].x, z[n].y), &y[(long long)n * prm.S]);
        }
    }
}

// ---------------------------------------------------------------------------
// Both outer levels in one pass (two-level plans).  A tile is TC = 512 / P2
// consecutive columns c of a row with all P1 * P2 outer points of each; the
// level-1 results stay in LDS (f16, as the workspace would hold them), so
// only the level-2 results travel through HBM; the inverse mirrors it.
//   forward: task (c, n2): P1-point DFT over n1 of z[(P2 n1 + n2) 4096 + c]
//     (P1/2 nonzero), twiddle W_M^{(n2 4096 + c) k1} -> LDS (k1, n2, c);
//     task (c, k1): P2-point DFT over n2, twiddle W_{M/P1}^{c k2} ->
//     workspace [k1][k2][c] (slab k1 P2 + k2);
//   inverse: the same in reverse, only the n1 < P1/2 outputs (t < N) to y.
// Workgroups of 256 threads (two per CU) are persistent: every global load
// of the next tile (data and twiddles) is issued before the current tile's
// second level, so HBM reads overlap the arithmetic and the stores.
// Gated rows (G): the forward pass multiplies u by the input gate, fetched
// for the current tile as its level 1 starts; the inverse pass fetches the
// output gate of each level-1 task as the task starts and multiplies the
// fp32 results before the store; it issues the next tile's prefetch after
// level 1, so that the gate's loads never wait behind it.
constexpr int kCol2Threads = 256;
constexpr int col2_cols(int P2) { return 512 / P2; }

template <int IO, int P1, int P2, bool INV, bool G, bool FULL>
__global__ void __launch_bounds__(kCol2Threads, 2) mp_col2_kernel(MpCol2Params prm) {
    constexpr int TC = col2_cols(P2), SLAB = 4096, TPR = SLAB / TC;
    // first-level points in u / y: P1 / 2, or all P1 at FFT size 2M (FULL)
    constexpr int NIN = FULL ? P1 : P1 / 2;
    constexpr int NT = kCol2Threads;
    constexpr int L1T = P2 * TC / NT;             // level-1 tasks per thread (2)
    constexpr int L2T = P1 * TC / NT;             // level-2 tasks per thread (2 or 4)
    static_assert(P2 <= P1 && P1 <= 2 * P2 && TC >= 16, "outer factor pair");
    // LDS word of (k1, n2, c); n2 is rotated by k1 so that level-2 tasks of
    // one wave (several k1) hit different banks
    __shared__ uint32_t s_t[P1 * P2 * TC];
    auto lidx = [](int k1, int n2, int c) { return (k1 * P2 + ((n2 + k1) & (P2 - 1))) * TC + c; };
    const int tid = threadIdx.x;
    const long long M2 = (long long)P2 * SLAB, M = (long long)P1 * M2;
    const long long roww = FULL ? M : M / 2;   // 32-bit words per I/O row
    const long long ntiles = prm.rows * TPR;
    const float sc1 = rsqrtf((float)P1), sc2 = rsqrtf((float)P2);
    // the first pass of a chunk clears the inner pass's claim counters
    if (!INV && blockIdx.x == 0 && tid < kClaimWords) prm.ctr[tid] = 0u;

    // Tiles 2k and 2k+1 share 128-byte lines (64 bytes each): they go to
    // workgroups b and b + 8, which sit on the same XCD (blocks are dealt to
    // the 8 XCDs round-robin), so one L2 fetch serves both.  The grid is a
    // multiple of 16.
    const int bid = blockIdx.x;
    const long long tile0 = (bid & ~15) + 2 * (bid & 7) + ((bid >> 3) & 1);
    auto row_of = [&](long long t, int& c0) {
        const long long r = t / TPR;
        c0 = (int)(t - r * TPR) * TC;
        return r;
    };
    auto mem_row = [&](long long r) {
        const unsigned bq = (unsigned)r / (unsigned)prm.hc;
        return (long long)bq * prm.H + prm.h0 + ((unsigned)r - bq * (unsigned)prm.hc);
    };

    if constexpr (!INV) {
        uint32_t raw[L1T][NIN];
        float2 tw1[L1T], tw2[L2T];
        auto fetch = [&](long long t) {
            int c0;
            const long long r = row_of(t, c0);
            const uint32_t* u = (const uint32_t*)prm.u + mem_row(r) * roww + c0;
#pragma unroll
            for (int i = 0; i < L1T; ++i) {
                const int task = tid + i * NT;
                const long long col = (long long)(task / TC) * SLAB + task % TC;
#pragma unroll
                for (int n1 = 0; n1 < NIN; ++n1)
                    raw[i][n1] = __builtin_nontemporal_load(&u[(long long)n1 * M2 + col]);
                tw1[i] = prm.tw1[col + c0];
            }
#pragma unroll
            for (int j = 0; j < L2T; ++j) tw2[j] = prm.tw2[c0 + (tid + j * NT) % TC];
        };
        long long t = tile0;
        if (t < ntiles) fetch(t);
#pragma unroll 1
        for (; t < ntiles; t += gridDim.x) {
            int c0;
            const long long r = row_of(t, c0);
            uint32_t graw[G ? L1T : 1][NIN];   // input gate of this tile
            if constexpr (G) {
                const uint32_t* w = (const uint32_t*)prm.w + mem_row(r) * roww + c0;
#pragma unroll
                for (int i = 0; i < L1T; ++i) {
                    const int task = tid + i * NT;
                    const long long col = (long long)(task / TC) * SLAB + task % TC;
#pragma unroll
                    for (int n1 = 0; n1 < NIN; ++n1)
                        graw[i][n1] = __builtin_nontemporal_load(&w[(long long)n1 * M2 + col]);
                }
            }
            // level 1: P1-point DFT of the P1/2 nonzero inputs, twiddle, to LDS
#pragma unroll
            for (int i = 0; i < L1T; ++i) {
                // one task at a time: interleaved tasks would not fit the registers
                __builtin_amdgcn_sched_barrier(0);
                const int task = tid + i * NT, c = task % TC, n2 = task / TC;
                rfloat2 xin[NIN], v[P1];
#pragma unroll
                for (int n1 = 0; n1 < NIN; ++n1) {
                    xin[n1] = f2_from_io<IO>(raw[i][n1]) * sc1;
                    if constexpr (G) xin[n1] = xin[n1] * f2_from_io<IO>(graw[i][n1]);
                }
                if constexpr (FULL) {
#pragma unroll
                    for (int n1 = 0; n1 < P1; ++n1) v[n1] = xin[n1];
                    dft_small<P1, false>(v);
                } else {
                    dft_half_in<P1>(xin, v);
                }
                const rfloat2 t1 = {tw1[i].x, tw1[i].y};
                rfloat2 w = t1;
                s_t[lidx(0, n2, c)] = pk2(v[0].x, v[0].y);
#pragma unroll
                for (int k1 = 1; k1 < P1; ++k1) {
                    const rfloat2 a = fmul(v[k1], w);
                    s_t[lidx(k1, n2, c)] = pk2(a.x, a.y);
                    w = fmul(w, t1);
                }
            }
            float2 tw2c[L2T];
#pragma unroll
            for (int j = 0; j < L2T; ++j) tw2c[j] = tw2[j];
            __syncthreads();
            if (t + gridDim.x < ntiles) fetch(t + gridDim.x);
            // level 2: P2-point DFT over n2, twiddle, to the workspace
            uint32_t* ws = (uint32_t*)prm.ws + r * M + c0;
#pragma unroll
            for (int j = 0; j < L2T; ++j) {
                // one task at a time: interleaved tasks would not fit the registers
                __builtin_amdgcn_sched_barrier(0);
                const int task = tid + j * NT, c = task % TC, k1 = task / TC;
                rfloat2 v[P2];
#pragma unroll
                for (int m = 0; m < P2; ++m) v[m] = f2_from_h2(s_t[lidx(k1, m, c)]) * sc2;
                dft_small<P2, false>(v);
                const rfloat2 t2 = {tw2c[j].x, tw2c[j].y};
                rfloat2 w = t2;
                uint32_t* o = ws + (long long)k1 * M2 + c;
                __builtin_nontemporal_store(pk2(v[0].x, v[0].y), &o[0]);
#pragma unroll
                for (int k2 = 1; k2 < P2; ++k2) {
                    const rfloat2 a = fmul(v[k2], w);
                    __builtin_nontemporal_store(pk2(a.x, a.y), &o[(long long)k2 * SLAB]);
                    w = fmul(w, t2);
                }
            }
            __syncthreads();
        }
    } else {
        uint32_t raw[L2T][P2];
        float2 tw1[L1T], tw2[L2T];
        auto fetch = [&](long long t) {
            int c0;
            const long long r = row_of(t, c0);
            const uint32_t* ws = (const uint32_t*)prm.ws + r * M + c0;
#pragma unroll
            for (int j = 0; j < L2T; ++j) {
                const int task = tid + j * NT, c = task % TC, k1 = task / TC;
                const uint32_t* in = ws + (long long)k1 * M2 + c;
#pragma unroll
                for (int k2 = 0; k2 < P2; ++k2) raw[j][k2] = __builtin_nontemporal_load(&in[(long long)k2 * SLAB]);
                tw2[j] = prm.tw2[c0 + c];
            }
#pragma unroll
            for (int i = 0; i < L1T; ++i) {
                const int task = tid + i * NT;
                tw1[i] = prm.tw1[(long long)(task / TC) * SLAB + c0 + task % TC];
            }
        };
        long long t = tile0;
        if (t < ntiles) fetch(t);
#pragma unroll 1
        for (; t < ntiles; t += gridDim.x) {
            int c0;
            const long long r = row_of(t, c0);
            // inverse level 2: conjugate twiddle, P2-point inverse DFT, to LDS
#pragma unroll
            for (int j = 0; j < L2T; ++j) {
                // one task at a time: interleaved tasks would not fit the registers
                __builtin_amdgcn_sched_barrier(0);
                const int task = tid + j * NT, c = task % TC, k1 = task / TC;
                const rfloat2 t2 = {tw2[j].x, tw2[j].y};
                rfloat2 v[P2], w = t2;
                v[0] = f2_from_h2(raw[j][0]) * sc2;
#pragma unroll
                for (int k2 = 1; k2 < P2; ++k2) {
                    v[k2] = fmulc(f2_from_h2(raw[j][k2]) * sc2, w);
                    w = fmul(w, t2);
                }
                dft_small<P2, true>(v);
#pragma unroll
                for (int m = 0; m < P2; ++m) s_t[lidx(k1, m, c)] = pk2(v[m].x, v[m].y);
            }
            float2 tw1c[L1T];
#pragma unroll
            for (int i = 0; i < L1T; ++i) tw1c[i] = tw1[i];
            __syncthreads();
            if constexpr (!G) {
                if (t + gridDim.x < ntiles) fetch(t + gridDim.x);
            }
            // inverse level 1: conjugate twiddle, P1-point inverse DFT, the
            // P1/2 outputs t < N to y
            uint32_t* y = (uint32_t*)prm.y + mem_row(r) * roww + c0;
#pragma unroll
            for (int i = 0; i < L1T; ++i) {
                // one task at a time: interleaved tasks would not fit the registers
                __builtin_amdgcn_sched_barrier(0);
                const int task = tid + i * NT, c = task % TC, n2 = task / TC;
                uint32_t graw[G ? NIN : 1];   // output gate of this task
                if constexpr (G) {
                    const uint32_t* gv = (const uint32_t*)prm.v + mem_row(r) * roww + c0 +
                                         (long long)n2 * SLAB + c;
#pragma unroll
                    for (int n1 = 0; n1 < NIN; ++n1)
                        graw[n1] = __builtin_nontemporal_load(&gv[(long long)n1 * M2]);
                }
                const rfloat2 t1 = {tw1c[i].x, tw1c[i].y};
                rfloat2 v[P1], w = t1;
                v[0] = f2_from_h2(s_t[lidx(0, n2, c)]) * sc1;
#pragma unroll
                for (int k1 = 1; k1 < P1; ++k1) {
                    v[k1] = fmulc(f2_from_h2(s_t[lidx(k1, n2, c)]) * sc1, w);
                    w = fmul(w, t1);
                }
                rfloat2 z[NIN];
                if constexpr (FULL) {
                    dft_small<P1, true>(v);
#pragma unroll
                    for (int n1 = 0; n1 < P1; ++n1) z[n1] = v[n1];
                } else {
                    idft_half_out<P1>(v, z);
                }
                if constexpr (G) {
#pragma unroll
                    for (int n1 = 0; n1 < NIN; ++n1) z[n1] = z[n1] * f2_from_io<IO>(graw[n1]);
                }
                uint32_t* o = y + (long long)n2 * SLAB + c;
#pragma unroll
                for (int n1 = 0; n1 < NIN; ++n1)
                    __builtin_nontemporal_store(pk2io<IO>(z[n1].x, z[n1].y), &o[(long long)n1 * M2]);
            }
            if constexpr (G) {
                if (t + gridDim.x < ntiles) fetch(t + gridDim.x);
            }
            __syncthreads();
        }
    }
}

// ---------------------------------------------------------------------------
// Forward two-level column pass on the matrix cores, P1 = P2 = 32 (M = 4M).
// A tile is 32 columns c (c0 .. c0 + 31 of the 4096-point slab) with all
// 1024 outer points; one workgroup of eight waves per CU holds it in LDS.
//   level 1: for each (n2, c) the 32-point DFT over n1 (16 nonzero inputs)
//     as 16 x 16 x 32 products (A = DFT matrix as a hi/lo pair, B = 16
//     tasks); twiddle W_M^{(4096 n2 + c0 + c) k1} = W_1024^{n2 k1} x
//     W_M^{(c0 + c) k1} from LDS tables; to LDS as f16;
//   level 2: for each (k1, c) the 32-point DFT over n2; twiddle
//     W_M^{32 (c0 + c) k2}; to the workspace [k1][k2][c] as f16.
// Every DFT entry is a hi/lo pair of 16-bit values, so the products are as
// accurate as fp32 arithmetic; the roundings are the same two f16 stores as
// in the vector-ALU pass.  Loads and stores cover whole 128-byte lines: lane
// groups g and g + 1 take the two 16-column halves of a row, and one
// exchange between 16-lane rows rearranges them into (or out of) operands.
// The intermediate is stored [k1][c][n2] with the 16-byte granule n2 / 4
// xor-ed with c % 8 (conflict-free 128-bit accesses).
// Gated rows (G): the input gate of the tile is fetched as the tile starts
// (the prefetch of u is already in) and u (.) w enters level 1 as f16, with
// f16 hi/lo DFT operands for both I/O types.
template <int IO, bool G>
__global__ void __launch_bounds__(512, 2) mp_col2m_fwd_kernel(MpCol2Params prm) {
    constexpr int SLAB = 4096, TC = 32, TPR = SLAB / TC;
    constexpr long long M2 = 32LL * SLAB, M = 32LL * M2;
    extern __shared__ uint4 s_lds[];
    uint4* s_mid = s_lds;                                   // 8192 granules
    float2* s_tw1 = (float2*)(s_mid + 8192);                // [k1][c]
    float2* s_tw2 = s_tw1 + 1024;                           // [k2][c]
    float2* s_twn = s_tw2 + 1024;                           // [n2][k1]
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, x = lane & 15;
    const long long ntiles = prm.rows * TPR;
    if (blockIdx.x == 0 && tid < kClaimWords) prm.ctr[tid] = 0u;

    uint4 a1[4][2], a2[4][2][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int hl = 0; hl < 2; ++hl) a1[mt][hl] = prm.a1[(mt * 2 + hl) * 64 + lane];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int hl = 0; hl < 2; ++hl) a2[mt][ks][hl] = prm.a2[((mt * 2 + ks) * 2 + hl) * 64 + lane];
    }
    const float2* g_twn = prm.tm;
    const float2* g_1 = g_twn + 1024;
    const float2* g_1b = g_1 + 4096;
    const float2* g_2 = g_1b + 1024;
    const float2* g_2b = g_2 + 4096;
    for (int i = tid; i < 1024; i += 512) s_twn[i] = g_twn[i];

    auto mma = [](uint4 a, uint4 b, rfloat4 c) {
        return (IO == IO_BF16 && !G) ? mma_bf16(a, b, c) : mma_f16(a, b, c);
    };
    auto cmulf = [](float2 a, float2 b) { return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x); };
    auto mid = [](int k1, int c, int gr) { return (k1 * 32 + c) * 8 + (gr ^ (c & 7)); };
    auto tile_of = [&](long long t, int& c0) {
        const long long r = t / TPR;
        c0 = (int)(t - r * TPR) * TC;
        return r;
    };
    // per-tile twiddle tables, [k][c] (lanes of a group read 16 columns c of
    // one k: distinct banks): entry (k, c) = Ta[c0 / 32][k] Tb[c][k]
    float2 tg[2][2];   // loaded operands of this thread's two entries
    auto tw_load = [&](const float2* Ta, const float2* Tb, int c0) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int e = tid + 512 * q, k = e >> 5, c = e & 31;
            tg[q][0] = Ta[(c0 >> 5) * 32 + k];
            tg[q][1] = Tb[c * 32 + k];
        }
    };
    auto tw_store = [&](float2* T) {
#pragma unroll
        for (int q = 0; q < 2; ++q) T[tid + 512 * q] = cmulf(tg[q][0], tg[q][1]);
    };
    // next tile's input: wave w takes n2 = 4 w + j; lane (g, x) loads rows
    // n1 = 8 (g / 2) + r of column 16 (g % 2) + x
    uint32_t raw[4][8];
    auto fetch_into = [&](uint32_t (&dst)[4][8], const void* base, long long t) {
        int c0;
        const long long r = tile_of(t, c0);
        const unsigned bq = (unsigned)r / (unsigned)prm.hc;
        const long long mrow = (long long)bq * prm.H + prm.h0 + ((unsigned)r - bq * (unsigned)prm.hc);
        const uint32_t* u = (const uint32_t*)base + mrow * (M / 2) + (long long)(8 * (g >> 1)) * M2 +
                            (long long)(4 * wave) * SLAB + c0 + 16 * (g & 1) + x;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 8; ++q) dst[j][q] = __builtin_nontemporal_load(&u[q * M2 + j * SLAB]);
    };
    auto fetch = [&](long long t) { fetch_into(raw, prm.u, t); };

    long long t = blockIdx.x;
    if (t < ntiles) {
        int c0;
        tile_of(t, c0);
        tw_load(g_1, g_1b, c0);
        tw_store(s_tw1);
        fetch(t);
    }
    __syncthreads();
#pragma unroll 1
    for (; t < ntiles; t += gridDim.x) {
        int c0;
        const long long r = tile_of(t, c0);
        tw_load(g_2, g_2b, c0);       // level-2 table of this tile, stored below
        if constexpr (G) {
            uint32_t graw[4][8];
            fetch_into(graw, prm.w, t);
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int q = 0; q < 8; ++q) raw[j][q] = gate_in<IO>(raw[j][q], graw[j][q]);
        }
        // ---------------- level 1
        {
            uint4 bop[4][2];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
#pragma unroll
                for (int q = 0; q < 4; ++q) swap16(raw[j][q], raw[j][q + 4]);
                bop[j][0] = make_uint4(raw[j][0], raw[j][1], raw[j][2], raw[j][3]);
                bop[j][1] = make_uint4(raw[j][4], raw[j][5], raw[j][6], raw[j][7]);
            }
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                rfloat4 cc[2][4];
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        rfloat4 acc = {0.f, 0.f, 0.f, 0.f};
                        acc = mma(a1[mt][0], bop[j][h], acc);
                        cc[h][j] = mma(a1[mt][1], bop[j][h], acc);
                    }
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int k1 = 8 * mt + 2 * g + e;
                    float2 tn[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) tn[j] = s_twn[(4 * wave + j) * 32 + k1];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int c = 16 * h + x;
                        const float2 t1 = s_tw1[k1 * 32 + c];
                        uint32_t v[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const float2 tw = cmulf(tn[j], t1);
                            const float2 a = cmulf(make_float2(cc[h][j][2 * e], cc[h][j][2 * e + 1]), tw);
                            v[j] = pk2(a.x, a.y);
                        }
                        s_mid[mid(k1, c, wave)] = make_uint4(v[0], v[1], v[2], v[3]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        tw_store(s_tw2);
        __syncthreads();
        const long long tn_ = t + gridDim.x;
        if (tn_ < ntiles) {
            int c0n;
            tile_of(tn_, c0n);
            tw_load(g_1, g_1b, c0n);   // older than the input loads: no wait on them
            fetch(tn_);
        }
        // ---------------- level 2: wave w takes k1 = 4 w + j
        {
            uint32_t* ws = (uint32_t*)prm.ws + r * M + c0 + 16 * (g & 1) + x;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int k1 = 4 * wave + j;
                uint4 b[2][2];
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) b[h][ks] = s_mid[mid(k1, 16 * h + x, 4 * ks + g)];
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    uint32_t o[2][2];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        rfloat4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int ks = 0; ks < 2; ++ks) {
                            acc = mma_f16(a2[mt][ks][0], b[h][ks], acc);
                            acc = mma_f16(a2[mt][ks][1], b[h][ks], acc);
                        }
                        const int c = 16 * h + x;
#pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            const float2 a = cmulf(make_float2(acc[2 * e], acc[2 * e + 1]),
                                                   s_tw2[(8 * mt + 2 * g + e) * 32 + c]);
                            o[h][e] = pk2(a.x, a.y);
                        }
                    }
                    // lane group g holds k2 = 8 mt + 2 g + e of both halves:
                    // exchange so each store covers a whole line of row
                    // k2 = 8 mt + 4 (g / 2) + e (+ 2 for the second value)
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        swap16(o[0][e], o[1][e]);
                        const int k2 = 8 * mt + 4 * (g >> 1) + e;
                        __builtin_nontemporal_store(o[0][e], &ws[(long long)k1 * M2 + (long long)k2 * SLAB]);
                        __builtin_nontemporal_store(o[1][e], &ws[(long long)k1 * M2 + (long long)(k2 + 2) * SLAB]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (tn_ < ntiles) tw_store(s_tw1);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Inverse two-level column pass on the matrix cores, P1 = P2 = 32: the
// mirror of the forward pass.
//   level 2: for each (k1, c) the workspace values over k2 times the
//     conjugate twiddle W_M^{-32 (c0 + c) k2} (fp32, rounded once to f16 for
//     the operand), the inverse 32-point DFT over k2, the conjugate twiddle
//     W_1024^{-n2 k1} W_M^{-(c0 + c) k1}; to LDS [n2][c][k1] as f16;
//   level 1: for each (n2, c) the inverse DFT over k1, only n1 < 16 (t < N),
//     to y.
// Gated rows (G): the output gate of the tile is fetched, at the stores'
// addresses, before level 1 and multiplies the fp32 results before the one
// rounding to the I/O type; the next tile's workspace values are then
// fetched after level 1 so that both sets of registers are never live
// together.
template <int IO, bool G>
__global__ void __launch_bounds__(512, 2) mp_col2m_inv_kernel(MpCol2Params prm) {
    constexpr int SLAB = 4096, TC = 32, TPR = SLAB / TC;
    constexpr long long M2 = 32LL * SLAB, M = 32LL * M2;
    extern __shared__ uint4 s_lds[];
    uint4* s_mid = s_lds;                                   // [n2][c][k1 granules]
    float2* s_tw1 = (float2*)(s_mid + 8192);                // [k1][c]
    float2* s_tw2 = s_tw1 + 1024;                           // [k2][c]
    float2* s_twn = s_tw2 + 1024;                           // [n2][k1]
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, x = lane & 15;
    const long long ntiles = prm.rows * TPR;

    const float2* g_twn = prm.tm;
    const float2* g_1 = g_twn + 1024;
    const float2* g_1b = g_1 + 4096;
    const float2* g_2 = g_1b + 1024;
    const float2* g_2b = g_2 + 4096;
    for (int i = tid; i < 1024; i += 512) s_twn[i] = g_twn[i];
    const __amdgpu_buffer_rsrc_t rs_a1 = buf_rsrc(prm.a1, 2 * 2 * 2 * 64 * 16);
    const __amdgpu_buffer_rsrc_t rs_a2 = buf_rsrc(prm.a2, 4 * 2 * 2 * 64 * 16);

    auto cmulf = [](float2 a, float2 b) { return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x); };
    auto cmulcf = [](float2 a, float2 b) { return make_float2(a.x * b.x + a.y * b.y, a.y * b.x - a.x * b.y); };
    auto mid = [](int n2, int c, int gr) { return (n2 * 32 + c) * 8 + (gr ^ (c & 7)); };
    auto tile_of = [&](long long t, int& c0) {
        const long long r = t / TPR;
        c0 = (int)(t - r * TPR) * TC;
        return r;
    };
    // per-tile twiddle tables [k][c], both built for the next tile during
    // level 1
    float2 tg[2][2][2];
    auto tw_load = [&](int c0) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int e = tid + 512 * q, k = e >> 5, c = e & 31;
            tg[0][q][0] = g_1[(c0 >> 5) * 32 + k];
            tg[0][q][1] = g_1b[c * 32 + k];
            tg[1][q][0] = g_2[(c0 >> 5) * 32 + k];
            tg[1][q][1] = g_2b[c * 32 + k];
        }
    };
    auto tw_store = [&]() {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            s_tw1[tid + 512 * q] = cmulf(tg[0][q][0], tg[0][q][1]);
            s_tw2[tid + 512 * q] = cmulf(tg[1][q][0], tg[1][q][1]);
        }
    };
    // next tile's workspace values: wave w takes k1 = 4 w + j; lane (g, x)
    // loads k2 = 16 ks + 8 (g / 2) + q of column 16 (g % 2) + x
    uint32_t raw[4][16];
    // (a wave-uniform base per row block and a 32-bit lane offset: no
    // 64-bit per-lane addresses to keep)
    const unsigned lofs = (unsigned)(8 * (g >> 1) * SLAB + 16 * (g & 1) + x);
    auto fetch = [&](long long t) {
        int c0;
        const long long r = tile_of(t, c0);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const uint32_t* wb = (const uint32_t*)prm.ws + r * M + (long long)(4 * wave + j) * M2 +
                                     (long long)((q >> 3) * 16 + (q & 7)) * SLAB + c0;
                raw[j][q] = __builtin_nontemporal_load(&wb[lofs]);
            }
    };

    long long t = blockIdx.x;
    if (t < ntiles) {
        int c0;
        tile_of(t, c0);
        tw_load(c0);
        tw_store();
        fetch(t);
    }
    __syncthreads();
#pragma unroll 1
    for (; t < ntiles; t += gridDim.x) {
        int c0;
        const long long r = tile_of(t, c0);
        // ---------------- inverse level 2: wave w takes k1 = 4 w + j
        {
            // conjugate input twiddles (each lane's own row k2 and column),
            // then the exchange into operands of both column halves
            uint4 bop[4][2][2];   // [j][h][ks]
            const int cl = 16 * (g & 1) + x;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int k2 = (q >> 3) * 16 + 8 * (g >> 1) + (q & 7);
                    const rfloat2 d = f2_from_h2(raw[j][q]);
                    const float2 v = cmulcf(make_float2(d.x, d.y), s_tw2[k2 * 32 + cl]);
                    raw[j][q] = pk2(v.x, v.y);
                }
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) swap16(raw[j][8 * ks + q], raw[j][8 * ks + q + 4]);
                    bop[j][0][ks] = make_uint4(raw[j][8 * ks], raw[j][8 * ks + 1], raw[j][8 * ks + 2], raw[j][8 * ks + 3]);
                    bop[j][1][ks] = make_uint4(raw[j][8 * ks + 4], raw[j][8 * ks + 5], raw[j][8 * ks + 6], raw[j][8 * ks + 7]);
                }
            }
            // the level-2 A operands one M-tile at a time (L2-resident): all
            // of them beside the operands of four tasks would not fit
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                uint4 a2[2][2];
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int hl = 0; hl < 2; ++hl) a2[ks][hl] = buf_ld16(rs_a2, lane * 16, (((mt * 2 + ks) * 2 + hl) * 64) * 16);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int c = 16 * h + x;
                    uint32_t v[2][4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int k1 = 4 * wave + j;
                        rfloat4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int ks = 0; ks < 2; ++ks) {
                            acc = mma_f16(a2[ks][0], bop[j][h][ks], acc);
                            acc = mma_f16(a2[ks][1], bop[j][h][ks], acc);
                        }
                        const float2 t1 = s_tw1[k1 * 32 + c];
#pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            const int n2 = 8 * mt + 2 * g + e;
                            const float2 tw = cmulf(s_twn[n2 * 32 + k1], t1);
                            const float2 a = cmulcf(make_float2(acc[2 * e], acc[2 * e + 1]), tw);
                            v[e][j] = pk2(a.x, a.y);
                        }
                    }
#pragma unroll
                    for (int e = 0; e < 2; ++e)
                        s_mid[mid(8 * mt + 2 * g + e, c, wave)] = make_uint4(v[e][0], v[e][1], v[e][2], v[e][3]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        __syncthreads();
        const long long tn_ = t + gridDim.x;
        const unsigned bq = (unsigned)r / (unsigned)prm.hc;
        const long long mrow = (long long)bq * prm.H + prm.h0 + ((unsigned)r - bq * (unsigned)prm.hc);
        // output gate at the stores' addresses: [j][mt][e][row n1, n1 + 2]
        uint32_t graw[G ? 4 : 1][2][2][2];
        if constexpr (G) {
            const uint32_t* gv = (const uint32_t*)prm.v + mrow * (M / 2) + c0 + 16 * (g & 1) + x;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int e = 0; e < 2; ++e)
#pragma unroll
                        for (int p2 = 0; p2 < 2; ++p2) {
                            const int n1 = 8 * mt + 4 * (g >> 1) + e + 2 * p2;
                            graw[j][mt][e][p2] = __builtin_nontemporal_load(
                                &gv[(long long)n1 * M2 + (long long)(4 * wave + j) * SLAB]);
                        }
        }
        uint4 a1[2][2][2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int hl = 0; hl < 2; ++hl) a1[mt][ks][hl] = buf_ld16(rs_a1, lane * 16, (((mt * 2 + ks) * 2 + hl) * 64) * 16);
        if (!G && tn_ < ntiles) {
            int c0n;
            tile_of(tn_, c0n);
            tw_load(c0n);
            fetch(tn_);
        }
        // ---------------- inverse level 1: wave w takes n2 = 4 w + j
        {
            uint32_t* y = (uint32_t*)prm.y + mrow * (M / 2) + c0 + 16 * (g & 1) + x;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n2 = 4 * wave + j;
                uint4 b[2][2];
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) b[h][ks] = s_mid[mid(n2, 16 * h + x, 4 * ks + g)];
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    uint32_t o[2][2];
                    if constexpr (G) {
                        // back to the layout of the results (the exchange
                        // below is its own inverse)
#pragma unroll
                        for (int e = 0; e < 2; ++e) swap16(graw[j][mt][e][0], graw[j][mt][e][1]);
                    }
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        rfloat4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int ks = 0; ks < 2; ++ks) {
                            acc = mma_f16(a1[mt][ks][0], b[h][ks], acc);
                            acc = mma_f16(a1[mt][ks][1], b[h][ks], acc);
                        }
#pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            if constexpr (G)
                                o[h][e] = pk2io<IO>(acc[2 * e] * io_lo<IO>(graw[j][mt][e][h]),
                                                    acc[2 * e + 1] * io_hi<IO>(graw[j][mt][e][h]));
                            else
                                o[h][e] = pk2io<IO>(acc[2 * e], acc[2 * e + 1]);
                        }
                    }
                    // rows n1 = 8 mt + 4 (g / 2) + e and + 2, whole lines
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        swap16(o[0][e], o[1][e]);
                        const int n1 = 8 * mt + 4 * (g >> 1) + e;
                        __builtin_nontemporal_store(o[0][e], &y[(long long)n1 * M2 + (long long)n2 * SLAB]);
                        __builtin_nontemporal_store(o[1][e], &y[(long long)(n1 + 2) * M2 + (long long)n2 * SLAB]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (G && tn_ < ntiles) {
            int c0n;
            tile_of(tn_, c0n);
            tw_load(c0n);
            fetch(tn_);
        }
        if (tn_ < ntiles) tw_store();
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Spectrum coefficients in the inner pass's engine order:
// [h][q < P_o/2][wave 4][region 2][kt 2][mt 4][lane 64][e 2], each
// (alpha, beta) as packed f16.  Region 0 of a wave holds its bin k; region 1
// holds conj(alpha_{-k}), conj(beta_{-k}) for the element-wise pairs, or,
// for wave 0 of the self unit, its own bin P_o (2 + 4 k').
__global__ void mp_coef_kernel(MpCoefParams P) {
    const int upr = P.Po / 2;
    const long long per_ch = (long long)upr * 8192;
    const long long total = (long long)P.hcount * per_ch;
    for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < total;
         i += (long long)gridDim.x * blockDim.x) {
        const long long hl = i / per_ch;
        const int rem = (int)(i - hl * per_ch);
        const int e = rem & 1;
        const int lane = (rem >> 1) & 63;
        const int mt = (rem >> 7) & 3;
        const int kt = (rem >> 9) & 1;
        const int reg = (rem >> 10) & 1;
        const int wave = (rem >> 11) & 3;
        const int q = rem >> 13;
        const int gg = lane >> 4, xx = lane & 15;
        const long long kp = kmap32(kt, xx) + 32 * rmid_perm(8 * mt + 2 * gg + e, 32);
        long long k;
        bool conj_neg = false;
        if (q == 0 && wave == 0) {
            k = (long long)P.Po * ((reg ? 2 : 0) + 4 * kp);
        } else {
            long long ko = q, j = wave;
            if (q == 0) {
                if (wave == 1) {
                    ko = 0;
                    j = 1;
                } else {
                    ko = P.Po / 2;
                    j = wave - 2;
                }
            }
            k = ko + (long long)P.Po * (j + 4 * kp);
            conj_neg = (reg == 1);
        }
        if (conj_neg) k = (P.M - k) % P.M;
        const float2* X = P.X + hl * P.L;
        const float2 K1 = X[k], K2 = X[k + P.M];
        double sn, cs;
        sincospi(2.0 * (double)k / (double)P.L, &sn, &cs);
        const float s = (float)sn, c = (float)cs;
        float2 al = make_float2(0.5f * ((1.f - s) * K1.x + (1.f + s) * K2.x),
                                0.5f * ((1.f - s) * K1.y + (1.f + s) * K2.y));
        const float2 dlt = make_float2(K1.x - K2.x, K1.y - K2.y);
        float2 be = make_float2(-0.5f * c * dlt.y, 0.5f * c * dlt.x);
        if (conj_neg) {
            al.y = -al.y;
            be.y = -be.y;
        }
        _Float16 hv[4] = {(_Float16)al.x, (_Float16)al.y, (_Float16)be.x, (_Float16)be.y};
        ((uint2*)P.kf)[(long long)(P.h0 + hl) * per_ch + rem] = *(const uint2*)hv;
    }
}

// ---------------------------------------------------------------------------
namespace {

template <int IO, int P>
hipError_t col_launch(int mode, const MpColParams& p, hipStream_t s) {
    const long long threads = p.rows * (long long)(p.M / P);
    const dim3 grid((unsigned)((threads + 255) / 256)), blk(256);
    if (p.full) {
        // rows at FFT size 2M: the first forward and the last inverse level
        if (mode == 0) hipLaunchKernelGGL((mp_col_kernel<IO, P, 0, true>), grid, blk, 0, s, p);
        else if (mode == 3) hipLaunchKernelGGL((mp_col_kernel<IO, P, 3, true>), grid, blk, 0, s, p);
        else return hipErrorInvalidValue;
        return hipGetLastError();
    }
    switch (mode) {
    case 0: hipLaunchKernelGGL((mp_col_kernel<IO, P, 0>), grid, blk, 0, s, p); break;
    case 1: hipLaunchKernelGGL((mp_col_kernel<IO, P, 1>), grid, blk, 0, s, p); break;
    case 2: hipLaunchKernelGGL((mp_col_kernel<IO, P, 2>), grid, blk, 0, s, p); break;
    case 4: hipLaunchKernelGGL((mp_col_kernel<IO, P, 4>), grid, blk, 0, s, p); break;
    case 5: hipLaunchKernelGGL((mp_col_kernel<IO, P, 5>), grid, blk, 0, s, p); break;
    default: hipLaunchKernelGGL((mp_col_kernel<IO, P, 3>), grid, blk, 0, s, p); break;
    }
    return hipGetLastError();
}

template <int IO>
hipError_t col_dispatch(int P, int mode, const MpColParams& p, hipStream_t s) {
    switch (P) {
    case 2: return col_launch<IO, 2>(mode, p, s);
    case 4: return col_launch<IO, 4>(mode, p, s);
    case 8: return col_launch<IO, 8>(mode, p, s);
    case 16: return col_launch<IO, 16>(mode, p, s);
    case 32: return col_launch<IO, 32>(mode, p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_mp_col(int io, int P, int mode, const MpColParams& p, hipStream_t s) {
    if (p.rows <= 0) return hipSuccess;
    // the kernel's index math: power-of-two M and S, whole blocks per row,
    // 32-bit thread indices
    const long long per_row = (long long)p.M / (P > 0 ? P : 1);
    if (P <= 0 || (p.M & (p.M - 1)) || (p.S & (p.S - 1)) || per_row % 256 ||
        p.rows * per_row > (1LL << 32))
        return hipErrorInvalidValue;
    return io == IO_BF16 ? col_dispatch<IO_BF16>(P, mode, p, s) : col_dispatch<IO_F16>(P, mode, p, s);
}

template <int IO, int P1, int P2>
hipError_t col2_launch(bool inv, const MpCol2Params& p, hipStream_t s) {
    const dim3 grid((unsigned)p.grid), blk(kCol2Threads);
    // 32 x 32 plans take the matrix-core passes; only their plain variant
    // of this kernel is kept (and no FFT-size variant: M = 4M is beyond the
    // longest circular plan)
    if constexpr (P1 == 32 && P2 == 32) {
        if (p.w || p.full) return hipErrorInvalidValue;
        if (inv) hipLaunchKernelGGL((mp_col2_kernel<IO, P1, P2, true, false, false>), grid, blk, 0, s, p);
        else hipLaunchKernelGGL((mp_col2_kernel<IO, P1, P2, false, false, false>), grid, blk, 0, s, p);
    } else if (p.full) {
        if (p.w) {
            if (inv) hipLaunchKernelGGL((mp_col2_kernel<IO, P1, P2, true, true, true>), grid, blk, 0, s, p);
            else hipLaunchKernelGGL((mp_col2_kernel<IO, P1, P2, false, true, true>), grid, blk, 0, s, p);
        } else {
            if (inv) hipLaunchKernelGGL((mp_col2_kernel<IO, P1, P2, true, false, true>), grid, blk, 0, s, p);
            else hipLaunchKernelGGL((mp_col2_kernel<IO, P1, P2, false, false, true>), grid, blk, 0, s, p);
        }
    } else if (p.w) {
        if (inv) hipLaunchKernelGGL((mp_col2_kernel<IO, P1, P2, true, true, false>), grid, blk, 0, s, p);
        else hipLaunchKernelGGL((mp_col2_kernel<IO, P1, P2, false, true, false>), grid, blk, 0, s, p);
    } else {
        if (inv) hipLaunchKernelGGL((mp_col2_kernel<IO, P1, P2, true, false, false>), grid, blk, 0, s, p);
        else hipLaunchKernelGGL((mp_col2_kernel<IO, P1, P2, false, false, false>), grid, blk, 0, s, p);
    }
    return hipGetLastError();
}

template <int IO>
hipError_t col2_dispatch(int P1, int P2, bool inv, const MpCol2Params& p, hipStream_t s) {
    switch (P1 * 64 + P2) {
    case 8 * 64 + 8: return col2_launch<IO, 8, 8>(inv, p, s);
    case 16 * 64 + 8: return col2_launch<IO, 16, 8>(inv, p, s);
    case 16 * 64 + 16: return col2_launch<IO, 16, 16>(inv, p, s);
    case 32 * 64 + 16: return col2_launch<IO, 32, 16>(inv, p, s);
    case 32 * 64 + 32: return col2_launch<IO, 32, 32>(inv, p, s);
    default: return hipErrorInvalidValue;
    }
}

long long mp_col2_tiles(int P2, long long rows) { return rows * (4096 / col2_cols(P2)); }

hipError_t launch_mp_col2(int io, int P1, int P2, bool inv, const MpCol2Params& p, hipStream_t s) {
    if (p.rows <= 0) return hipSuccess;
    if (p.grid <= 0 || p.grid % 16 || P2 > P1 || P1 > 2 * P2) return hipErrorInvalidValue;
    return io == IO_BF16 ? col2_dispatch<IO_BF16>(P1, P2, inv, p, s) : col2_dispatch<IO_F16>(P1, P2, inv, p, s);
}

template <int IO, bool G>
static hipError_t col2m_fwd_t(const MpCol2Params& p, hipStream_t s) {
    const hipError_t e = hipFuncSetAttribute((const void*)mp_col2m_fwd_kernel<IO, G>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, kCol2mLds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((mp_col2m_fwd_kernel<IO, G>), dim3((unsigned)p.grid), dim3(512), kCol2mLds, s, p);
    return hipGetLastError();
}

hipError_t launch_mp_col2m_fwd(int io, const MpCol2Params& p, hipStream_t s) {
    if (p.rows <= 0) return hipSuccess;
    if (p.grid <= 0 || p.M != 4194304 || !p.a1 || !p.a2 || !p.tm) return hipErrorInvalidValue;
    if (p.w) return io == IO_BF16 ? col2m_fwd_t<IO_BF16, true>(p, s) : col2m_fwd_t<IO_F16, true>(p, s);
    return io == IO_BF16 ? col2m_fwd_t<IO_BF16, false>(p, s) : col2m_fwd_t<IO_F16, false>(p, s);
}

template <int IO, bool G>
static hipError_t col2m_inv_t(const MpCol2Params& p, hipStream_t s) {
    const hipError_t e = hipFuncSetAttribute((const void*)mp_col2m_inv_kernel<IO, G>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, kCol2mLds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((mp_col2m_inv_kernel<IO, G>), dim3((unsigned)p.grid), dim3(512), kCol2mLds, s, p);
    return hipGetLastError();
}

hipError_t launch_mp_col2m_inv(int io, const MpCol2Params& p, hipStream_t s) {
    if (p.rows <= 0) return hipSuccess;
    if (p.grid <= 0 || p.M != 4194304 || !p.a1 || !p.a2 || !p.tm) return hipErrorInvalidValue;
    if (p.v) return io == IO_BF16 ? col2m_inv_t<IO_BF16, true>(p, s) : col2m_inv_t<IO_F16, true>(p, s);
    return io == IO_BF16 ? col2m_inv_t<IO_BF16, false>(p, s) : col2m_inv_t<IO_F16, false>(p, s);
}

hipError_t launch_mp_coef(const MpCoefParams& p, hipStream_t s) {
    hipLaunchKernelGGL(mp_coef_kernel, dim3(2048), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace fftconv
