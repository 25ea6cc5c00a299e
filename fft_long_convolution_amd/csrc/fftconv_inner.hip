// Inner pass of the multi-pass path (page "FlashFFTConv: Efficient
// Convolutions for Long Sequences with Tensor Cores", sections 3.2 and 3.4):
// units of two 4096-point slabs of the f16 workspace go through the 4-point
// outer stage and the 4 x 32 x 32 engine with the spectrum product, and back.
// The slab algebra (mirror pairing across slabs) is described with the
// column passes in fftconv_mp.hip.  Compiled with the max-ILP scheduling
// strategy (measured faster for this kernel only).
#include "fftconv_engine.h"

namespace fftconv {

using namespace eng;

// ---------------------------------------------------------------------------
// Inner pass: persistent workgroups of four waves, one unit (two 4096-point
// slabs, eight 1024-point regions) at a time.
//   pair unit (slabs of k_o and P_o - k_o):  wave j holds region 2j = slab
//     A sub-row j (4-point DFT output j, twiddle w_j) and region 2j + 1 =
//     conj(slab B output 3 - j) w_{j+1}; the pairing is element-wise.
//   self unit (slabs 0 and P_o/2): regions 0..3 are slab 0 laid out like a
//     fused row of the wide kernel (wave 0: sub-rows 0 and 2 pair within
//     themselves, wave 1: sub-row 1 and conj(sub-row 3) w_1); regions 4..7
//     are slab P_o/2 sub-rows 0, 1 with conj(output 3) w_1 and
//     conj(output 2) w_2.
// The inner outer stage as one 16 x 16 x 16 matrix product per 16 columns.
// Region r of a unit is (conj or not) output k of the 4-point DFT of one of
// its two slabs; the twiddle of region r is W_4096^{n' m(r)}.
//   pair unit: r = 2m -> slab A, k = m; r = 2m + 1 -> conj(slab B, k = 3 - m);
//              m(r) = (r + 1) / 2
//   self unit: r -> (slab, k, conj) = (0,0) (0,2) (0,1) (0,3)* (1,0) (1,3)*
//              (1,1) (1,2)*;  m(r) = 0 2 1 1 0 1 1 2
// The DFT entries are 0, +-1, +-i, exact in f16, so the product (fp32
// accumulate) is as exact as the same sums in fp32.
__device__ __forceinline__ void region_map(bool self, int r, int& slab, int& k, bool& cj) {
    if (!self) {
        slab = r & 1;
        k = (r & 1) ? 3 - (r >> 1) : (r >> 1);
        cj = (r & 1) != 0;
    } else {
        constexpr int ks = 0x21303120;     // k of r = 0..7, 4 bits each
        slab = r >> 2;
        k = (ks >> (4 * r)) & 15;
        cj = (r == 3) || (r == 5) || (r == 7);
    }
}
__device__ __forceinline__ int region_twiddle(bool self, int r) {
    return self ? (0x21101120 >> (4 * r)) & 15 : (r + 1) >> 1;
}
// Real matrix entry: complex coefficient W_4^{e} on an input taken as is or
// conjugated; ro/ki = real (0) or imaginary (1) part of output/input.
__device__ __forceinline__ float w4_entry(int e, bool cj, int ro, int ki) {
    const int q = e & 3;
    const float wr = q == 0 ? 1.f : (q == 2 ? -1.f : 0.f);
    const float wi = q == 1 ? -1.f : (q == 3 ? 1.f : 0.f);
    if (!cj) return ro == 0 ? (ki == 0 ? wr : -wi) : (ki == 0 ? wi : wr);
    return ro == 0 ? (ki == 0 ? wr : wi) : (ki == 0 ? wi : -wr);
}
// A operand (rows = outputs, K = inputs; real/imaginary interleaved) of lane
// (g, x): row x, K columns 4g..4g+3.  Forward: inputs = slab values
// 4 slab + n1, outputs = regions.  Inverse: inputs = regions after their
// conjugate twiddle, outputs = slab values.
__device__ __forceinline__ uint2 outer4_a(bool self, bool inv, int g, int x) {
    _Float16 h[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int o = x >> 1, ro = x & 1, c = 2 * g + (j >> 1), ki = j & 1;
        float v = 0.f;
        int slab, k;
        bool cj;
        if (!inv) {
            region_map(self, o, slab, k, cj);
            if ((c >> 2) == slab) v = w4_entry(cj ? -(c & 3) * k : (c & 3) * k, cj, ro, ki);
        } else {
            region_map(self, c, slab, k, cj);
            if ((o >> 2) == slab) v = w4_entry(-(o & 3) * k, cj, ro, ki);
        }
        h[j] = (_Float16)v;
    }
    return __builtin_bit_cast(uint2, h);
}
__device__ __forceinline__ rfloat4 mma16_f16(uint2 a, uint2 b) {
    typedef _Float16 rhalf4 __attribute__((ext_vector_type(4)));
    const rfloat4 z = {0.f, 0.f, 0.f, 0.f};
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(rhalf4, a),
                                                 __builtin_bit_cast(rhalf4, b), z, 0, 0, 0);
}

template <int IO, bool SK>
__global__ void __launch_bounds__(256, 2) mp_inner_kernel(MpInnerParams prm) {
    constexpr int Q = 1024, T = 256, SLAB = 4096;

    extern __shared__ uint4 s_lds[];
    uint4* s_f1b = s_lds;                              // [ks 2][jt 4][64]
    uint4* s_i1a = s_f1b + 8 * 64;                     // [mt 4][ks 2][64]
    uint32_t* s_two = (uint32_t*)(s_i1a + 8 * 64);     // W_4096^{n' m}, [m 5][engine position]
    uint32_t* s_buf = s_two + 5 * Q;                   // [8 regions][Q]
    uint32_t* s_scr = s_buf + 8 * Q;                   // [39 k_b slots][16 x]
    int* s_claim = (int*)(s_scr + 39 * 16);            // [2] claimed unit indices
    uint2* s_aop = (uint2*)(s_claim + 4);              // outer-stage A operands [4][64]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, x = lane & 15;
    const int upr = prm.Po / 2;                        // units per row
    // units q >= upr_active hold only zeroed bins (a frequency-sparse call)
    // and are not computed: the claimed index runs over the others
    const int upa = prm.upr_active;
    const int total = prm.B * prm.hc * upa;
    // unit index (hl * upr + q) * B + b: the B units that share spectrum
    // coefficients are neighbours; units are claimed one ahead from the
    // counters of this workgroup's XCD group (as in the wide kernel)
    const XcdClaim claimer(prm.ctr, gridDim.x, blockIdx.x);
    // the workspace chunk through one buffer descriptor (no 64-bit per-lane
    // addresses; the chunk is at most 256 MB)
    const __amdgpu_buffer_rsrc_t rws = buf_rsrc(prm.ws, -1);

    for (int i = tid; i < 8 * 64; i += T) {
        s_f1b[i] = ((const uint4*)prm.f1b)[i];
        s_i1a[i] = ((const uint4*)prm.i1a)[i];
    }
    for (int i = tid; i < 5 * Q / 4; i += T) ((uint4*)s_two)[i] = ((const uint4*)prm.two)[i];
    if (tid == 0) {
        const long long c0 = claimer.next(), c1 = claimer.next();
        s_claim[0] = (int)(c0 < total ? c0 : total);
        s_claim[1] = (int)(c1 < total ? c1 : total);
    }
    Regs E;
    load_regs(E, prm.f2a, SK ? prm.i2bs : prm.i2b, prm.twf, lane);

    // outer stage: each wave takes 16 column tiles of 16 columns; lane (g, x)
    // holds slab g / 2, rows n1 = 2 (g % 2) + e of column x, and after the
    // product regions 2 g + e
    const int sl_g = g >> 1;
    // A operands [inverse][self] of every lane, read once per unit and stage
    if (tid < 64) {
#pragma unroll
        for (int v = 0; v < 4; ++v) s_aop[v * 64 + lane] = outer4_a(v & 1, v >> 1, g, x);
    }
    constexpr int TPW = 16;                            // column tiles per wave
    // Tile i = 4 blk + k of wave w holds the 16 columns n' = 32 n_a + n_b with
    // n_a = 8 w + 4 (blk / 2) + k and n_b = 16 (blk % 2) + x: after the four
    // tiles of a block, lane (g, x) has four consecutive n_a of one n_b,
    // which the engine layout keeps in one 16-byte word (conflict-free
    // 128-bit LDS accesses, the twiddle table in the same layout).
    // 16-byte word of block blk in a region; recomputed where used (the
    // empty asm keeps the compiler from hoisting four more live registers
    // out of the unit loop)
    auto buf_word = [&](int blk) {
        int xv = x;
        asm volatile("" : "+v"(xv));
        const int xx1 = xv == 0 ? 0 : 16 - xv;
        return eng_addr(8 * wave + 4 * (blk >> 1), blk & 1, (blk & 1) ? xx1 : xv) >> 2;
    };
    auto col_of = [&](int i) { return 32 * (8 * wave + 4 * (i >> 3) + (i & 3)) + 16 * ((i >> 2) & 1) + x; };
    // P1 and the units per row are powers of two: shifts and masks
    const int lg_p1 = __builtin_ctz((unsigned)prm.P1), lg_upr = __builtin_ctz((unsigned)upr);
    auto sigma = [&](int ko) { return (ko & (prm.P1 - 1)) * prm.P2 + (ko >> lg_p1); };
    // unit -> (row, q, slabs)
    // row is the workspace row of the unit (b * hc + local channel), h the
    // channel (its spectrum coefficients)
    auto unit_rows = [&](int idx, long long& row, int& h, int& q, int& sa, int& sb) {
        const int hq = (int)((unsigned)idx / (unsigned)prm.B), b = idx - hq * prm.B;
        int hl;
        if (upa == upr) {
            hl = hq >> lg_upr;
            q = hq & (upr - 1);
        } else {
            hl = (int)((unsigned)hq / (unsigned)upa);
            q = hq - hl * upa;
        }
        h = prm.h0 + hl;
        row = (long long)b * prm.hc + hl;
        sa = sigma(q);
        sb = sigma(q == 0 ? prm.Po / 2 : prm.Po - q);
    };
    uint2 xin[TPW];            // [tile]: rows 2 (g % 2) + e of slab g / 2 (after the exchange)
    auto load_in = [&](int idx) {
        long long row;
        int h, q, sa, sb;
        unit_rows(idx, row, h, q, sa, sb);
        // tiles i (n_b < 16) and i + 4 (n_b >= 16) share 128-byte lines: lane
        // groups g and g + 1 load the two halves of rows 0..3 of slab g / 2,
        // and one exchange between 16-lane rows turns them into the operands
        // of both tiles (whole lines per load)
        // buffer loads: the row in a scalar offset, the lane's slab and
        // column in one 32-bit register, the tile in the immediate
        const int srow = (int)(row * prm.M * 4);
        const unsigned vs = (unsigned)(((sl_g ? sb : sa) * SLAB + col_of(0) + 16 * (g & 1)) * 4);
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            if ((i >> 2) & 1) continue;
            const int d = 4 * (col_of(i) - col_of(0));     // compile-time
            uint32_t r0 = __builtin_amdgcn_raw_buffer_load_b32(rws, vs + d, srow, 2);
            uint32_t r1 = __builtin_amdgcn_raw_buffer_load_b32(rws, vs + d, srow + 4 * Q, 2);
            uint32_t r2 = __builtin_amdgcn_raw_buffer_load_b32(rws, vs + d, srow + 8 * Q, 2);
            uint32_t r3 = __builtin_amdgcn_raw_buffer_load_b32(rws, vs + d, srow + 12 * Q, 2);
            xin[i].x = r0;
            xin[i].y = r1;
            xin[i + 4].x = r2;
            xin[i + 4].y = r3;
        }
    };
    __syncthreads();
    int cur = s_claim[0], nxt = s_claim[1];
    if (cur >= total) return;   // uniform over the workgroup
    load_in(cur);

    uint32_t* scr = s_scr + x;
    const int i1_base = (16 * (g >> 1) + x) * 4 + 2 * (g & 1);

    while (cur < total) {
        long long row;
        int h, q, sa, sb;
        unit_rows(cur, row, h, q, sa, sb);
        const bool self = (q == 0);
        const int inext = nxt < total ? nxt : cur;
        // ---------------- inner outer stage: 4-point DFTs of both slabs on
        // the matrix cores, twiddles in packed f16, into the engine's layout
        {
#pragma unroll
            for (int i = 0; i < TPW; ++i) {
                if ((i >> 2) & 1) continue;
                swap16(xin[i].x, xin[i + 4].x);
                swap16(xin[i].y, xin[i + 4].y);
            }
            const uint2 af = s_aop[(self ? 1 : 0) * 64 + lane];
            const uint4* tw0 = (const uint4*)(s_two + region_twiddle(self, 2 * g) * Q);
            const uint4* tw1 = (const uint4*)(s_two + region_twiddle(self, 2 * g + 1) * Q);
            uint4* b0 = (uint4*)(s_buf + 2 * g * Q);
            uint4* b1 = (uint4*)(s_buf + (2 * g + 1) * Q);
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
                uint32_t v0[4], v1[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const rfloat4 c = mma16_f16(af, xin[4 * blk + k]);
                    v0[k] = pk2(c[0], c[1]);
                    v1[k] = pk2(c[2], c[3]);
                }
                const int w4 = buf_word(blk);
                const uint4 t0 = tw0[w4], t1 = tw1[w4];
                const uint32_t t0a[4] = {t0.x, t0.y, t0.z, t0.w}, t1a[4] = {t1.x, t1.y, t1.z, t1.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    v0[k] = as_u32(hmul(as_h2(v0[k]), as_h2(t0a[k])));
                    v1[k] = as_u32(hmul(as_h2(v1[k]), as_h2(t1a[k])));
                }
                b0[w4] = make_uint4(v0[0], v0[1], v0[2], v0[3]);
                b1[w4] = make_uint4(v1[0], v1[1], v1[2], v1[3]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // claim the row after next now: the atomic returns long before the
        // value is published, and it is older than the loads it must not
        // delay
        long long c2 = 0;
        if (tid == 0) c2 = claimer.next();
        __syncthreads();

        // ---------------- engine: regions 2*wave and 2*wave + 1
        {
            const uint4* cf = (const uint4*)prm.kf + (((long long)h * upr + q) * 4 + wave) * 1024;
            uint4 cfr[2][2][4];   // [region][kt][mt]
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) cfr[s][0][mt] = cf[(s * 2) * 256 + mt * 64 + lane];
            uint32_t z[2][2][4][2];
            forward<SK>(s_buf + (2 * wave) * Q, s_f1b, E, lane, z[0]);
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) cfr[s][1][mt] = cf[(s * 2 + 1) * 256 + mt * 64 + lane];
            __builtin_amdgcn_sched_barrier(0);
            forward<SK>(s_buf + (2 * wave + 1) * Q, s_f1b, E, lane, z[1]);
            __builtin_amdgcn_sched_barrier(0);

            uint4 a2[2][2][2];
            if (self && wave == 0) {
                uint32_t zq[4][2];
                self_exchange(z[0], scr, g, zq);
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    pair_self<SK>(kt, x == 0, z[0], z[1], zq, cfr[0][kt], cfr[1][kt], a2[0][kt], a2[1][kt]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    pair_elem<SK>(kt, z[0], z[1], cfr[0][kt], cfr[1][kt], a2[0][kt], a2[1][kt]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            // publish the unit after next; then the next unit's input (after
            // the coefficient loads: the load counter retires in order)
            if (tid == 0) s_claim[0] = (int)(c2 < total ? c2 : total);
            load_in(inext);

            inverse<SK>(a2[0], s_i1a, E, lane, i1_base, s_buf + (2 * wave) * Q);
            __builtin_amdgcn_sched_barrier(0);
            inverse<SK>(a2[1], s_i1a, E, lane, i1_base, s_buf + (2 * wave + 1) * Q);
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
        const int nn = s_claim[0];
        // ---------------- inverse inner outer stage (conjugate twiddles in
        // packed f16, 4-point inverse DFTs on the matrix cores), back to the
        // workspace
        {
            const uint2 ai = s_aop[(self ? 3 : 2) * 64 + lane];
            const uint4* tw0 = (const uint4*)(s_two + region_twiddle(self, 2 * g) * Q);
            const uint4* tw1 = (const uint4*)(s_two + region_twiddle(self, 2 * g + 1) * Q);
            const uint4* b0 = (const uint4*)(s_buf + 2 * g * Q);
            const uint4* b1 = (const uint4*)(s_buf + (2 * g + 1) * Q);
            const int srow = (int)(row * prm.M * 4);
            const unsigned vs = (unsigned)(((sl_g ? sb : sa) * SLAB + col_of(0) + 16 * (g & 1)) * 4);
#pragma unroll
            for (int nah = 0; nah < 2; ++nah) {
                uint32_t o[2][4][2];   // [n_b half][k][e]
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int blk = 2 * nah + h;
                    const int w4 = buf_word(blk);
                    const uint4 r0 = b0[w4], r1 = b1[w4], t0 = tw0[w4], t1 = tw1[w4];
                    const uint32_t r0a[4] = {r0.x, r0.y, r0.z, r0.w}, r1a[4] = {r1.x, r1.y, r1.z, r1.w};
                    const uint32_t t0a[4] = {t0.x, t0.y, t0.z, t0.w}, t1a[4] = {t1.x, t1.y, t1.z, t1.w};
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        uint2 bv;
                        bv.x = as_u32(hmulc(as_h2(r0a[k]), as_h2(t0a[k])));
                        bv.y = as_u32(hmulc(as_h2(r1a[k]), as_h2(t1a[k])));
                        const rfloat4 c = mma16_f16(ai, bv);
                        o[h][k][0] = pk2(c[0], c[1]);
                        o[h][k][1] = pk2(c[2], c[3]);
                    }
                }
                // lane group g holds rows n1 = 2 (g % 2) + e of both halves:
                // exchange so that each store covers whole 128-byte lines
                // (rows 0..3 of slab g / 2, half g % 2)
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    swap16(o[0][k][0], o[1][k][0]);
                    swap16(o[0][k][1], o[1][k][1]);
                    const int d = col_of(8 * nah + k) - col_of(0);   // compile-time
                    __builtin_amdgcn_raw_buffer_store_b32(o[0][k][0], rws, vs + 4 * d, srow, 2);
                    __builtin_amdgcn_raw_buffer_store_b32(o[0][k][1], rws, vs + 4 * d, srow + 4 * Q, 2);
                    __builtin_amdgcn_raw_buffer_store_b32(o[1][k][0], rws, vs + 4 * d, srow + 8 * Q, 2);
                    __builtin_amdgcn_raw_buffer_store_b32(o[1][k][1], rws, vs + 4 * d, srow + 12 * Q, 2);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        cur = nxt;
        nxt = nn;
    }
}

// ---------------------------------------------------------------------------
// Kernel gradient on the same units (page "FlashFFTConv: Efficient
// Convolutions for Long Sequences with Tensor Cores", section 3: gradients
// of an FFT convolution multiply by conjugate spectra; the input spectra are
// recomputed, not kept).  One workgroup per (local channel hl, unit q): for
// every batch row b the unit of u and of dy (workspace rows b * hc + hl,
// after the forward column passes) goes through the 4-point stage and the
// engine's forward transform, exactly as in the inner pass; the packed
// gradient spectrum G = sum_b conj(U_b) DY_b is accumulated in fp32
// registers, in the same element-wise pair form as the forward pairing:
// with a, d the values of u and dy at a bin k of the wave's first region
// and c, e the conjugated mirror values its second region holds there,
//   4 Z_g[k]       = 2 conj(E2) d + conj(O') (Od' - W Ed2)
//   4 conj Z_g[-k] = 2 conj(E2) e + conj(O') (Od' + W Ed2)
// (E2 = a + c, O' = a - c, Ed2 = d + e, Od' = d - e, W = exp(2 pi i k / M)),
// and wave 0 of the self unit pairs within its regions (k' <-> -k' through
// LDS, k' <-> 1023 - k' one lane over).  Bin k of a position is
// k_o + P_o (j + 4 k'), so W is the position's exp(2 pi i k' / 1024) times a
// factor of the (unit, wave, region).  The result goes through the engine's
// inverse and the inverse 4-point stage into result row hl.
template <int IO, bool ONE, bool SELF>
__global__ void __launch_bounds__(256, 2) kgrad_mp_kernel(KgMpParams prm) {
    constexpr int Q = 1024, T = 256, SLAB = 4096;

    extern __shared__ uint4 s_lds[];
    uint4* s_f1b = s_lds;                              // [ks 2][jt 4][64]
    uint4* s_i1a = s_f1b + 8 * 64;                     // [mt 4][ks 2][64]
    uint32_t* s_two = (uint32_t*)(s_i1a + 8 * 64);     // W_4096^{n' m}, [m 5][engine position]
    uint32_t* s_buf = s_two + 5 * Q;                   // [8 regions][Q]
    uint32_t* s_scr = s_buf + 8 * Q;                   // [u, dy][39 k_b slots][16 x]
    uint32_t* s_wb = s_scr + 2 * 39 * 16;              // [kt][mt][e][lane] exp(2 pi i k'/1024)
    uint2* s_aop = (uint2*)(s_wb + 16 * 64);           // outer-stage A operands [4][64]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, x = lane & 15;
    const int upr = prm.Po / 2;
    const int lg_p1 = __builtin_ctz((unsigned)prm.P1);
    // SELF: the self units (q = 0, one per channel); otherwise units 1 ..
    // P_o/2 - 1 of every channel
    int hl = (int)blockIdx.x, q = 0;
    if constexpr (!SELF) {
        hl = (int)(blockIdx.x / (unsigned)(upr - 1));
        q = 1 + (int)blockIdx.x - hl * (upr - 1);
    }
    constexpr bool self = SELF;
    auto sigma = [&](int ko) { return (ko & (prm.P1 - 1)) * prm.P2 + (ko >> lg_p1); };
    const int sa = sigma(q), sb = sigma(q == 0 ? prm.Po / 2 : prm.Po - q);
    const __amdgpu_buffer_rsrc_t ru = buf_rsrc(prm.wsu, -1), rd = buf_rsrc(prm.wsd, -1),
                                 rg = buf_rsrc(prm.wsg, -1);

    for (int i = tid; i < 8 * 64; i += T) {
        s_f1b[i] = ((const uint4*)prm.f1b)[i];
        s_i1a[i] = ((const uint4*)prm.i1a)[i];
    }
    for (int i = tid; i < 5 * Q / 4; i += T) ((uint4*)s_two)[i] = ((const uint4*)prm.two)[i];
    if (tid < 64) {
#pragma unroll
        for (int v = 0; v < 4; ++v) s_aop[v * 64 + lane] = outer4_a(v & 1, v >> 1, g, x);
    } else if (tid < 128) {
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
    Regs E;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) E.f2a[mt][ks] = ((const uint4*)prm.f2a)[(mt * 2 + ks) * 64 + lane];
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) E.twf[it][kt][r] = prm.twf[lane * 16 + (it * 2 + kt) * 4 + r];

    // W factor of the wave's regions: bin k = k_o + P_o (j + 4 k') with
    // (k_o, j) the wave's (slab outer bin, 4-point output); wave 0 of the
    // self unit: k = P_o (0 + 4 k') and P_o (2 + 4 k')
    uint32_t wsub[2];
    {
        int ko = q, j = wave;
        if (self) {
            if (wave == 1) {
                ko = 0;
                j = 1;
            } else if (wave >= 2) {
                ko = prm.Po / 2;
                j = wave - 2;
            }
        }
        const float inv_m = 1.f / (float)prm.M;
        float sn, cs;
        if (self && wave == 0) {
            sincospif(2.f * (float)(2 * prm.Po) * inv_m, &sn, &cs);
            wsub[0] = pk2(1.f, 0.f);
            wsub[1] = pk2(cs, sn);
        } else {
            sincospif(2.f * (float)(ko + prm.Po * j) * inv_m, &sn, &cs);
            wsub[0] = wsub[1] = pk2(cs, sn);
        }
    }

    // ---- geometry of the 4-point stage (as the inner pass)
    const int sl_g = g >> 1;
    constexpr int TPW = 16;
    auto buf_word = [&](int blk) {
        int xv = x;
        asm volatile("" : "+v"(xv));
        const int xx1 = xv == 0 ? 0 : 16 - xv;
        return eng_addr(8 * wave + 4 * (blk >> 1), blk & 1, (blk & 1) ? xx1 : xv) >> 2;
    };
    auto col_of = [&](int i) { return 32 * (8 * wave + 4 * (i >> 3) + (i & 3)) + 16 * ((i >> 2) & 1) + x; };
    const unsigned vs = (unsigned)(((sl_g ? sb : sa) * SLAB + col_of(0) + 16 * (g & 1)) * 4);
    // forward 4-point stage of workspace row `row` of buffer r into s_buf
    auto outer_fwd = [&](__amdgpu_buffer_rsrc_t r, int row) {
        uint2 xin[TPW];
        const int srow = (int)(row * prm.M * 4);
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            if ((i >> 2) & 1) continue;
            const int d = 4 * (col_of(i) - col_of(0));
            xin[i].x = __builtin_amdgcn_raw_buffer_load_b32(r, vs + d, srow, 2);
            xin[i].y = __builtin_amdgcn_raw_buffer_load_b32(r, vs + d, srow + 4 * Q, 2);
            xin[i + 4].x = __builtin_amdgcn_raw_buffer_load_b32(r, vs + d, srow + 8 * Q, 2);
            xin[i + 4].y = __builtin_amdgcn_raw_buffer_load_b32(r, vs + d, srow + 12 * Q, 2);
        }
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            if ((i >> 2) & 1) continue;
            swap16(xin[i].x, xin[i + 4].x);
            swap16(xin[i].y, xin[i + 4].y);
        }
        const uint2 af = s_aop[(self ? 1 : 0) * 64 + lane];
        const uint4* tw0 = (const uint4*)(s_two + region_twiddle(self, 2 * g) * Q);
        const uint4* tw1 = (const uint4*)(s_two + region_twiddle(self, 2 * g + 1) * Q);
        uint4* b0 = (uint4*)(s_buf + 2 * g * Q);
        uint4* b1 = (uint4*)(s_buf + (2 * g + 1) * Q);
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            uint32_t v0[4], v1[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const rfloat4 c = mma16_f16(af, xin[4 * blk + k]);
                v0[k] = pk2(c[0], c[1]);
                v1[k] = pk2(c[2], c[3]);
            }
            const int w4 = buf_word(blk);
            const uint4 t0 = tw0[w4], t1 = tw1[w4];
            const uint32_t t0a[4] = {t0.x, t0.y, t0.z, t0.w}, t1a[4] = {t1.x, t1.y, t1.z, t1.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                v0[k] = as_u32(hmul(as_h2(v0[k]), as_h2(t0a[k])));
                v1[k] = as_u32(hmul(as_h2(v1[k]), as_h2(t1a[k])));
            }
            b0[w4] = make_uint4(v0[0], v0[1], v0[2], v0[3]);
            b1[w4] = make_uint4(v1[0], v1[1], v1[2], v1[3]);
        }
    };
    __syncthreads();

    // fp32 sums over the batch, or with a batch of one the scaled products
    // straight into the inverse operands
    float2 acc[ONE ? 1 : 2][2][4][2];   // [region][kt][mt][e]
    uint32_t pz1[ONE ? 2 : 1][2][4][2];
    if constexpr (!ONE) {
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int e = 0; e < 2; ++e) acc[r][kt][mt][e] = make_float2(0.f, 0.f);
    }
    auto add = [&](int r, int kt, int mt, int e, rhalf2 R) {
        if constexpr (ONE) {
            pz1[r][kt][mt][e] = pk2((float)R.x * prm.pre, (float)R.y * prm.pre);
        } else {
            acc[r][kt][mt][e].x += (float)R.x;
            acc[r][kt][mt][e].y += (float)R.y;
        }
    };
    uint32_t* scr_u = s_scr + x;
    uint32_t* scr_d = s_scr + 39 * 16 + x;
    for (int b = 0; b < (ONE ? 1 : prm.B); ++b) {
        const int row = b * prm.hc + hl;
        uint32_t zu[2][2][4][2], zd[2][2][4][2];   // [region][kt][mt][e]
        outer_fwd(ru, row);
        __syncthreads();
        forward(s_buf + (2 * wave) * Q, s_f1b, E, lane, zu[0]);
        forward(s_buf + (2 * wave + 1) * Q, s_f1b, E, lane, zu[1]);
        __syncthreads();
        outer_fwd(rd, row);
        __syncthreads();
        forward(s_buf + (2 * wave) * Q, s_f1b, E, lane, zd[0]);
        forward(s_buf + (2 * wave + 1) * Q, s_f1b, E, lane, zd[1]);
        if (!(self && wave == 0)) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const rhalf2 W = hmul(as_h2(s_wb[((kt * 4 + mt) * 2 + e) * 64 + lane]), as_h2(wsub[0]));
                        rhalf2 RX, RY;
                        kg_pair(zu[0][kt][mt][e], zu[1][kt][mt][e], zd[0][kt][mt][e], zd[1][kt][mt][e], W,
                                RX, RY);
                        add(0, kt, mt, e, RX);
                        add(1, kt, mt, e, RY);
                    }
        } else {
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
                        const uint32_t rpu = kt == 0 ? rot_up(zu[1][1][pm][e]) : rot_down(zu[1][0][pm][e]);
                        const uint32_t rpd = kt == 0 ? rot_up(zd[1][1][pm][e]) : rot_down(zd[1][0][pm][e]);
                        const rhalf2 W0 = as_h2(s_wb[((kt * 4 + mt) * 2 + e) * 64 + lane]);
                        const rhalf2 W1 = hmul(W0, as_h2(wsub[1]));
                        const rhalf2 R0 = kg_self(zu[0][kt][mt][e], nu, zd[0][kt][mt][e], nd, W0);
                        const rhalf2 R1 = kg_self(zu[1][kt][mt][e], rpu, zd[1][kt][mt][e], rpd, W1);
                        add(0, kt, mt, e, R0);
                        add(1, kt, mt, e, R1);
                    }
                }
        }
        __syncthreads();
    }

    // ---- inverse of the accumulated spectrum: engine, then the 4-point stage
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) E.i2b[ks][jt] = ((const uint4*)prm.i2b)[(ks * 4 + jt) * 64 + lane];
    uint4 a2[2][2][2];   // [region][kt][ks]
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            uint32_t pz[4][2];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    if constexpr (ONE)
                        pz[mt][e] = pz1[r][kt][mt][e];
                    else
                        pz[mt][e] = pk2(acc[r][kt][mt][e].x * prm.pre, acc[r][kt][mt][e].y * prm.pre);
                }
            pack_a2(pz, a2[r][kt]);
        }
    const int i1_base = (16 * (g >> 1) + x) * 4 + 2 * (g & 1);
    inverse(a2[0], s_i1a, E, lane, i1_base, s_buf + (2 * wave) * Q);
    inverse(a2[1], s_i1a, E, lane, i1_base, s_buf + (2 * wave + 1) * Q);
    __syncthreads();
    {
        const uint2 ai = s_aop[(self ? 3 : 2) * 64 + lane];
        const uint4* tw0 = (const uint4*)(s_two + region_twiddle(self, 2 * g) * Q);
        const uint4* tw1 = (const uint4*)(s_two + region_twiddle(self, 2 * g + 1) * Q);
        const uint4* b0 = (const uint4*)(s_buf + 2 * g * Q);
        const uint4* b1 = (const uint4*)(s_buf + (2 * g + 1) * Q);
        const int srow = (int)(hl * prm.M * 4);
#pragma unroll
        for (int nah = 0; nah < 2; ++nah) {
            uint32_t o[2][4][2];   // [n_b half][k][e]
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int blk = 2 * nah + h;
                const int w4 = buf_word(blk);
                const uint4 r0 = b0[w4], r1 = b1[w4], t0 = tw0[w4], t1 = tw1[w4];
                const uint32_t r0a[4] = {r0.x, r0.y, r0.z, r0.w}, r1a[4] = {r1.x, r1.y, r1.z, r1.w};
                const uint32_t t0a[4] = {t0.x, t0.y, t0.z, t0.w}, t1a[4] = {t1.x, t1.y, t1.z, t1.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    uint2 bv;
                    bv.x = as_u32(hmulc(as_h2(r0a[k]), as_h2(t0a[k])));
                    bv.y = as_u32(hmulc(as_h2(r1a[k]), as_h2(t1a[k])));
                    const rfloat4 c = mma16_f16(ai, bv);
                    o[h][k][0] = pk2(c[0], c[1]);
                    o[h][k][1] = pk2(c[2], c[3]);
                }
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                swap16(o[0][k][0], o[1][k][0]);
                swap16(o[0][k][1], o[1][k][1]);
                const int d = col_of(8 * nah + k) - col_of(0);
                __builtin_amdgcn_raw_buffer_store_b32(o[0][k][0], rg, vs + 4 * d, srow, 2);
                __builtin_amdgcn_raw_buffer_store_b32(o[0][k][1], rg, vs + 4 * d, srow + 4 * Q, 2);
                __builtin_amdgcn_raw_buffer_store_b32(o[1][k][0], rg, vs + 4 * d, srow + 8 * Q, 2);
                __builtin_amdgcn_raw_buffer_store_b32(o[1][k][1], rg, vs + 4 * d, srow + 12 * Q, 2);
            }
        }
    }
}

int kgrad_mp_lds() {
    return 16 * 64 * 16 + (5 + 8) * 1024 * 4 + 2 * 39 * 16 * 4 + 16 * 64 * 4 + 4 * 64 * 8;
}

template <int IO, bool ONE>
static hipError_t kgrad_mp_t(const KgMpParams& p, long long grid, hipStream_t s) {
    const int lds = kgrad_mp_lds();
    hipError_t e = hipFuncSetAttribute((const void*)kgrad_mp_kernel<IO, ONE, true>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e == hipSuccess)
        e = hipFuncSetAttribute((const void*)kgrad_mp_kernel<IO, ONE, false>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    // the self units (one per channel, the longer workgroups: their wave 0
    // pairs within its regions) first, then the pair units
    hipLaunchKernelGGL((kgrad_mp_kernel<IO, ONE, true>), dim3((unsigned)p.hc), dim3(256), lds, s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long npair = grid - p.hc;
    hipLaunchKernelGGL((kgrad_mp_kernel<IO, ONE, false>), dim3((unsigned)npair), dim3(256), lds, s, p);
    return hipGetLastError();
}

hipError_t launch_kgrad_mp(int io, const KgMpParams& p, hipStream_t s) {
    if (p.hc <= 0 || p.B <= 0) return hipSuccess;
    const int upr = p.Po / 2;
    if (p.Po < 8 || (p.Po & (p.Po - 1)) || (p.P1 & (p.P1 - 1)) || p.P1 * p.P2 != p.Po ||
        p.M != p.Po * 4096)
        return hipErrorInvalidValue;
    const long long grid = (long long)p.hc * upr;
    // buffer offsets of the workspace rows stay within 31 bits
    if (grid > 0x7fffffffLL || (long long)p.B * p.hc * p.M * 4 > 0x7fffffffLL) return hipErrorInvalidValue;
    if (io == IO_BF16)
        return p.B == 1 ? kgrad_mp_t<IO_BF16, true>(p, grid, s) : kgrad_mp_t<IO_BF16, false>(p, grid, s);
    return p.B == 1 ? kgrad_mp_t<IO_F16, true>(p, grid, s) : kgrad_mp_t<IO_F16, false>(p, grid, s);
}

// ---------------------------------------------------------------------------

template <int IO, bool SK>
static hipError_t mp_inner_t(const MpInnerParams& p, int lds, hipStream_t s) {
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute((const void*)mp_inner_kernel<IO, SK>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((mp_inner_kernel<IO, SK>), dim3((unsigned)p.grid), dim3(256), lds, s, p);
    return hipGetLastError();
}

hipError_t launch_mp_inner(int io, const MpInnerParams& p, int lds, hipStream_t s) {
    if (io == IO_BF16)
        return p.skip_hi ? mp_inner_t<IO_BF16, true>(p, lds, s) : mp_inner_t<IO_BF16, false>(p, lds, s);
    return p.skip_hi ? mp_inner_t<IO_F16, true>(p, lds, s) : mp_inner_t<IO_F16, false>(p, lds, s);
}

}  // namespace fftconv
