// Host side of libfftconv: planning (factorisation, launch shapes), the
// fp64 construction of every DFT-matrix and twiddle table in the exact lane
// layout the kernels consume, and the C ABI declared in include/fftconv.h.
//
// Method: page "FlashFFTConv: Efficient Convolutions for Long Sequences with
// Tensor Cores", section 3.4 -- the convolution theorem with causal 2N
// padding, the real-to-complex packing (one-stage decimation in time), the
// order-p Monarch factorisation of the DFT, implicit zero padding, and the
// kernel spectrum computed once per channel.  Plans follow the page's
// "pre-select p offline per length" (section 3.4, cost-model heuristic) with
// factors sized for gfx950: 8/16/32-point stages on 16x16 matrix-core
// tiles, the whole row in one workgroup's LDS up to 16K points, and a
// three-pass schedule through an fp32 workspace beyond that (the partial
// fusion of the page's order-4 algorithm).
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <complex>
#include <cmath>
#include <functional>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/fftconv.h"
#include "fftconv_internal.h"

using namespace fftconv;

namespace {

constexpr size_t kMinN = 256;
constexpr size_t kMaxN = 4194304;
constexpr int kFusedMaxM = 16384;
// full plans on the wide and 16-bit multi-pass kernels (else on the
// LDS-staged ones)
constexpr bool kFullWide = true, kFullMp = true;

bool is_pow2(size_t v) { return v && !(v & (v - 1)); }
int ilog2(size_t v) {
    int r = 0;
    while ((size_t(1) << r) < v) ++r;
    return r;
}

// ---------------------------------------------------------------- planning

struct Shape {
    size_t N = 0, M = 0;
    int p = 0;
    int f[kMaxStages] = {0};
    int path = 0;        // 0 fused, 1 multi-pass
    int n_outer = 0;     // multi-pass: outer factors f[0..n_outer)
    int Min = 0, Qo = 1; // multi-pass slab length and slab count
    int ct = 0;          // outer-pass batch columns per tile
    int thr_fused = 64, thr_outer = 256, thr_inner = 512;
    int lds_fused = 0, lds_outer = 0, lds_inner = 0;
    int wide_P = 0;      // > 0: fused P x 32 x 32 kernel (P/2 waves per row)
    int mp_P1 = 0;       // > 0: multi-pass with outer levels P1 [x mp_P2] and
    int mp_P2 = 1;       //      4096-point inner slabs (4 x 32 x 32)
    bool grad = false;   // the kernel-gradient plan: LDS-staged kernels only
    bool generic = false;  // LDS-staged kernels even where a register-resident
                           // (row / wide) or 16-bit multi-pass kernel exists
    bool full = false;     // circular operators at FFT size N: M = N/2, no
                           // zero half (every packed point in and out)
    fftconv_dtype dtype = FFTCONV_F32;
};

// Fused factorisations by log2(M): all but the last may be 8/16/32, the
// last (the stage fused with the spectrum product) is 16 or 32.
bool default_fused(int lg, std::vector<int>& out) {
    switch (lg) {
    case 8: out = {16, 16}; return true;
    case 9: out = {32, 16}; return true;
    case 10: out = {32, 32}; return true;
    case 11: out = {8, 16, 16}; return true;
    case 12: out = {16, 16, 16}; return true;
    case 13: out = {32, 16, 16}; return true;
    case 14: out = {32, 32, 16}; return true;
    default: return false;
    }
}

// Search for exactly p fused factors (radix exponents 3..5, last 4..5),
// preferring larger leading factors.
bool search_factors(int lg, int p, std::vector<int>& out) {
    if (p < 2 || p > kMaxStages) return false;
    std::vector<int> e(p, 0);
    // enumerate exponents in descending-lexicographic order
    std::function<bool(int, int)> rec = [&](int i, int left) -> bool {
        if (i == p - 1) {
            if (left == 4 || left == 5) { e[i] = left; return true; }
            return false;
        }
        for (int x = 5; x >= 3; --x) {
            if (left - x < 4 + 3 * (p - 2 - i)) continue;
            e[i] = x;
            if (rec(i + 1, left - x)) return true;
        }
        return false;
    };
    if (!rec(0, lg)) return false;
    out.clear();
    for (int i = 0; i < p; ++i) out.push_back(1 << e[i]);
    return true;
}

bool generic_forced();

// The shape of one candidate plan: order p (0: the family's own order for
// N) on the LDS-staged kernels (generic) or on the kernel family that
// covers N (row, wide or 16-bit multi-pass), grad: the shape of the
// kernel-gradient passes, which hold two lines (u and dy) per workgroup:
// LDS-staged kernels only, fused up to M = 8192 and multi-pass slabs of at
// most 4096 points above.  full: the circular operators at FFT size N (an
// N-point real transform, M = N/2 packed points, none of them zero), N in
// [512, 4M]; the kernel families are the same, chosen by M.
fftconv_status make_shape_fixed(size_t N, int p, fftconv_dtype dtype, Shape& s,
                                bool grad, bool generic, bool full = false) {
    if (dtype != FFTCONV_F32 && dtype != FFTCONV_F16 && dtype != FFTCONV_BF16)
        return FFTCONV_ERR_UNSUPPORTED;
    if (!is_pow2(N) || N < (full ? 2 * kMinN : kMinN) || N > kMaxN) return FFTCONV_ERR_UNSUPPORTED;
    if (p < 0 || p == 1 || p > kMaxStages) return FFTCONV_ERR_UNSUPPORTED;
    if (full && grad) return FFTCONV_ERR_UNSUPPORTED;
    s = Shape();
    s.N = N;
    s.M = full ? N / 2 : N;
    s.full = full;
    s.dtype = dtype;
    const int lg = ilog2(s.M);
    std::vector<int> fac;
    s.grad = grad;
    s.generic = generic || grad;
    if (full && dtype != FFTCONV_F32 &&
        ((lg >= 12 && lg <= 14 && !kFullWide) || (lg >= 15 && !kFullMp)))
        s.generic = true;
    if (dtype != FFTCONV_F32 && lg == 15 && (p == 0 || p == 3) && !s.generic && !full) {
        // 16-bit I/O at N = 32K: 32 x 32 x 32 on the one-workgroup-per-row
        // kernel (eight waves, two mirror pairs each), fused
        s.path = 0;
        s.wide_P = 32;
        fac = {32, 32, 32};
    } else if (s.M <= (size_t)(grad ? 8192 : kFusedMaxM)) {
        s.path = 0;
        if (!default_fused(lg, fac)) return FFTCONV_ERR_UNSUPPORTED;
        // 16-bit I/O at N = 4K..16K: order 3 as P x 32 x 32 on the
        // one-workgroup-per-row kernel
        if (dtype != FFTCONV_F32 && lg >= 12 && lg <= 14 && (p == 0 || p == 3) &&
            !s.generic) {
            s.wide_P = 1 << (lg - 10);
            fac = {s.wide_P, 32, 32};
        }
        if (p != 0 && p != (int)fac.size() && !search_factors(lg, p, fac))
            return FFTCONV_ERR_UNSUPPORTED;
        // every stage must leave >= 16 columns and the pairing >= 4 blocks
        for (int x : fac)
            if ((int)(s.M / x) < 16) return FFTCONV_ERR_UNSUPPORTED;
        if ((int)(s.M / fac.back()) < 4) return FFTCONV_ERR_UNSUPPORTED;
        const int waves = s.M <= 1024 ? 1 : (s.M <= 4096 ? 4 : 8);
        s.thr_fused = 64 * waves;
        s.lds_fused = (int)(s.M * 8 + waves * 32 * 8);
    } else if (dtype != FFTCONV_F32 && !s.generic) {
        s.path = 1;
        const int Po = (int)(s.M / 4096);
        switch (Po) {
        case 8: case 16: case 32: s.mp_P1 = Po; s.mp_P2 = 1; break;
        case 64: s.mp_P1 = 8; s.mp_P2 = 8; break;
        case 128: s.mp_P1 = 16; s.mp_P2 = 8; break;
        case 256: s.mp_P1 = 16; s.mp_P2 = 16; break;
        case 512: s.mp_P1 = 32; s.mp_P2 = 16; break;
        case 1024: s.mp_P1 = 32; s.mp_P2 = 32; break;
        default: return FFTCONV_ERR_UNSUPPORTED;
        }
        fac = {s.mp_P1};
        if (s.mp_P2 > 1) fac.push_back(s.mp_P2);
        fac.insert(fac.end(), {4, 32, 32});
        if (p != 0 && p != (int)fac.size()) return FFTCONV_ERR_UNSUPPORTED;
        s.n_outer = s.mp_P2 > 1 ? 2 : 1;
    } else {
        s.path = 1;
        std::vector<int> outer, inner;
        if (grad && lg <= 14) {
            s.Min = 2048;
            inner = {8, 16, 16};
        } else if (lg <= 18 || grad) {
            s.Min = 4096;
            inner = {16, 16, 16};
        } else {
            s.Min = 8192;
            inner = {32, 16, 16};
        }
        s.Qo = (int)(s.M / s.Min);
        switch (ilog2(s.Qo)) {
        case 3: outer = {8}; break;
        case 4: outer = {16}; break;
        case 5: outer = {32}; break;
        case 6: outer = {8, 8}; break;
        case 7: outer = {16, 8}; break;
        case 8: outer = {16, 16}; break;
        case 9: outer = {32, 16}; break;
        case 10: outer = {32, 32}; break;
        default: return FFTCONV_ERR_UNSUPPORTED;
        }
        if (p != 0 && p != (int)(outer.size() + inner.size()))
            return FFTCONV_ERR_UNSUPPORTED;
        s.n_outer = (int)outer.size();
        fac = outer;
        fac.insert(fac.end(), inner.begin(), inner.end());
        s.ct = s.Qo >= 256 ? 16 : 4096 / s.Qo;
        if (s.ct > s.Min) s.ct = s.Min;
        s.thr_outer = 256;
        s.thr_inner = 512;
        s.lds_outer = s.Qo * s.ct * 8;
        s.lds_inner = 2 * s.Min * 8 + (s.thr_inner / 64) * 32 * 8;
    }
    s.p = (int)fac.size();
    for (int i = 0; i < s.p; ++i) s.f[i] = fac[i];
    return FFTCONV_OK;
}

size_t kf_entry_bytes(fftconv_dtype dt) { return dt == FFTCONV_F32 ? 16 : 8; }

double mfma_flops_per_row(const Shape& s) {
    // real flops of the complex DFT-matrix products (8 per complex MAC):
    // forward stage 1 contracts half its digits, the last inverse stage
    // produces half its outputs (both whole on full plans).
    double f = 0;
    for (int i = 0; i < s.p; ++i) {
        const double per = 8.0 * (double)s.M * s.f[i];
        f += (i == 0 && !s.full) ? per : 2.0 * per;
    }
    return f;
}

bool generic_forced() {
    const char* kenv = getenv("FFTCONV_KERNEL");
    return kenv && strcmp(kenv, "generic") == 0;
}

// The register-resident kernel covers N = 32 x NB (NB = 16, 32) with 16-bit
// I/O; FFTCONV_KERNEL=generic keeps such plans on the LDS-staged kernel.
bool row_kernel_applies(const Shape& s) {
    return s.path == 0 && s.p == 2 && s.f[0] == 32 && (s.f[1] == 16 || s.f[1] == 32) &&
           s.dtype != FFTCONV_F32 && !s.generic;
}

// ------------------------------------------------------------ cost model
//
// An MI355X analogue of the page's cost model (FlashFFTConv page, section
// 3.4, "The GPU Cost Model for Order-p Decompositions", Equation 2): per
// row, the work of every decomposition level is charged to the unit that
// runs it -- DFT-matrix products on the matrix cores (tau_M), small DFTs
// done with butterflies, twiddles and the spectrum pairing on the vector ALU
// (tau_V), stage data and operand tables through LDS (sigma_S), and the
// compulsory streams plus any workspace round trips through HBM
// (sigma_H).  Unlike Equation 2's plain sum, compute and HBM overlap: the
// matrix, vector and LDS instructions of a wave share its issue stream and
// are summed, the memory streams run beside them, so the predicted time is
// max(t_HBM, t_MFMA + t_VALU + t_LDS).  The HBM rate is the practical one a
// streaming copy reaches on the part (the page likewise measures its
// constants); the others are the published peaks of MI355X.
namespace cost {
constexpr double kHbm = 5.2e12;        // B/s, streaming copy on MI355X
constexpr double kMfmaF16 = 2.5e15;    // dense f16/bf16 matrix flop/s
constexpr double kMfmaF32 = 157.3e12;  // dense fp32 matrix flop/s
constexpr double kValuF16 = 157.3e12;  // packed-f16 vector flop/s
constexpr double kValuF32 = 78.6e12;   // fp32 vector flop/s (no packed fp32)
constexpr double kLds = 256 * 128 * 2.4e9;   // B/s: 128 B/clk per CU
}  // namespace cost

struct CostTerms {
    double hbm_bytes = 0, mfma_flops = 0, valu_flops_f16 = 0, valu_flops_f32 = 0, lds_bytes = 0;
    double t_hbm = 0, t_mfma = 0, t_valu = 0, t_lds = 0, t_pred = 0;
};

// Work of one call over B x H rows of the plan shape s.  B = 0: the per-row
// cost of a large batch, the spectrum's read amortised away (H rows).
CostTerms estimate(const Shape& s, size_t B, size_t H) {
    CostTerms c;
    const double R = (double)(B ? B : 1) * (double)H, M = (double)s.M, N = (double)s.N;
    const double sio = s.dtype == FFTCONV_F32 ? 4.0 : 2.0;
    const double skf = s.dtype == FFTCONV_F32 ? 16.0 : 8.0;
    const bool f32 = s.dtype == FFTCONV_F32;
    const bool bf16 = s.dtype == FFTCONV_BF16;
    const bool row = row_kernel_applies(s);
    // --- HBM: u, y once; k_f once per channel; workspace round trips
    double hbm = R * 2.0 * N * sio + (B ? (double)H * M * skf : 0.0);
    if (s.path == 1) hbm += R * M * (s.mp_P1 ? 16.0 : 32.0);
    // --- per level: matrix products, or butterflies on the vector ALU
    double mf = 0, vf16 = 0, vf32 = 0, lds = 0;
    for (int i = 0; i < s.p; ++i) {
        const double n = (double)s.f[i];
        const double half = (i == 0) ? 0.5 : 1.0;   // the zero half / half outputs
        bool valu_level = false;
        if (s.wide_P && i == 0) valu_level = true;
        if (s.mp_P1 && i < s.n_outer && !(s.mp_P1 == 32 && s.mp_P2 == 32)) valu_level = true;
        if (valu_level) {
            // radix-2 butterflies, both directions: 5 M log2(n) flops each
            const double fl = half * 2.0 * 5.0 * M * std::log2(n);
            if (bf16 || f32) vf32 += fl; else vf16 += fl;
        } else {
            double fl = half * 16.0 * M * n;
            // hi/lo split operands: bf16 rows into the row kernel's first
            // stage, both 32-point levels of the 4M column passes
            if (row && bf16 && i == 0) fl *= 2.0;
            if (s.mp_P1 == 32 && s.mp_P2 == 32 && i < 2) fl *= 2.0;
            mf += fl;
        }
    }
    // twiddles between levels (both directions) and the spectrum pairing
    // (two complex multiply-adds per bin)
    const double tw = (double)(s.p - 1) * 2.0 * 6.0 * M, pair = 16.0 * M;
    if (f32) vf32 += tw + pair;
    else vf16 += tw + pair;
    // --- LDS traffic
    if (row) {
        // the four stage tables read at each use, one 16-byte operand per
        // lane and tile (KB per row: first stage 4, or 8 with the bf16 hi/lo
        // split; second (NB/8)(NB/16); its inverse 2 (NB/16)^2; last 4),
        // and the spectrum coefficients (8 B per bin)
        const double q = (double)s.f[1] / 16.0;
        const double tabs_kb = (bf16 ? 8.0 : 4.0) + 2.0 * q * q + 2.0 * q * q + 4.0;
        lds = tabs_kb * 1024.0 + M * 8.0;
    } else if (s.wide_P || s.mp_P1) {
        // sub-rows written and read around the engine, both directions;
        // engine operand tables per 1024-point sub-row; outer twiddles
        lds = 16.0 * M + 16.0 * M + 4.0 * M;
        if (s.mp_P1) lds += 16.0 * M;   // column tiles of the outer passes
    } else {
        // LDS-staged: every stage reads and writes the row (fp32 complex)
        // in both directions, as column gathers and scatters that reach
        // about 1/6 of the LDS peak for 16- and 32-point stages and 1/10
        // for 8-point ones (measured on MI355X, 16-bit plans at N = 1K..16K;
        // charged here as extra bytes at the peak rate)
        for (int i = 0; i < s.p; ++i) lds += 32.0 * M * (s.f[i] >= 16 ? 6.0 : 10.0);
    }
    c.hbm_bytes = hbm;
    c.mfma_flops = R * mf;
    c.valu_flops_f16 = R * vf16;
    c.valu_flops_f32 = R * vf32;
    c.lds_bytes = R * lds;
    c.t_hbm = hbm / cost::kHbm;
    c.t_mfma = c.mfma_flops / (f32 ? cost::kMfmaF32 : cost::kMfmaF16);
    c.t_valu = c.valu_flops_f16 / cost::kValuF16 + c.valu_flops_f32 / cost::kValuF32;
    c.t_lds = c.lds_bytes / cost::kLds;
    const double comp = c.t_mfma + c.t_valu + c.t_lds;
    c.t_pred = c.t_hbm > comp ? c.t_hbm : comp;
    return c;
}

// p = 0: the candidate of lowest predicted time among every order the
// kernels support for N, on the LDS-staged kernels and on the kernel family
// that covers N (ties: the lower order).  FFTCONV_KERNEL=generic restricts
// the choice to the LDS-staged kernels.
fftconv_status make_shape(size_t N, int p, fftconv_dtype dtype, Shape& s,
                          bool grad = false, bool full = false) {
    const bool force_generic = generic_forced();
    // full plans take the family's own factorisation (the cost model
    // prices the causal kernels)
    if (p != 0 || grad || full) return make_shape_fixed(N, p, dtype, s, grad, force_generic, full);
    fftconv_status first = FFTCONV_ERR_UNSUPPORTED;
    bool found = false;
    double best = 0;
    for (int q = 2; q <= kMaxStages; ++q)
        for (int gen = force_generic ? 1 : 0; gen <= 1; ++gen) {
            Shape c;
            const fftconv_status st = make_shape_fixed(N, q, dtype, c, false, gen != 0);
            if (st != FFTCONV_OK) {
                if (first == FFTCONV_ERR_UNSUPPORTED) first = st;
                continue;
            }
            const double t = estimate(c, 0, 1).t_pred;
            if (!found || t < best * (1.0 - 1e-9)) {
                best = t;
                s = c;
                found = true;
            }
        }
    return found ? FFTCONV_OK : first;
}

// The outer factor P of the digit-block sparsity pattern: the outer stage
// before the 1024- or 4096-point inner transform (wide and multi-pass
// kernels); 1 where the kernels have no such outer stage.
int sparse_outer(const Shape& s) {
    if (s.wide_P) return s.wide_P;
    if (s.mp_P1) return (int)(s.M / 4096);
    return 1;
}

void fill_info(const Shape& s, fftconv_plan_info* info) {
    memset(info, 0, sizeof(*info));
    info->N = s.N;
    info->M = s.M;
    info->order = s.p;
    for (int i = 0; i < s.p; ++i) info->factors[i] = s.f[i];
    info->path = s.path;
    info->outer_factors = s.n_outer;
    info->dtype = s.dtype;
    info->spectrum_bytes_per_channel = s.M * kf_entry_bytes(s.dtype);
    info->workspace_bytes_per_row = s.path ? s.M * (s.mp_P1 ? 4 : 8) : 0;
    info->mfma_flops_per_row = mfma_flops_per_row(s);
    info->kernel_variant = s.mp_P1 ? 4 : s.path ? 2 : (s.wide_P ? 3 : (row_kernel_applies(s) ? 1 : 0));
    info->sparse_outer = sparse_outer(s);
    info->circular = s.full ? 1 : 0;
}

// ------------------------------------------------------- table construction

enum MatKind { MAT_REG, MAT_MID_FWD, MAT_MID_INV };

int mid_perm(int slot, int n) { return slot < n / 2 ? slot : 3 * n / 2 - 1 - slot; }

uint16_t f32_to_f16_bits(float f) {
    _Float16 h = (_Float16)f;
    uint16_t b;
    memcpy(&b, &h, 2);
    return b;
}

// A-operand tiles of one stage's real-embedded DFT matrix, [MT][KS][lane]
// with 8 halves (f16 plans) or 1 float (fp32 plans) per lane.
// inverse: exponent sign +; half_in: only the first n/2 input digits;
// half_out: only the first n/2 output digits.
std::vector<uint8_t> build_matrix(int n, bool inverse, bool half_in,
                                  bool half_out, MatKind kind, bool f32) {
    const int nin = half_in ? n / 2 : n;
    const int nout = half_out ? n / 2 : n;
    const int KS = f32 ? nin / 2 : (nin <= 16 ? 1 : nin / 16);
    const int MT = nout / 8 > 0 ? nout / 8 : 1;
    const int per = f32 ? 1 : 8;
    const size_t esz = f32 ? 4 : 2;
    std::vector<uint8_t> out((size_t)MT * KS * 64 * per * esz, 0);
    const double sgn = inverse ? 1.0 : -1.0;
    const double scale = 1.0 / sqrt((double)n);
    for (int mt = 0; mt < MT; ++mt)
        for (int ks = 0; ks < KS; ++ks)
            for (int lane = 0; lane < 64; ++lane) {
                const int g = lane >> 4, x = lane & 15;
                const int row = 16 * mt + x;
                const int oslot = row >> 1, c = row & 1;
                for (int j = 0; j < per; ++j) {
                    int islot, d;
                    bool chain = (kind == MAT_MID_INV);
                    if (!f32) {
                        if (chain) {
                            islot = 16 * ks + 8 * (j >> 2) + 2 * g + ((j >> 1) & 1);
                        } else {
                            islot = 16 * ks + 4 * g + (j >> 1);
                        }
                        d = j & 1;
                    } else {
                        if (chain) {
                            islot = 8 * (ks >> 2) + 2 * g + ((ks & 3) >> 1);
                            d = ks & 1;
                        } else {
                            islot = 2 * ks + (g >> 1);
                            d = g & 1;
                        }
                    }
                    double val = 0.0;
                    const bool ok = oslot < nout && (chain || islot < nin);
                    if (ok) {
                        const int ko = (kind == MAT_MID_FWD) ? mid_perm(oslot, n) : oslot;
                        const int ni = chain ? mid_perm(islot, n) : islot;
                        const long long e = ((long long)ko * ni) % n;
                        const double ang = sgn * 2.0 * M_PI * (double)e / (double)n;
                        const double wr = cos(ang) * scale, wi = sin(ang) * scale;
                        if (c == 0) val = (d == 0) ? wr : -wi;
                        else val = (d == 0) ? wi : wr;
                    }
                    const size_t idx = (((size_t)(mt * KS + ks) * 64 + lane) * per + j);
                    if (f32) {
                        float fv = (float)val;
                        memcpy(&out[idx * 4], &fv, 4);
                    } else {
                        uint16_t hv = f32_to_f16_bits((float)val);
                        memcpy(&out[idx * 2], &hv, 2);
                    }
                }
            }
    return out;
}

// W_S^{k c} for k < n, c < S/n, laid out [k][c] (fp64 -> fp32).
std::vector<float> build_twiddles(int n, long long S) {
    const long long s = S / n;
    std::vector<float> t((size_t)S * 2);
    for (long long k = 0; k < n; ++k)
        for (long long c = 0; c < s; ++c) {
            const long long e = (k * c) % S;
            const double ang = -2.0 * M_PI * (double)e / (double)S;
            t[(size_t)(k * s + c) * 2] = (float)cos(ang);
            t[(size_t)(k * s + c) * 2 + 1] = (float)sin(ang);
        }
    return t;
}

// Position of lower bin part q for the digit list fac[0..cnt) with
// in-place strides str[0..cnt) (divided by the unit 'unit').
std::vector<int> build_digrev(const int* fac, const long long* str, int cnt,
                              long long unit) {
    long long Q = 1;
    for (int i = 0; i < cnt; ++i) Q *= fac[i];
    std::vector<int> r((size_t)Q);
    for (long long q = 0; q < Q; ++q) {
        long long rem = q, pos = 0;
        for (int i = 0; i < cnt; ++i) {
            const long long dgt = rem % fac[i];
            rem /= fac[i];
            pos += dgt * (str[i] / unit);
        }
        r[(size_t)q] = (int)pos;
    }
    return r;
}


// ----------------------------------------------- row-kernel tables (32 x NB)

double emb(double wr, double wi, int c, int d) {
    return c == 0 ? (d == 0 ? wr : -wi) : (d == 0 ? wi : wr);
}
int kmap32h(int kt, int x) { return kt == 0 ? x : (x == 0 ? 16 : 32 - x); }
// n_b digit held by row y of tile t in the row kernel (mirror map for
// NB = 32 so forward and inverse twiddle positions coincide).
int nbmaph(int NB, int t, int y) { return NB == 32 ? kmap32h(t, y) : 16 * t + y; }

// Inner forward stage (A operand, rows in mirror-pairing order) whose K
// index follows the first stage's accumulator rows: K-step ks, group g,
// slot j <-> n_b = nbmap(ks, 4g + j/2), part j&1.
std::vector<uint8_t> row_f2a(int NB) {
    const int KS = NB / 16, MT = NB / 8;
    std::vector<uint8_t> out((size_t)MT * KS * 64 * 8 * 2);
    const double sc = 1.0 / sqrt((double)NB);
    for (int mt = 0; mt < MT; ++mt)
        for (int ks = 0; ks < KS; ++ks)
            for (int lane = 0; lane < 64; ++lane) {
                const int g = lane >> 4, x = lane & 15;
                const int row = 16 * mt + x, oslot = row >> 1, c = row & 1;
                const int kb = mid_perm(oslot, NB);
                for (int j = 0; j < 8; ++j) {
                    const int nb = nbmaph(NB, ks, 4 * g + (j >> 1)), d = j & 1;
                    const double ang = -2.0 * M_PI * (double)((kb * nb) % NB) / (double)NB;
                    const double v = emb(cos(ang) * sc, sin(ang) * sc, c, d);
                    const uint16_t hv = f32_to_f16_bits((float)v);
                    memcpy(&out[((((size_t)(mt * KS + ks)) * 64 + lane) * 8 + j) * 2], &hv, 2);
                }
            }
    return out;
}

uint16_t f32_to_bf16_bits(float f) {
    uint32_t b;
    memcpy(&b, &f, 4);
    const uint32_t lsb = (b >> 16) & 1u;
    return (uint16_t)((b + 0x7fffu + lsb) >> 16);
}
float bf16_bits_to_f32(uint16_t h) {
    uint32_t b = (uint32_t)h << 16;
    float f;
    memcpy(&f, &b, 4);
    return f;
}

// First stage as the B operand: K = (n_a < 16, part d), columns
// (k_a tile, part c), k_a = kmap32(tile, x).  bf16 plans get a hi/lo split
// so the bf16 input feeds the matrix core directly at ~2^-16 accuracy.
// full: a second set of tiles for n_a = 16..31 (the K-step of the upper
// half), [half][tile][lane].
std::vector<uint16_t> row_f1b(bool bf16, bool full = false) {
    const int T = bf16 ? 8 : 4, NH = full ? 2 : 1;
    std::vector<uint16_t> out((size_t)NH * T * 64 * 8);
    const double sc = 1.0 / sqrt(32.0);
    for (int hf = 0; hf < NH; ++hf)
    for (int tt = 0; tt < T; ++tt) {
        const int jt = tt & 3;
        const bool lo = tt >= 4;
        for (int lane = 0; lane < 64; ++lane) {
            const int g = lane >> 4, x = lane & 15;
            const int kt = jt >> 1, c = jt & 1, ka = kmap32h(kt, x);
            for (int j = 0; j < 8; ++j) {
                const int na = 16 * hf + 4 * g + (j >> 1), d = j & 1;
                const double ang = -2.0 * M_PI * (double)((na * ka) % 32) / 32.0;
                const double v = emb(cos(ang) * sc, sin(ang) * sc, c, d);
                uint16_t bits;
                if (bf16) {
                    const uint16_t hi = f32_to_bf16_bits((float)v);
                    bits = lo ? f32_to_bf16_bits((float)(v - (double)bf16_bits_to_f32(hi))) : hi;
                } else {
                    bits = f32_to_f16_bits((float)v);
                }
                out[((size_t)(hf * T + tt) * 64 + lane) * 8 + j] = bits;
            }
        }
    }
    return out;
}

// Last inverse stage as the A operand: rows (n_a < 16, part c; all 32 n_a
// when full), K the accumulator order of the preceding stage:
// k_a = kmap32(ks, 4g + j/2).
std::vector<uint16_t> row_i1a(bool full = false) {
    const int MT = full ? 4 : 2;
    std::vector<uint16_t> out((size_t)MT * 2 * 64 * 8);
    const double sc = 1.0 / sqrt(32.0);
    for (int mt = 0; mt < MT; ++mt)
        for (int ks = 0; ks < 2; ++ks)
            for (int lane = 0; lane < 64; ++lane) {
                const int g = lane >> 4, x = lane & 15;
                const int row = 16 * mt + x, na = row >> 1, c = row & 1;
                for (int j = 0; j < 8; ++j) {
                    const int ka = kmap32h(ks, 4 * g + (j >> 1)), d = j & 1;
                    const double ang = 2.0 * M_PI * (double)((na * ka) % 32) / 32.0;
                    const double v = emb(cos(ang) * sc, sin(ang) * sc, c, d);
                    out[(((size_t)(mt * 2 + ks)) * 64 + lane) * 8 + j] = f32_to_f16_bits((float)v);
                }
            }
    return out;
}

// Inner inverse stage as the B operand: K in accumulator (chain) order of
// the permuted inner forward stage, columns (n_b tile, part c).
// K-step ks, half h of a lane's 8 values: M-tile 2 ks + h of the forward
// accumulators, or ks + h KS with `split` (the row kernel: its K-step 1 then
// holds exactly the tiles of the middle k_b, which a band limit zeroes).
std::vector<uint16_t> row_i2b(int NB, bool split = false) {
    const int KS = NB / 16, JT = 2 * (NB / 16);
    std::vector<uint16_t> out((size_t)KS * JT * 64 * 8);
    const double sc = 1.0 / sqrt((double)NB);
    for (int ks = 0; ks < KS; ++ks)
        for (int jt = 0; jt < JT; ++jt)
            for (int lane = 0; lane < 64; ++lane) {
                const int g = lane >> 4, x = lane & 15;
                const int nt = jt >> 1, c = jt & 1, nb = nbmaph(NB, nt, x);
                for (int j = 0; j < 8; ++j) {
                    const int mt = split ? ks + KS * (j >> 2) : 2 * ks + (j >> 2);
                    const int slot = 8 * mt + 2 * g + ((j >> 1) & 1);
                    const int kb = mid_perm(slot, NB), d = j & 1;
                    const double ang = 2.0 * M_PI * (double)((kb * nb) % NB) / (double)NB;
                    const double v = emb(cos(ang) * sc, sin(ang) * sc, c, d);
                    out[(((size_t)(ks * JT + jt)) * 64 + lane) * 8 + j] = f32_to_f16_bits((float)v);
                }
            }
    return out;
}

// Per-lane twiddles W_M^{+-k_a n_b} at the positions each lane holds,
// as packed f16 (re, im) pairs.
std::vector<uint16_t> row_twiddles(int NB, bool inverse) {
    const int M = 32 * NB, IT = NB / 16;
    std::vector<uint16_t> out((size_t)64 * IT * 8 * 2);
    for (int lane = 0; lane < 64; ++lane) {
        const int g = lane >> 4, x = lane & 15;
        for (int a = 0; a < IT; ++a)          // fwd: it;   inv: nt
            for (int kt = 0; kt < 2; ++kt)
                for (int r = 0; r < 4; ++r) {
                    int ka, nb, idx;
                    if (!inverse) {
                        ka = kmap32h(kt, x);
                        nb = nbmaph(NB, a, 4 * g + r);
                        idx = lane * (IT * 8) + (a * 2 + kt) * 4 + r;
                    } else {
                        ka = kmap32h(kt, 4 * g + r);
                        nb = nbmaph(NB, a, x);
                        idx = lane * (IT * 8) + (kt * IT + a) * 4 + r;
                    }
                    const double ang = (inverse ? 2.0 : -2.0) * M_PI *
                                       (double)(((long long)ka * nb) % M) / (double)M;
                    out[(size_t)idx * 2] = f32_to_f16_bits((float)cos(ang));
                    out[(size_t)idx * 2 + 1] = f32_to_f16_bits((float)sin(ang));
                }
    }
    return out;
}


// ------------------------------------------- wide-kernel tables (P x 32 x 32)

// First engine stage as the B operand over all 32 n_a (two K-steps), scaled
// so that the outer P-point stage, this stage and the next one together are
// unitary: 1/sqrt(32 P).
std::vector<uint16_t> wide_f1b(int P) {
    std::vector<uint16_t> out((size_t)8 * 64 * 8);
    const double sc = 1.0 / sqrt(32.0 * P);
    for (int ks = 0; ks < 2; ++ks)
        for (int jt = 0; jt < 4; ++jt)
            for (int lane = 0; lane < 64; ++lane) {
                const int g = lane >> 4, x = lane & 15;
                const int kt = jt >> 1, c = jt & 1, ka = kmap32h(kt, x);
                for (int j = 0; j < 8; ++j) {
                    const int na = 16 * ks + 4 * g + (j >> 1), d = j & 1;
                    const double ang = -2.0 * M_PI * (double)((na * ka) % 32) / 32.0;
                    const double v = emb(cos(ang) * sc, sin(ang) * sc, c, d);
                    out[(((size_t)(ks * 4 + jt)) * 64 + lane) * 8 + j] = f32_to_f16_bits((float)v);
                }
            }
    return out;
}

// Last inverse engine stage as the A operand producing all 32 n_a.
std::vector<uint16_t> wide_i1a(int P) {
    std::vector<uint16_t> out((size_t)8 * 64 * 8);
    const double sc = 1.0 / sqrt(32.0 * P);
    for (int mt = 0; mt < 4; ++mt)
        for (int ks = 0; ks < 2; ++ks)
            for (int lane = 0; lane < 64; ++lane) {
                const int g = lane >> 4, x = lane & 15;
                const int row = 16 * mt + x, na = row >> 1, c = row & 1;
                for (int j = 0; j < 8; ++j) {
                    const int ka = kmap32h(ks, 4 * g + (j >> 1)), d = j & 1;
                    const double ang = 2.0 * M_PI * (double)((na * ka) % 32) / 32.0;
                    const double v = emb(cos(ang) * sc, sin(ang) * sc, c, d);
                    out[(((size_t)(mt * 2 + ks)) * 64 + lane) * 8 + j] = f32_to_f16_bits((float)v);
                }
            }
    return out;
}

// Outer-stage twiddles W_M^{n' k1}, k1 = 1..P/2, for the columns each
// thread owns: n_b = t & 31, n_a = CPT (t >> 5) + j.
// Threads of the wide kernel's workgroup: one wave per mirror pair of
// sub-rows, at most eight.
int wide_threads(int P) { return 64 * (P / 2 < 8 ? P / 2 : 8); }

std::vector<uint16_t> wide_outer_twiddles(int P) {
    const int T = wide_threads(P), CPT = 1024 / T, M = 1024 * P;
    std::vector<uint16_t> out((size_t)(P / 2) * T * CPT * 2);
    for (int k1 = 1; k1 <= P / 2; ++k1)
        for (int t = 0; t < T; ++t)
            for (int j = 0; j < CPT; ++j) {
                const int nb = t & 31, na = CPT * (t >> 5) + j;
                const long long np = 32LL * na + nb;
                const double ang = -2.0 * M_PI * (double)((np * k1) % M) / (double)M;
                const size_t idx = (((size_t)(k1 - 1) * T + t) * CPT + j) * 2;
                out[idx] = f32_to_f16_bits((float)cos(ang));
                out[idx + 1] = f32_to_f16_bits((float)sin(ang));
            }
    return out;
}

// Inner-pass twiddles W_4096^{n' m}, m = 1..4, for the columns each thread
// owns (as in the wide kernel with 256 threads: n_b = t & 31,
// n_a = 4 (t >> 5) + j).
std::vector<uint16_t> mp_inner_twiddles() {
    // W_4096^{n' m} for m = 0..4, n' = 32 n_a + n_b < 1024 (packed f16),
    // [m][engine position of (n_a, n_b)]: the position of the 32 x 32
    // engine's LDS layout, 4 consecutive n_a per 16-byte word
    const int Q = 1024, Mi = 4096;
    std::vector<uint16_t> out((size_t)5 * Q * 2);
    for (int m = 0; m <= 4; ++m)
        for (int na = 0; na < 32; ++na)
            for (int nb = 0; nb < 32; ++nb) {
                const int it = nb < 16 ? 0 : 1;
                const int xx = nb < 16 ? nb : (nb == 16 ? 0 : 32 - nb);
                const int pos = (((it * 2 + (na >> 4)) * 64 + 16 * ((na >> 2) & 3) + xx) << 2) + (na & 3);
                const int np = 32 * na + nb;
                const double ang = -2.0 * M_PI * (double)((np * m) % Mi) / (double)Mi;
                const size_t idx = ((size_t)m * Q + pos) * 2;
                out[idx] = f32_to_f16_bits((float)cos(ang));
                out[idx + 1] = f32_to_f16_bits((float)sin(ang));
            }
    return out;
}

// Matrix-core two-level passes (P1 = P2 = 32): A operands of a 32-point
// DFT (scaled 1/sqrt(32); inverse: exponent sign +) over the first nin
// inputs and nout outputs, as hi/lo pairs of 16-bit values (bf16 or f16),
// [mt][ks][hi/lo][lane][8]:
// lane (g, x) holds real row 16 mt + x (output digit and re/im) and real
// columns 32 ks + 8 g .. + 7 (input digit and re/im).
std::vector<uint16_t> col2m_dft_a(bool bf16, int nin, int nout = 32, bool inverse = false) {
    const int KS = nin * 2 / 32, MT = nout * 2 / 16;
    std::vector<uint16_t> out((size_t)MT * KS * 2 * 64 * 8);
    const double sc = 1.0 / sqrt(32.0);
    for (int mt = 0; mt < MT; ++mt)
        for (int ks = 0; ks < KS; ++ks)
            for (int lane = 0; lane < 64; ++lane)
                for (int i = 0; i < 8; ++i) {
                    const int g = lane >> 4, x = lane & 15;
                    const int R = 16 * mt + x, kk = 32 * ks + 8 * g + i;
                    const int o = R >> 1, ro = R & 1, n = kk >> 1, ki = kk & 1;
                    const double ang = (inverse ? 2.0 : -2.0) * M_PI * (double)((o * n) % 32) / 32.0;
                    const double fr = cos(ang) * sc, fi = sin(ang) * sc;
                    const double v = ro == 0 ? (ki == 0 ? fr : -fi) : (ki == 0 ? fi : fr);
                    uint16_t hi, lo;
                    if (bf16) {
                        hi = f32_to_bf16_bits((float)v);
                        lo = f32_to_bf16_bits((float)(v - (double)bf16_bits_to_f32(hi)));
                    } else {
                        hi = f32_to_f16_bits((float)v);
                        _Float16 hh;
                        memcpy(&hh, &hi, 2);
                        lo = f32_to_f16_bits((float)(v - (double)(float)hh));
                    }
                    for (int hl = 0; hl < 2; ++hl)
                        out[((((size_t)(mt * KS + ks) * 2 + hl) * 64 + lane) * 8) + i] = hl ? lo : hi;
                }
    return out;
}

// Twiddles of the matrix-core forward pass (fp32 pairs, computed in fp64):
// [W_1024^{n2 k1}: 32 x 32][W_M^{32 i k1}: 128 x 32][W_M^{c k1}: 32 x 32]
// [W_M^{1024 i k2}: 128 x 32][W_M^{32 c k2}: 32 x 32]
std::vector<float> col2m_twiddles(long long M) {
    std::vector<float> out;
    auto put = [&](long long num, long long den) {
        const double ang = -2.0 * M_PI * (double)(num % den) / (double)den;
        out.push_back((float)cos(ang));
        out.push_back((float)sin(ang));
    };
    for (int n2 = 0; n2 < 32; ++n2)
        for (int k = 0; k < 32; ++k) put((long long)n2 * k, 1024);
    for (int i = 0; i < 128; ++i)
        for (int k = 0; k < 32; ++k) put(32LL * i * k, M);
    for (int c = 0; c < 32; ++c)
        for (int k = 0; k < 32; ++k) put((long long)c * k, M);
    for (int i = 0; i < 128; ++i)
        for (int k = 0; k < 32; ++k) put(1024LL * i * k, M);
    for (int c = 0; c < 32; ++c)
        for (int k = 0; k < 32; ++k) put(32LL * c * k, M);
    return out;
}

// Column-pass twiddle bases W_n^c, c < count, fp32 (computed in fp64).
std::vector<float> col_twiddles(long long n, long long count) {
    std::vector<float> out((size_t)count * 2);
    for (long long c = 0; c < count; ++c) {
        const double ang = -2.0 * M_PI * (double)c / (double)n;
        out[(size_t)c * 2] = (float)cos(ang);
        out[(size_t)c * 2 + 1] = (float)sin(ang);
    }
    return out;
}

}  // namespace

// --------------------------------------------------------------- the plan

struct fftconv_plan_s {
    Shape s;
    int device = 0;
    std::vector<void*> allocs;
    FwdParams fused{};      // path 0
    FwdParams outer{};      // path 1, outer passes
    FwdParams inner{};      // path 1, inner pass
    int num_cu = 256;
    long long row_max_channels = 1;   // channels whose spectra fit the row LDS
    bool use_row = false;   // register-resident kernel for N = 32 x NB
    int row_nb = 0;
    int lds_row = 0;
    RowParams row{};
    int lds_wide = 0;
    int wide_wgs_per_cu = 1;
    WideParams wide{};
    int lds_mp = 0;
    MpInnerParams mp{};
    const uint4* mp2m_a1 = nullptr;   // matrix-core forward pass (4M): level-1 A operands
    const uint4* mp2m_a1h = nullptr;  // the same in f16 (gated rows)
    const uint4* mp2m_a2 = nullptr;   //   level-2 A operands
    const uint4* mp2m_ia1 = nullptr;  // inverse pass: level-1 inverse A operands
    const uint4* mp2m_ia2 = nullptr;  //   level-2 inverse A operands
    const float2* mp2m_tm = nullptr;  //   twiddle tables
    const float2* mp_tw1 = nullptr;   // W_M^c, c < M / P1
    const float2* mp_tw2 = nullptr;   // W_{M/P1}^c, c < 4096 (two levels)
    fftconv_plan_s* grad = nullptr;   // LDS-staged plan of the kernel gradient
    // the plan whose engine computes the kernel gradient when it is not this
    // plan's own (N = 32K: the forward is the fused 32 x 32 x 32 kernel, the
    // gradient the multi-pass engine)
    fftconv_plan_s* kg = nullptr;
};

namespace {

hipError_t upload(fftconv_plan_s* pl, const void* host, size_t bytes, void** dev) {
    void* d = nullptr;
    hipError_t e = hipMalloc(&d, bytes ? bytes : 16);
    if (e != hipSuccess) return e;
    pl->allocs.push_back(d);
    e = hipMemcpy(d, host, bytes, hipMemcpyHostToDevice);
    *dev = d;
    return e;
}

void free_plan(fftconv_plan_s* pl) {
    if (!pl) return;
    free_plan(pl->grad);
    free_plan(pl->kg);
    for (void* p : pl->allocs) (void)hipFree(p);
    delete pl;
}

fftconv_status build_mp_tables(fftconv_plan_s* pl);
fftconv_status plan_create(size_t N, int p, fftconv_dtype dtype, bool full,
                           fftconv_plan_t* out);
fftconv_status spectrum_impl(fftconv_plan_t plan, const float* k, size_t H,
                             fftconv_kernel_kind kind, long long cutoff, void* k_f,
                             void* stream, int blk_a = 0, int blk_d = 0);
constexpr size_t kMpChunkBytes = (size_t)1024 << 20;

fftconv_status forward_check(fftconv_plan_t plan, const void* u, const void* w,
                             const void* v, const void* k_f, void* y, size_t B,
                             size_t H, size_t N, void* workspace,
                             size_t workspace_bytes, size_t chunk_cap);
fftconv_status forward_impl(fftconv_plan_t plan, const void* u, const void* w,
                            const void* v, const void* k_f, void* y, size_t B,
                            size_t H, size_t N, void* workspace,
                            size_t workspace_bytes, void* stream, int skip_hi,
                            size_t chunk_cap, int outer_keep = 0);
fftconv_status backward_dk(const fftconv_plan_s* plan, const void* u, const void* dy,
                           float* dk, size_t B, size_t H, size_t N, void* workspace,
                           hipStream_t st, const void* k_f_adj = nullptr,
                           void* du = nullptr);

fftconv_status build_device_tables(fftconv_plan_s* pl) {
    const Shape& s = pl->s;
    if (s.mp_P1) return build_mp_tables(pl);
    const bool f32 = s.dtype == FFTCONV_F32;
    long long S[kMaxStages], str[kMaxStages];
    {
        long long blk = (long long)s.M;
        for (int i = 0; i < s.p; ++i) {
            S[i] = blk;
            str[i] = blk / s.f[i];
            blk = str[i];
        }
    }
    // regular stages: twiddles + matrices
    StageDev reg[kMaxStages];
    memset(reg, 0, sizeof(reg));
    for (int i = 0; i < s.p - 1; ++i) {
        const int n = s.f[i];
        const bool outermost = (i == 0);
        std::vector<float> tw = build_twiddles(n, S[i]);
        void *dtw = nullptr, *dmf = nullptr, *dmi = nullptr;
        if (upload(pl, tw.data(), tw.size() * 4, &dtw) != hipSuccess) return FFTCONV_ERR_HIP;
        const bool half = outermost && !s.full;
        std::vector<uint8_t> mf = build_matrix(n, false, half, false, MAT_REG, f32);
        std::vector<uint8_t> mi = build_matrix(n, true, false, half, MAT_REG, f32);
        if (upload(pl, mf.data(), mf.size(), &dmf) != hipSuccess) return FFTCONV_ERR_HIP;
        if (upload(pl, mi.data(), mi.size(), &dmi) != hipSuccess) return FFTCONV_ERR_HIP;
        reg[i].n = n;
        reg[i].tw = (const float2*)dtw;
        reg[i].mat_f = dmf;
        reg[i].mat_i = dmi;
        reg[i].tw_stride = (int)str[i];
    }
    // middle stage
    MidDev mid{};
    {
        const int n = s.f[s.p - 1];
        std::vector<uint8_t> mf = build_matrix(n, false, false, false, MAT_MID_FWD, f32);
        std::vector<uint8_t> mi = build_matrix(n, true, false, false, MAT_MID_INV, f32);
        void *dmf = nullptr, *dmi = nullptr, *ddr = nullptr;
        if (upload(pl, mf.data(), mf.size(), &dmf) != hipSuccess) return FFTCONV_ERR_HIP;
        if (upload(pl, mi.data(), mi.size(), &dmi) != hipSuccess) return FFTCONV_ERR_HIP;
        const int first = s.path ? s.n_outer : 0;
        std::vector<int> dr = build_digrev(s.f + first, str + first,
                                           s.p - 1 - first, n);
        if (upload(pl, dr.data(), dr.size() * 4, &ddr) != hipSuccess) return FFTCONV_ERR_HIP;
        mid.n = n;
        mid.slab = s.path ? s.Min : (int)s.M;
        mid.Q = mid.slab / n;
        mid.digrev = (const int*)ddr;
        mid.mat_f = dmf;
        mid.mat_i = dmi;
    }
    if (s.path == 0) {
        FwdParams& P = pl->fused;
        memset(&P, 0, sizeof(P));
        P.M = (int)s.M;
        P.N = (int)s.N;
        P.nst = s.p - 1;
        P.outer_half = s.full ? 0 : 1;
        for (int i = 0; i < P.nst; ++i) {
            P.st[i] = reg[i];
            P.st[i].Sb = (int)S[i];
            P.st[i].sb = (int)str[i];
            P.st[i].Cb = 1;
            P.st[i].tw_mul = 1;
            P.st[i].ncols = (int)(s.M / s.f[i]);
        }
        P.mid = mid;
        P.Qo = 1;
        P.threads = s.thr_fused;
    } else {
        FwdParams& O = pl->outer;
        memset(&O, 0, sizeof(O));
        O.M = (int)s.M;
        O.N = (int)s.N;
        O.nst = s.n_outer;
        O.outer_half = s.full ? 0 : 1;
        for (int i = 0; i < s.n_outer; ++i) {
            O.st[i] = reg[i];
            O.st[i].Sb = (int)(S[i] / s.Min);
            O.st[i].sb = (int)(str[i] / s.Min);
            O.st[i].Cb = s.ct;
            O.st[i].tw_mul = s.Min;
            O.st[i].ncols = s.Qo * s.ct / s.f[i];
        }
        O.Qo = s.Qo;
        O.ct = s.ct;
        O.threads = s.thr_outer;
        FwdParams& I = pl->inner;
        memset(&I, 0, sizeof(I));
        I.M = (int)s.M;
        I.N = (int)s.N;
        I.nst = s.p - 1 - s.n_outer;
        I.outer_half = 0;
        for (int i = 0; i < I.nst; ++i) {
            const int gi = s.n_outer + i;
            I.st[i] = reg[gi];
            I.st[i].Sb = (int)S[gi];
            I.st[i].sb = (int)str[gi];
            I.st[i].Cb = 1;
            I.st[i].tw_mul = 1;
            I.st[i].ncols = 2 * s.Min / s.f[gi];
        }
        I.mid = mid;
        I.Qo = s.Qo;
        I.nunits = s.Qo / 2 + 1;
        I.threads = s.thr_inner;
        std::vector<int> dro = build_digrev(s.f, str, s.n_outer, s.Min);
        void* d = nullptr;
        if (upload(pl, dro.data(), dro.size() * 4, &d) != hipSuccess) return FFTCONV_ERR_HIP;
        I.digrev_o = (const int*)d;
        O.digrev_o = (const int*)d;
    }
    if (row_kernel_applies(s)) {
        const int NB = s.f[1];
        const bool bf = s.dtype == FFTCONV_BF16;
        std::vector<uint16_t> f1b = row_f1b(bf, s.full), i1a = row_i1a(s.full),
                              i2b = row_i2b(NB), i2bs = row_i2b(NB, true);
        std::vector<uint8_t> f2a = row_f2a(NB);
        std::vector<uint16_t> twf = row_twiddles(NB, false), twi = row_twiddles(NB, true);
        RowParams& R = pl->row;
        void* d = nullptr;
        if (upload(pl, f1b.data(), f1b.size() * 2, &d) != hipSuccess) return FFTCONV_ERR_HIP;
        R.f1b = d;
        R.f1h = d;
        if (bf) {
            // gated rows feed u (.) w to the first stage as f16
            std::vector<uint16_t> f1h = row_f1b(false, s.full);
            if (upload(pl, f1h.data(), f1h.size() * 2, &d) != hipSuccess) return FFTCONV_ERR_HIP;
            R.f1h = d;
        }
        if (upload(pl, i1a.data(), i1a.size() * 2, &d) != hipSuccess) return FFTCONV_ERR_HIP;
        R.i1a = d;
        if (upload(pl, i2b.data(), i2b.size() * 2, &d) != hipSuccess) return FFTCONV_ERR_HIP;
        R.i2b = d;
        if (upload(pl, i2bs.data(), i2bs.size() * 2, &d) != hipSuccess) return FFTCONV_ERR_HIP;
        R.i2bs = d;
        if (upload(pl, f2a.data(), f2a.size(), &d) != hipSuccess) return FFTCONV_ERR_HIP;
        R.f2a = d;
        if (upload(pl, twf.data(), twf.size() * 2, &d) != hipSuccess) return FFTCONV_ERR_HIP;
        R.twf = (const uint32_t*)d;
        if (upload(pl, twi.data(), twi.size() * 2, &d) != hipSuccess) return FFTCONV_ERR_HIP;
        R.twi = (const uint32_t*)d;
        R.N = (int)s.N;
        R.full = s.full ? 1 : 0;
        pl->use_row = true;
        pl->row_nb = NB;
        // fixed part: the four stage tables, claim counter, exchange
        // scratch of every wave; the rest of a 144 KB budget (one
        // workgroup per CU) holds spectra
        const int NH = s.full ? 2 : 1;
        const int tables = NH * ((bf ? 8 : 4) + 4) + (NB / 8) * (NB / 16) + (NB / 16) * 2 * (NB / 16);
        const int fixed = tables * 64 * 16 + 16 + kRowWaves * 16 * NB * 4;
        pl->row_max_channels = (144 * 1024 - fixed) / ((int)s.M * 8);
        pl->lds_row = fixed + (int)pl->row_max_channels * (int)s.M * 8;
    }
    if (s.wide_P) {
        const int P = s.wide_P;
        std::vector<uint16_t> f1b = wide_f1b(P), i1a = wide_i1a(P), i2b = row_i2b(32),
                              i2bs = row_i2b(32, true);
        std::vector<uint8_t> f2a = row_f2a(32);
        std::vector<uint16_t> twf = row_twiddles(32, false), two = wide_outer_twiddles(P);
        WideParams& W = pl->wide;
        void* d = nullptr;
        if (upload(pl, f1b.data(), f1b.size() * 2, &d) != hipSuccess) return FFTCONV_ERR_HIP;
        W.f1b = d;
        if (upload(pl, i1a.data(), i1a.size() * 2, &d) != hipSuccess) return FFTCONV_ERR_HIP;
        W.i1a = d;
        if (upload(pl, i2b.data(), i2b.size() * 2, &d) != hipSuccess) return FFTCONV_ERR_HIP;
        W.i2b = d;
        if (upload(pl, i2bs.data(), i2bs.size() * 2, &d) != hipSuccess) return FFTCONV_ERR_HIP;
        W.i2bs = d;
        if (upload(pl, f2a.data(), f2a.size(), &d) != hipSuccess) return FFTCONV_ERR_HIP;
        W.f2a = d;
        if (upload(pl, twf.data(), twf.size() * 2, &d) != hipSuccess) return FFTCONV_ERR_HIP;
        W.twf = (const uint32_t*)d;
        if (upload(pl, two.data(), two.size() * 2, &d) != hipSuccess) return FFTCONV_ERR_HIP;
        W.two = (const uint32_t*)d;
        W.N = (int)s.N;
        W.pairs = P / 2;
        W.full = s.full ? 1 : 0;
        // stage tables (16 KB) + outer twiddles (read through L2 at P = 32)
        // + one row of f16 points + the k_b exchange
        pl->lds_wide = 16 * 1024 + (P <= 16 ? (P / 2) * 4096 : 0) + (int)s.M * 4 +
                       39 * 16 * 4 + 16;
        // two waves per SIMD (256 registers each), LDS permitting
        const int by_waves = 8 / (wide_threads(P) / 64);
        const int by_lds = (160 * 1024) / pl->lds_wide;
        pl->wide_wgs_per_cu = by_waves < by_lds ? by_waves : by_lds;
        if (pl->wide_wgs_per_cu < 1) pl->wide_wgs_per_cu = 1;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, pl->device) == hipSuccess && prop.multiProcessorCount > 0)
        pl->num_cu = prop.multiProcessorCount;
    return FFTCONV_OK;
}

fftconv_status build_mp_tables(fftconv_plan_s* pl) {
    const Shape& s = pl->s;
    std::vector<uint16_t> f1b = wide_f1b(4), i1a = wide_i1a(4), i2b = row_i2b(32),
                          i2bs = row_i2b(32, true);
    std::vector<uint8_t> f2a = row_f2a(32);
    std::vector<uint16_t> twf = row_twiddles(32, false), two = mp_inner_twiddles();
    MpInnerParams& I = pl->mp;
    void* d = nullptr;
    if (upload(pl, f1b.data(), f1b.size() * 2, &d) != hipSuccess) return FFTCONV_ERR_HIP;
    I.f1b = d;
    if (upload(pl, i1a.data(), i1a.size() * 2, &d) != hipSuccess) return FFTCONV_ERR_HIP;
    I.i1a = d;
    if (upload(pl, i2b.data(), i2b.size() * 2, &d) != hipSuccess) return FFTCONV_ERR_HIP;
    I.i2b = d;
    if (upload(pl, i2bs.data(), i2bs.size() * 2, &d) != hipSuccess) return FFTCONV_ERR_HIP;
    I.i2bs = d;
    if (upload(pl, f2a.data(), f2a.size(), &d) != hipSuccess) return FFTCONV_ERR_HIP;
    I.f2a = d;
    if (upload(pl, twf.data(), twf.size() * 2, &d) != hipSuccess) return FFTCONV_ERR_HIP;
    I.twf = (const uint32_t*)d;
    if (upload(pl, two.data(), two.size() * 2, &d) != hipSuccess) return FFTCONV_ERR_HIP;
    I.two = (const uint32_t*)d;
    I.M = (int)s.M;
    I.Po = (int)(s.M / 4096);
    I.upr_active = I.Po / 2;
    I.P1 = s.mp_P1;
    I.P2 = s.mp_P2;
    std::vector<float> t1 = col_twiddles((long long)s.M, (long long)s.M / s.mp_P1);
    if (upload(pl, t1.data(), t1.size() * 4, &d) != hipSuccess) return FFTCONV_ERR_HIP;
    pl->mp_tw1 = (const float2*)d;
    if (s.mp_P2 > 1) {
        std::vector<float> t2 = col_twiddles((long long)s.M / s.mp_P1, 4096);
        if (upload(pl, t2.data(), t2.size() * 4, &d) != hipSuccess) return FFTCONV_ERR_HIP;
        pl->mp_tw2 = (const float2*)d;
    }
    if (s.mp_P1 == 32 && s.mp_P2 == 32) {
        std::vector<uint16_t> a1 = col2m_dft_a(s.dtype == FFTCONV_BF16, 16), a2 = col2m_dft_a(false, 32);
        std::vector<float> tm = col2m_twiddles((long long)s.M);
        if (upload(pl, a1.data(), a1.size() * 2, &d) != hipSuccess) return FFTCONV_ERR_HIP;
        pl->mp2m_a1 = (const uint4*)d;
        pl->mp2m_a1h = pl->mp2m_a1;
        if (s.dtype == FFTCONV_BF16) {
            // gated rows feed u (.) w to level 1 as f16
            std::vector<uint16_t> a1h = col2m_dft_a(false, 16);
            if (upload(pl, a1h.data(), a1h.size() * 2, &d) != hipSuccess) return FFTCONV_ERR_HIP;
            pl->mp2m_a1h = (const uint4*)d;
        }
        if (upload(pl, a2.data(), a2.size() * 2, &d) != hipSuccess) return FFTCONV_ERR_HIP;
        pl->mp2m_a2 = (const uint4*)d;
        if (upload(pl, tm.data(), tm.size() * 4, &d) != hipSuccess) return FFTCONV_ERR_HIP;
        pl->mp2m_tm = (const float2*)d;
        std::vector<uint16_t> ia1 = col2m_dft_a(false, 32, 16, true), ia2 = col2m_dft_a(false, 32, 32, true);
        if (upload(pl, ia1.data(), ia1.size() * 2, &d) != hipSuccess) return FFTCONV_ERR_HIP;
        pl->mp2m_ia1 = (const uint4*)d;
        if (upload(pl, ia2.data(), ia2.size() * 2, &d) != hipSuccess) return FFTCONV_ERR_HIP;
        pl->mp2m_ia2 = (const uint4*)d;
    }
    // stage tables (16 KB) + inner twiddles (20 KB) + two slabs of f16
    // points (32 KB) + the k_b exchange + claims + outer-stage operands
    pl->lds_mp = 16 * 1024 + 20 * 1024 + 8 * 1024 * 4 + 39 * 16 * 4 + 16 + 4 * 64 * 8;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, pl->device) == hipSuccess && prop.multiProcessorCount > 0)
        pl->num_cu = prop.multiProcessorCount;
    return FFTCONV_OK;
}

// The kernel-gradient plan of a plan: the same N and dtype on the
// LDS-staged kernels (two lines per workgroup), whose accumulators must fit
// the kernels' fixed number of lane-slot steps per wave (two for a 16-point
// innermost stage, one for a 32-point one).

fftconv_status build_grad_plan(fftconv_plan_s* pl) {
    // plans at FFT size N (circular operators) have no kernel gradient
    if (pl->s.full) return FFTCONV_OK;
    if (pl->s.wide_P == 32) {
        // the kernel gradient at 32K runs on the multi-pass engine
        Shape m;
        fftconv_status st = make_shape_fixed(pl->s.N, 4, pl->s.dtype, m, false, false);
        if (st != FFTCONV_OK) return st;
        if (!m.mp_P1) return FFTCONV_ERR_UNSUPPORTED;
        fftconv_plan_s* kp = new (std::nothrow) fftconv_plan_s();
        if (!kp) return FFTCONV_ERR_HIP;
        kp->s = m;
        kp->device = pl->device;
        st = build_device_tables(kp);
        if (st != FFTCONV_OK) {
            free_plan(kp);
            return st;
        }
        pl->kg = kp;
    }
    Shape g;
    fftconv_status st = make_shape(pl->s.N, 0, pl->s.dtype, g, true);
    if (st != FFTCONV_OK) return st;
    const int nm = g.f[g.p - 1];
    const int slab = g.path ? g.Min : (int)g.M;
    const int Q = slab / nm;
    const int LS = g.path ? Q : Q / 2;
    const int waves = (g.path ? g.thr_inner : g.thr_fused) / 64;
    if ((LS + 15) / 16 > (nm == 32 ? 1 : 2) * waves) return FFTCONV_ERR_UNSUPPORTED;
    fftconv_plan_s* gp = new (std::nothrow) fftconv_plan_s();
    if (!gp) return FFTCONV_ERR_HIP;
    gp->s = g;
    gp->device = pl->device;
    st = build_device_tables(gp);
    if (st != FFTCONV_OK) {
        free_plan(gp);
        return st;
    }
    pl->grad = gp;
    return FFTCONV_OK;
}

// Batch slices of the fused kernel-gradient pass: enough workgroups to
// give every SIMD a few waves (each slice is a workgroup per channel).
int kgrad_splits(const fftconv_plan_s* pl, size_t B, size_t H) {
    const Shape& g = pl->grad->s;
    if (g.path != 0 || B <= 1 || H == 0) return 1;
    const long long waves = g.thr_fused / 64;
    const long long want = 4LL * 4 * pl->num_cu;   // waves: four per SIMD
    long long n = (want + H * waves - 1) / (H * waves);
    if (n > (long long)B) n = (long long)B;
    if (n > 64) n = 64;
    return n < 1 ? 1 : (int)n;
}

// The row-engine kernel gradient (N = 1024, 16-bit I/O).
bool kgrad_on_row(const fftconv_plan_s* pl) {
    return pl->use_row && pl->row_nb == 32 && pl->s.dtype != FFTCONV_F32;
}

// Batch slices per channel for the engine kernel gradients: the (channel,
// slice) tasks run `at_once` at a time, each over ceil(B / S) rows, so the
// time goes as rounds x rows per task; the smallest S (fewest partial rows
// to sum) of the minimum, at most 64.
int kgrad_best_slices(size_t B, size_t H, long long at_once) {
    if (B == 0 || H == 0 || at_once <= 0) return 1;
    const long long smax = std::min<long long>((long long)B, 64);
    long long best = 1, best_cost = -1;
    for (long long sl = 1; sl <= smax; ++sl) {
        const long long rounds = ((long long)H * sl + at_once - 1) / at_once;
        const long long rows = ((long long)B + sl - 1) / sl;
        const long long cost = rounds * rows;
        if (best_cost < 0 || cost < best_cost) {
            best_cost = cost;
            best = sl;
        }
    }
    return (int)best;
}

// Row engine: one wave per task, eight-wave workgroups, one per CU.
int kgrad_row_slices(const fftconv_plan_s* pl, size_t B, size_t H) {
    return kgrad_best_slices(B, H, 8LL * pl->num_cu);
}

// The wide-engine kernel gradient (N = P x 1024, 16-bit I/O): a workgroup
// per (channel, slice), two per CU.
int kgrad_wide_slices(const fftconv_plan_s* pl, size_t B, size_t H) {
    return kgrad_best_slices(B, H, 2LL * pl->num_cu);
}

// The multi-pass engine kernel gradient (N >= 32K, 16-bit I/O): chunks of
// channels x batch rows whose outer-transformed rows of u and of dy each
// fit one workspace chunk (1 GB); every batch chunk runs the whole pipeline
// and adds its share to dk (the inverse transform is linear).
bool kgrad_on_mp(const fftconv_plan_s* pl, size_t) {
    return pl->s.mp_P1 && pl->s.dtype != FFTCONV_F32;
}

size_t kgrad_mp_batch(const fftconv_plan_s* pl, size_t B) {
    size_t bc = kMpChunkBytes / (pl->s.M * 4);
    if (bc > B) bc = B;
    return bc < 1 ? 1 : bc;
}

size_t kgrad_mp_channels(const fftconv_plan_s* pl, size_t B, size_t H) {
    const size_t per_ch = kgrad_mp_batch(pl, B) * pl->s.M * 4;
    size_t hc = kMpChunkBytes / per_ch;
    if (hc > H) hc = H;
    return hc < 1 ? 1 : hc;
}

size_t kgrad_workspace_bytes(const fftconv_plan_s* pl, size_t B, size_t H) {
    if (pl->kg) return kgrad_workspace_bytes(pl->kg, B, H);
    if (kgrad_on_row(pl)) return (size_t)kgrad_row_slices(pl, B, H) * H * 64 * 32 * 4;
    if (kgrad_on_mp(pl, B)) {
        // rows of u and dy after the forward column passes, and one result
        // row per channel of the chunk; the claim counters the column passes
        // clear
        const size_t bc = kgrad_mp_batch(pl, B), hc = kgrad_mp_channels(pl, B, H);
        return (2 * bc + 1) * hc * pl->s.M * 4 + kClaimBytes;
    }
    if (pl->s.wide_P)
        return (size_t)kgrad_wide_slices(pl, B, H) * H * (pl->s.wide_P / 2) * 64 * 64 * 4;
    const Shape& g = pl->grad->s;
    if (g.path == 0) {
        const int ns = kgrad_splits(pl, B, H);
        return ns > 1 ? (size_t)ns * H * g.N * 4 : 0;
    }
    // outer-transformed rows of u and dy, and one result row per channel
    return (2 * B * H + H) * g.M * 8;
}

int kgrad_lds(const Shape& g) {
    return g.path ? 4 * g.Min * 8 + (g.thr_inner / 64) * 64 * 8
                  : (int)g.M * 2 * 8 + (g.thr_fused / 64) * 64 * 8;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Forward column pass(es) of the multi-pass path for one channel chunk:
// channels h0 .. h0 + hc - 1 of all B rows of src ([B][H][N]) into
// workspace rows b * hc + (h - h0), in the layout the inner passes read.
hipError_t mp_cols_fwd(const fftconv_plan_s* plan, int io, const void* src, void* ws,
                       uint32_t* ctr, size_t B, size_t H, size_t h0, size_t hc,
                       hipStream_t st) {
    const Shape& s = plan->s;
    const long long rows = (long long)B * (long long)hc;
    if (s.mp_P2 > 1) {
        MpCol2Params D{};
        D.rows = rows;
        D.H = (int)H;
        D.h0 = (int)h0;
        D.hc = (int)hc;
        D.M = (int)s.M;
        D.tw1 = plan->mp_tw1;
        D.tw2 = plan->mp_tw2;
        D.u = src;
        D.ws = ws;
        D.ctr = ctr;
        D.grid = (int)std::min<long long>(mp_col2_tiles(s.mp_P2, rows),
                                          std::max<long long>(16, (2LL * plan->num_cu) & ~15LL));
        if (plan->mp2m_a1) {
            D.a1 = plan->mp2m_a1;
            D.a2 = plan->mp2m_a2;
            D.tm = plan->mp2m_tm;
            D.grid = (int)std::min<long long>(rows * 128, plan->num_cu);
            return launch_mp_col2m_fwd(io, D, st);
        }
        return launch_mp_col2(io, s.mp_P1, s.mp_P2, false, D, st);
    }
    MpColParams C{};
    C.rows = rows;
    C.H = (int)H;
    C.h0 = (int)h0;
    C.hc = (int)hc;
    C.M = (int)s.M;
    C.S = (int)(s.M / s.mp_P1);
    C.tw = plan->mp_tw1;
    C.u = src;
    C.ws = ws;
    C.ctr = ctr;
    return launch_mp_col(io, s.mp_P1, 0, C, st);
}

// Both outer levels' pass parameters of one chunk, from its one-level
// column-pass parameters: persistent workgroups, two per CU, a multiple of
// 16 (the tile count is a multiple of 64).
MpCol2Params mp_col2_params(const fftconv_plan_s* plan, const MpColParams& C) {
    MpCol2Params D{};
    D.rows = C.rows;
    D.H = C.H;
    D.h0 = C.h0;
    D.hc = C.hc;
    D.M = C.M;
    D.tw1 = plan->mp_tw1;
    D.tw2 = plan->mp_tw2;
    D.u = C.u;
    D.y = C.y;
    D.w = C.w;
    D.v = C.v;
    D.ws = C.ws;
    D.ctr = C.ctr;
    D.full = C.full;
    D.grid = (int)std::min<long long>(mp_col2_tiles(plan->s.mp_P2, D.rows),
                                      std::max<long long>(16, (2LL * plan->num_cu) & ~15LL));
    return D;
}

// Workgroups of the inner pass for `units` slab-pair units: two per CU, a
// multiple of 8 (every XCD the same share), no more than the units need.
int mp_inner_grid(const fftconv_plan_s* plan, long long units) {
    long long G = 2LL * plan->num_cu;
    G = G < 8 ? 8 : G & ~7LL;
    const long long need = (units + 7) & ~7LL;
    return (int)(G < need ? G : need);
}

// The rest of one multi-pass chunk once its workspace holds the forward
// column passes' output: the inner pass (the spectrum product included),
// the clearing of the units it skips, and the inverse column pass(es) into
// the chunk's output rows.  C: the chunk's one-level column-pass parameters
// (workspace, counters, output rows and gate).
hipError_t mp_inner_inverse(const fftconv_plan_s* plan, int io, const MpInnerParams& I,
                            const MpColParams& C, hipStream_t st) {
    const Shape& s = plan->s;
    hipError_t e = launch_mp_inner(io, I, plan->lds_mp, st);
    if (e == hipSuccess)
        e = launch_mp_zero_units(C.ws, C.rows, (int)s.M, I.Po, I.P1, I.P2, I.upr_active, st);
    if (e != hipSuccess) return e;
    if (s.mp_P2 > 1) {
        const MpCol2Params D = mp_col2_params(plan, C);
        if (plan->mp2m_ia1) {
            MpCol2Params F = D;
            F.a1 = plan->mp2m_ia1;
            F.a2 = plan->mp2m_ia2;
            F.tm = plan->mp2m_tm;
            F.grid = (int)std::min<long long>(D.rows * 128, plan->num_cu);
            return launch_mp_col2m_inv(io, F, st);
        }
        return launch_mp_col2(io, s.mp_P1, s.mp_P2, true, D, st);
    }
    return launch_mp_col(io, s.mp_P1, 3, C, st);
}

// Channels per chunk of the multi-pass path: the passes run chunk by chunk
// to bound the workspace (B * hc * M f16 complex, at most 1 GB).  Every
// chunk costs three launches with their ramp-up and tail; measured at
// N = 4M, 256 MB chunks (small enough for the Infinity Cache) ran 5%
// slower than 1 GB ones, so the cache does not decide the size.
// Batch rows per chunk: all of them unless one channel's rows alone exceed
// the bound (then the chunk is one channel of a slice of the batch).
// `cap` is the chunk bound in bytes (kMpChunkBytes, or what the static
// scratch array of the allocation-free call leaves beside the counters).
size_t mp_chunk_batch(const Shape& s, size_t B, size_t cap = kMpChunkBytes) {
    size_t bc = cap / (s.M * 4);
    if (bc < 1) bc = 1;
    return B < bc ? (B ? B : 1) : bc;
}

size_t mp_chunk_channels(const Shape& s, size_t B, size_t H, size_t cap = kMpChunkBytes) {
    B = mp_chunk_batch(s, B, cap);
    const size_t per_ch = B * s.M * 4;
    size_t hc = cap / per_ch;
    if (hc < 1) hc = 1;
    if (hc > H) hc = H;
    return hc;
}

// Workspace bytes of a forward call whose multi-pass chunks are bounded by
// `cap` (fftconv_workspace_bytes with the default bound).
size_t forward_workspace_bytes(const fftconv_plan_s* plan, size_t B, size_t H,
                               size_t cap = kMpChunkBytes) {
    if (plan->s.path == 0) return 0;
    // multi-pass: one channel chunk of f16 complex rows, then the counters
    if (plan->s.mp_P1)
        return mp_chunk_batch(plan->s, B, cap) * mp_chunk_channels(plan->s, B, H, cap) *
                   plan->s.M * 4 + kClaimBytes;
    return B * H * plan->s.M * 8;
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

}  // namespace

// ------------------------------------------------------------------ C ABI

extern "C" {

const char* fftconv_version(void) { return "fftconv-gfx950 0.2"; }

fftconv_status fftconv_stream_copy(const void* src, void* dst, size_t bytes, void* stream) {
    if (!src || !dst || (bytes & 15)) return FFTCONV_ERR_INVALID_ARG;
    if (!aligned16(src) || !aligned16(dst)) return FFTCONV_ERR_ALIGNMENT;
    if (overlap(src, bytes, dst, bytes)) return FFTCONV_ERR_INVALID_ARG;
    if (bytes == 0) return FFTCONV_OK;
    int dev = 0, cu = 256;
    if (hipGetDevice(&dev) != hipSuccess) return FFTCONV_ERR_HIP;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess && prop.multiProcessorCount > 0)
        cu = prop.multiProcessorCount;
    return launch_stream_copy(src, dst, (long long)(bytes / 16), cu, (hipStream_t)stream) == hipSuccess
               ? FFTCONV_OK : FFTCONV_ERR_HIP;
}

const char* fftconv_status_string(fftconv_status st) {
    switch (st) {
    case FFTCONV_OK: return "ok";
    case FFTCONV_ERR_INVALID_ARG: return "invalid argument";
    case FFTCONV_ERR_UNSUPPORTED: return "unsupported length, order or dtype";
    case FFTCONV_ERR_ALIGNMENT: return "tensor pointer not 16-byte aligned";
    case FFTCONV_ERR_WORKSPACE: return "workspace missing or too small";
    case FFTCONV_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

fftconv_status fftconv_plan_query(size_t N, int p, fftconv_dtype dtype,
                                  fftconv_plan_info* info) {
    if (!info) return FFTCONV_ERR_INVALID_ARG;
    Shape s;
    fftconv_status st = make_shape(N, p, dtype, s);
    if (st != FFTCONV_OK) return st;
    fill_info(s, info);
    return FFTCONV_OK;
}

fftconv_status fftconv_plan_estimate(size_t N, int p, fftconv_dtype dtype, int lds_staged,
                                     size_t B, size_t H, fftconv_estimate* out) {
    if (!out) return FFTCONV_ERR_INVALID_ARG;
    Shape s;
    fftconv_status st;
    if (lds_staged) {
        if (p == 0) {
            // the LDS-staged kernels' own choice: lowest predicted order
            st = FFTCONV_ERR_UNSUPPORTED;
            double best = 0;
            for (int q = 2; q <= kMaxStages; ++q) {
                Shape c;
                if (make_shape_fixed(N, q, dtype, c, false, true) != FFTCONV_OK) continue;
                const double t = estimate(c, 0, 1).t_pred;
                if (st != FFTCONV_OK || t < best * (1.0 - 1e-9)) {
                    best = t;
                    s = c;
                    st = FFTCONV_OK;
                }
            }
        } else {
            st = make_shape_fixed(N, p, dtype, s, false, true);
        }
    } else {
        st = make_shape(N, p, dtype, s);
    }
    if (st != FFTCONV_OK) return st;
    memset(out, 0, sizeof(*out));
    fftconv_plan_info info;
    fill_info(s, &info);
    out->order = s.p;
    for (int i = 0; i < s.p; ++i) out->factors[i] = s.f[i];
    out->path = info.path;
    out->kernel_variant = info.kernel_variant;
    const CostTerms c = estimate(s, B, H);
    out->hbm_bytes = c.hbm_bytes;
    out->mfma_flops = c.mfma_flops;
    out->valu_flops = c.valu_flops_f16 + c.valu_flops_f32;
    out->lds_bytes = c.lds_bytes;
    out->t_hbm = c.t_hbm;
    out->t_mfma = c.t_mfma;
    out->t_valu = c.t_valu;
    out->t_lds = c.t_lds;
    out->t_pred = c.t_pred;
    return FFTCONV_OK;
}

fftconv_status fftconv_plan(size_t N, int p, fftconv_dtype dtype,
                            fftconv_plan_t* out) {
    return plan_create(N, p, dtype, false, out);
}

fftconv_status fftconv_plan_circular(size_t N, int p, fftconv_dtype dtype,
                                     fftconv_plan_t* out) {
    return plan_create(N, p, dtype, true, out);
}

fftconv_status fftconv_plan_circular_query(size_t N, int p, fftconv_dtype dtype,
                                           fftconv_plan_info* info) {
    if (!info) return FFTCONV_ERR_INVALID_ARG;
    Shape s;
    fftconv_status st = make_shape(N, p, dtype, s, false, true);
    if (st != FFTCONV_OK) return st;
    fill_info(s, info);
    return FFTCONV_OK;
}
}  // extern "C"

namespace {
fftconv_status plan_create(size_t N, int p, fftconv_dtype dtype, bool full,
                           fftconv_plan_t* out) {
    if (!out) return FFTCONV_ERR_INVALID_ARG;
    *out = nullptr;
    Shape s;
    fftconv_status st = make_shape(N, p, dtype, s, false, full);
    if (st != FFTCONV_OK) return st;
    fftconv_plan_s* pl = new (std::nothrow) fftconv_plan_s();
    if (!pl) return FFTCONV_ERR_HIP;
    pl->s = s;
    if (hipGetDevice(&pl->device) != hipSuccess) {
        delete pl;
        return FFTCONV_ERR_HIP;
    }
    st = build_device_tables(pl);
    if (st == FFTCONV_OK) st = build_grad_plan(pl);
    if (st != FFTCONV_OK) {
        free_plan(pl);
        return st;
    }
    *out = pl;
    return FFTCONV_OK;
}
}  // namespace

extern "C" {

fftconv_status fftconv_plan_get_info(fftconv_plan_t plan,
                                     fftconv_plan_info* info) {
    if (!plan || !info) return FFTCONV_ERR_INVALID_ARG;
    fill_info(plan->s, info);
    return FFTCONV_OK;
}

void fftconv_plan_destroy(fftconv_plan_t plan) { free_plan(plan); }

size_t fftconv_spectrum_bytes(fftconv_plan_t plan, size_t H) {
    if (!plan) return 0;
    return H * plan->s.M * kf_entry_bytes(plan->s.dtype);
}

size_t fftconv_backward_workspace_bytes(fftconv_plan_t plan, size_t B, size_t H) {
    if (!plan || !plan->grad) return 0;
    const size_t a = fftconv_workspace_bytes(plan, B, H);
    const size_t b = kgrad_workspace_bytes(plan, B, H);
    return a > b ? a : b;
}

size_t fftconv_workspace_bytes(fftconv_plan_t plan, size_t B, size_t H) {
    if (!plan) return 0;
    return forward_workspace_bytes(plan, B, H);
}

fftconv_status fftconv_kernel_spectrum(fftconv_plan_t plan, const float* k,
                                       size_t H, void* k_f, void* stream) {
    return fftconv_kernel_spectrum_kind(plan, k, H, FFTCONV_CAUSAL, k_f, stream);
}

fftconv_status fftconv_kernel_spectrum_kind(fftconv_plan_t plan, const float* k,
                                            size_t H, fftconv_kernel_kind kind,
                                            void* k_f, void* stream) {
    return spectrum_impl(plan, k, H, kind, -1, k_f, stream);
}

fftconv_status fftconv_kernel_spectrum_lowpass(fftconv_plan_t plan, const float* k,
                                               size_t H, size_t cutoff, void* k_f,
                                               void* stream) {
    if (!plan) return FFTCONV_ERR_INVALID_ARG;
    if (cutoff > plan->s.N) return FFTCONV_ERR_INVALID_ARG;
    return spectrum_impl(plan, k, H, FFTCONV_CAUSAL, (long long)cutoff, k_f, stream);
}

}  // extern "C"

namespace {

// Kernel spectrum of operator `kind`, band-limited to frequencies within
// `cutoff` of zero when cutoff >= 0.
fftconv_status spectrum_impl(fftconv_plan_t plan, const float* k, size_t H,
                             fftconv_kernel_kind kind, long long cutoff, void* k_f,
                             void* stream, int blk_a, int blk_d) {
    if (!plan) return FFTCONV_ERR_INVALID_ARG;
    if ((int)kind < 0 || (int)kind > 3) return FFTCONV_ERR_INVALID_ARG;
    // a plan at FFT size N computes the circular kinds only, unmasked
    if (plan->s.full && (kind == FFTCONV_CAUSAL || kind == FFTCONV_CAUSAL_ADJOINT ||
                         cutoff >= 0 || blk_a > 0 || blk_d > 0))
        return FFTCONV_ERR_UNSUPPORTED;
    if (H == 0) return FFTCONV_OK;
    if (!k || !k_f) return FFTCONV_ERR_INVALID_ARG;
    if (!aligned16(k) || !aligned16(k_f)) return FFTCONV_ERR_ALIGNMENT;
    const Shape& s = plan->s;
    if (overlap(k, H * s.N * 4, k_f, fftconv_spectrum_bytes(plan, H)))
        return FFTCONV_ERR_INVALID_ARG;
    if (H > 0x7fffffff) return FFTCONV_ERR_UNSUPPORTED;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return FFTCONV_ERR_HIP;
    if (dev != plan->device) return FFTCONV_ERR_INVALID_ARG;
    hipStream_t st = (hipStream_t)stream;
    // the real transform's length: 2N (causal padding) or N (full plans)
    const long long L = 2LL * (long long)s.M;
    const size_t per_ch = (size_t)L * sizeof(float2) * 2;
    size_t hc = (size_t)512 << 20;
    hc = hc / per_ch;
    if (hc < 1) hc = 1;
    if (hc > H) hc = H;
    void* X = nullptr;
    if (hipMallocAsync(&X, hc * per_ch, st) != hipSuccess) return FFTCONV_ERR_HIP;
    float2* X0 = (float2*)X;
    float2* X1 = X0 + hc * L;
    hipError_t e = hipSuccess;
    const int io = (int)s.dtype;
    for (size_t h0 = 0; h0 < H && e == hipSuccess; h0 += hc) {
        const int cnt = (int)((H - h0) < hc ? (H - h0) : hc);
        e = launch_kpad(k + h0 * s.N, X0, cnt, (int)s.N, (int)L, (int)kind, st);
        float2 *a = X0, *b = X1;
        for (long long Ns = 1; Ns < L && e == hipSuccess; Ns *= 2) {
            e = launch_stockham(a, b, cnt, (int)L, (int)Ns, st);
            float2* t = a;
            a = b;
            b = t;
        }
        if (e == hipSuccess && cutoff >= 0) e = launch_band_limit(a, cnt, (int)L, (int)cutoff, st);
        if (e == hipSuccess && (blk_a > 0 || blk_d > 0))
            e = launch_block_mask(a, cnt, (int)L, (int)s.M, sparse_outer(s), blk_a, blk_d, st);
        if (e != hipSuccess) break;
        if (s.mp_P1) {
            MpCoefParams mp{};
            mp.M = (int)s.M;
            mp.L = (int)L;
            mp.Po = (int)(s.M / 4096);
            mp.h0 = (int)h0;
            mp.hcount = cnt;
            mp.X = a;
            mp.kf = k_f;
            e = launch_mp_coef(mp, st);
            continue;
        }
        if (s.wide_P) {
            WideCoefParams wp{};
            wp.M = (int)s.M;
            wp.L = (int)L;
            wp.P = s.wide_P;
            wp.h0 = (int)h0;
            wp.hcount = cnt;
            wp.X = a;
            wp.kf = k_f;
            e = launch_wide_coef(wp, st);
            continue;
        }
        SpecParams sp{};
        sp.M = (int)s.M;
        sp.N = (int)s.N;
        sp.L = (int)L;
        sp.p = s.p;
        for (int i = 0; i < s.p; ++i) sp.factors[i] = s.f[i];
        sp.h0 = (int)h0;
        sp.hcount = cnt;
        sp.X = a;
        sp.kf = k_f;
        e = launch_alphabeta(io, sp, st);
    }
    hipError_t e2 = hipFreeAsync(X, st);
    if (e != hipSuccess || e2 != hipSuccess) return FFTCONV_ERR_HIP;
    return FFTCONV_OK;
}

// Shared body of the plain and the gated forward call; w and v are both
// null (plain) or both set (gated), which the callers guarantee.
// Argument checks of a forward call (the plan's length, pointers,
// alignment, aliasing, workspace size); FFTCONV_OK when the call may run.
fftconv_status forward_check(fftconv_plan_t plan, const void* u, const void* w,
                             const void* v, const void* k_f, void* y, size_t B,
                             size_t H, size_t N, void* workspace,
                             size_t workspace_bytes, size_t chunk_cap) {
    if (!plan) return FFTCONV_ERR_INVALID_ARG;
    const Shape& s = plan->s;
    if (N != s.N) return FFTCONV_ERR_INVALID_ARG;
    const size_t rows = B * H;
    if (B != 0 && rows / B != H) return FFTCONV_ERR_INVALID_ARG;
    if (rows == 0) return FFTCONV_OK;
    if (!u || !k_f || !y) return FFTCONV_ERR_INVALID_ARG;
    if (!aligned16(u) || !aligned16(y) || !aligned16(k_f)) return FFTCONV_ERR_ALIGNMENT;
    if (w && (!aligned16(w) || !aligned16(v))) return FFTCONV_ERR_ALIGNMENT;
    if (rows > 0x7fffffffULL || H > 0x7fffffffULL) return FFTCONV_ERR_UNSUPPORTED;
    const size_t esz = s.dtype == FFTCONV_F32 ? 4 : 2;
    const size_t io_bytes = rows * N * esz;
    const size_t kf_bytes = fftconv_spectrum_bytes(plan, H);
    if (overlap(y, io_bytes, u, io_bytes) || overlap(y, io_bytes, k_f, kf_bytes))
        return FFTCONV_ERR_INVALID_ARG;
    if (w && (overlap(y, io_bytes, w, io_bytes) || overlap(y, io_bytes, v, io_bytes)))
        return FFTCONV_ERR_INVALID_ARG;
    const size_t ws_need = forward_workspace_bytes(plan, B, H, chunk_cap);
    if (ws_need) {
        if (!workspace || workspace_bytes < ws_need) return FFTCONV_ERR_WORKSPACE;
        if (!aligned16(workspace)) return FFTCONV_ERR_ALIGNMENT;
        if (overlap(workspace, ws_need, y, io_bytes) ||
            overlap(workspace, ws_need, u, io_bytes) ||
            overlap(workspace, ws_need, k_f, kf_bytes))
            return FFTCONV_ERR_INVALID_ARG;
        if (w && (overlap(workspace, ws_need, w, io_bytes) ||
                  overlap(workspace, ws_need, v, io_bytes)))
            return FFTCONV_ERR_INVALID_ARG;
    }
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return FFTCONV_ERR_HIP;
    if (dev != plan->device) return FFTCONV_ERR_INVALID_ARG;
    return FFTCONV_OK;
}

fftconv_status forward_impl(fftconv_plan_t plan, const void* u, const void* w,
                            const void* v, const void* k_f, void* y, size_t B,
                            size_t H, size_t N, void* workspace,
                            size_t workspace_bytes, void* stream, int skip_hi,
                            size_t chunk_cap, int outer_keep) {
    const fftconv_status chk =
        forward_check(plan, u, w, v, k_f, y, B, H, N, workspace, workspace_bytes, chunk_cap);
    if (chk != FFTCONV_OK) return chk;
    const Shape& s = plan->s;
    const size_t rows = B * H;
    if (rows == 0) return FFTCONV_OK;
    const size_t esz = s.dtype == FFTCONV_F32 ? 4 : 2;
    const size_t ws_need = forward_workspace_bytes(plan, B, H, chunk_cap);
    hipStream_t st = (hipStream_t)stream;
    const int io = (int)s.dtype;
    hipError_t e;
    if (plan->use_row) {
        RowParams R = plan->row;
        R.B = (int)B;
        R.H = (int)H;
        // one persistent workgroup per CU, each a contiguous channel-major
        // slice of rows; the slice's channels' spectra must fit the LDS
        const long long rows_all = (long long)B * (long long)H;
        long long G = plan->num_cu;
        long long per = (rows_all + G - 1) / G;
        const long long max_ch = plan->row_max_channels;
        while ((per + B - 1) / B + 1 > max_ch && per > 1) per = (per + 1) / 2;
        R.rows_per_wg = per;
        R.grid = (int)((rows_all + per - 1) / per);
        R.u = u;
        R.y = y;
        R.kf = k_f;
        R.w = w;
        R.v = v;
        R.skip_hi = skip_hi;
        e = launch_row(io, plan->row_nb, R, plan->lds_row, st);
    } else if (s.mp_P1) {
        const size_t hc_max = mp_chunk_channels(s, B, H, chunk_cap);
        const size_t bc_max = mp_chunk_batch(s, B, chunk_cap);
        MpColParams C1{};
        C1.H = (int)H;
        C1.M = (int)s.M;
        C1.S = (int)(s.M / s.mp_P1);
        C1.tw = plan->mp_tw1;
        C1.u = u;
        C1.y = y;
        C1.w = w;
        C1.v = v;
        C1.ws = workspace;
        C1.ctr = (uint32_t*)((char*)workspace + (ws_need - kClaimBytes));
        C1.full = s.full ? 1 : 0;
        MpInnerParams I = plan->mp;
        I.skip_hi = skip_hi;
        I.upr_active = outer_keep > 0 && outer_keep < I.Po / 2 ? outer_keep : I.Po / 2;
        I.B = (int)B;
        I.H = (int)H;
        I.ws = workspace;
        I.ctr = C1.ctr;
        I.kf = k_f;
        if ((long long)bc_max * (long long)hc_max * (I.Po / 2) > 0x7fffffffLL)
            return FFTCONV_ERR_UNSUPPORTED;
        e = hipSuccess;
        // chunks of bc_max batch rows x hc_max channels: the passes address
        // rows relative to the chunk's first batch row
        const size_t row_bytes = H * N * esz;
        for (size_t b0 = 0; b0 < B && e == hipSuccess; b0 += bc_max)
        for (size_t h0 = 0; h0 < H && e == hipSuccess; h0 += hc_max) {
            const size_t bcur = B - b0 < bc_max ? B - b0 : bc_max;
            const size_t hc = H - h0 < hc_max ? H - h0 : hc_max;
            C1.u = (const char*)u + b0 * row_bytes;
            C1.y = (char*)y + b0 * row_bytes;
            C1.w = w ? (const char*)w + b0 * row_bytes : nullptr;
            C1.v = v ? (const char*)v + b0 * row_bytes : nullptr;
            I.B = (int)bcur;
            C1.h0 = I.h0 = (int)h0;
            C1.hc = I.hc = (int)hc;
            C1.rows = (long long)bcur * (long long)hc;
            I.grid = mp_inner_grid(plan, C1.rows * I.upr_active);
            if (s.mp_P2 > 1) {
                // both outer levels in one pass each way
                const MpCol2Params D = mp_col2_params(plan, C1);
                if (plan->mp2m_a1) {
                    // P1 = P2 = 32: the forward pass on the matrix cores,
                    // one workgroup per CU
                    MpCol2Params F = D;
                    F.a1 = w ? plan->mp2m_a1h : plan->mp2m_a1;
                    F.a2 = plan->mp2m_a2;
                    F.tm = plan->mp2m_tm;
                    F.grid = (int)std::min<long long>(D.rows * 128, plan->num_cu);
                    e = launch_mp_col2m_fwd(io, F, st);
                } else {
                    e = launch_mp_col2(io, s.mp_P1, s.mp_P2, false, D, st);
                }
            } else {
                e = launch_mp_col(io, s.mp_P1, 0, C1, st);
            }
            if (e == hipSuccess) e = mp_inner_inverse(plan, io, I, C1, st);
        }
    } else if (s.wide_P) {
        WideParams W = plan->wide;
        W.B = (int)B;
        W.H = (int)H;
        // persistent workgroups striding over the channel-major rows; a
        // multiple of 8 so every XCD gets the same share
        const long long rows_all = (long long)B * (long long)H;
        long long G = (long long)plan->wide_wgs_per_cu * plan->num_cu;
        G = G < 8 ? 8 : G & ~7LL;
        const long long need = (rows_all + 7) & ~7LL;
        W.grid = (int)(G < need ? G : need);
        W.u = u;
        W.y = y;
        W.kf = k_f;
        W.w = w;
        W.v = v;
        W.skip_hi = skip_hi;
        W.pairs = outer_keep > 0 && outer_keep < s.wide_P / 2 ? outer_keep : s.wide_P / 2;
        // static row claims (no counters: measured as fast as claiming
        // from per-XCD counters at the workload sizes, and faster for small
        // calls, which no longer pay a counter-clearing launch)
        W.ctr = nullptr;
        e = launch_wide(io, s.wide_P, W, plan->lds_wide, st);
    } else if (s.path == 0) {
        FwdParams P = plan->fused;
        P.rows = (long long)rows;
        P.H = (int)H;
        P.u = u;
        P.y = y;
        P.kf = k_f;
        P.w = w;
        P.v = v;
        e = launch_fused(io, P, s.lds_fused, st);
    } else {
        FwdParams O = plan->outer, I = plan->inner;
        O.rows = I.rows = (long long)rows;
        O.H = I.H = (int)H;
        O.u = I.u = u;
        O.y = I.y = y;
        O.w = I.w = w;
        O.v = I.v = v;
        O.kf = I.kf = k_f;
        O.ws = I.ws = (float2*)workspace;
        e = launch_outer_fwd(io, O, s.lds_outer, st);
        if (e == hipSuccess) e = launch_inner(io, I, s.lds_inner, st);
        if (e == hipSuccess) e = launch_outer_inv(io, O, s.lds_outer, st);
    }
    return e == hipSuccess ? FFTCONV_OK : FFTCONV_ERR_HIP;
}

}  // namespace

extern "C" {

fftconv_status fftconv_forward(fftconv_plan_t plan, const void* u,
                               const void* k_f, void* y, size_t B, size_t H,
                               size_t N, void* workspace,
                               size_t workspace_bytes, void* stream) {
    return forward_impl(plan, u, nullptr, nullptr, k_f, y, B, H, N, workspace,
                        workspace_bytes, stream, 0, kMpChunkBytes);
}

fftconv_status fftconv_forward_noalloc(fftconv_plan_t plan, const void* u,
                                       const void* k_f, void* y, size_t B, size_t H,
                                       size_t N, void* stream) {
    if (!plan) return FFTCONV_ERR_INVALID_ARG;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return FFTCONV_ERR_HIP;
    if (dev != plan->device) return FFTCONV_ERR_INVALID_ARG;
    // the library's static scratch array on this device (its address is
    // looked up once per device)
    void* scratch = nullptr;
    size_t scratch_bytes = 0;
    if (scratch_buffer(dev, &scratch, &scratch_bytes) != hipSuccess) return FFTCONV_ERR_HIP;
    // multi-pass chunks sized to what the array holds beside the counters;
    // a single row must fit
    const size_t cap = scratch_bytes - kClaimBytes;
    if (plan->s.mp_P1 && plan->s.M * 4 > cap) return FFTCONV_ERR_WORKSPACE;
    if (B * H != 0 && forward_workspace_bytes(plan, B, H, cap) > scratch_bytes)
        return FFTCONV_ERR_WORKSPACE;
    return forward_impl(plan, u, nullptr, nullptr, k_f, y, B, H, N, scratch,
                        scratch_bytes, stream, 0, cap);
}

fftconv_status fftconv_forward_lowpass(fftconv_plan_t plan, const void* u,
                                       const void* k_f, size_t cutoff, void* y,
                                       size_t B, size_t H, size_t N, void* workspace,
                                       size_t workspace_bytes, void* stream) {
    if (!plan) return FFTCONV_ERR_INVALID_ARG;
    if (plan->s.full) return FFTCONV_ERR_UNSUPPORTED;
    if (cutoff > plan->s.N) return FFTCONV_ERR_INVALID_ARG;
    // the 32 x 32 engine (row kernel at N = 1024, wide kernel, multi-pass
    // inner pass) skips the tiles of k_b = 8..23: the top digit of the bin,
    // so those packed bins k lie in [M/4, 3M/4), all beyond a cutoff below
    // M/4
    const bool engine = (plan->use_row && plan->row_nb == 32) || plan->s.wide_P || plan->s.mp_P1;
    const int skip = (engine && cutoff < plan->s.M / 4) ? 1 : 0;
    return forward_impl(plan, u, nullptr, nullptr, k_f, y, B, H, N, workspace,
                        workspace_bytes, stream, skip, kMpChunkBytes);
}

// a and d of the digit-block pattern: a even in [0, 32]; d in [0, P) with P
// the plan's outer factor (d = 0 when P = 1)
bool blocksparse_args_ok(const fftconv_plan_s* plan, int a, int d) {
    const int P = sparse_outer(plan->s);
    return a >= 0 && a <= 32 && (a % 2) == 0 && d >= 0 && d < P;
}

fftconv_status fftconv_kernel_spectrum_blocksparse(fftconv_plan_t plan, const float* k,
                                                   size_t H, int a, int d, void* k_f,
                                                   void* stream) {
    if (!plan) return FFTCONV_ERR_INVALID_ARG;
    if (plan->s.full) return FFTCONV_ERR_UNSUPPORTED;
    if (!blocksparse_args_ok(plan, a, d)) return FFTCONV_ERR_INVALID_ARG;
    return spectrum_impl(plan, k, H, FFTCONV_CAUSAL, -1, k_f, stream, a, d);
}

fftconv_status fftconv_forward_blocksparse(fftconv_plan_t plan, const void* u,
                                           const void* k_f, int a, int d, void* y,
                                           size_t B, size_t H, size_t N, void* workspace,
                                           size_t workspace_bytes, void* stream) {
    if (!plan) return FFTCONV_ERR_INVALID_ARG;
    if (plan->s.full) return FFTCONV_ERR_UNSUPPORTED;
    if (!blocksparse_args_ok(plan, a, d)) return FFTCONV_ERR_INVALID_ARG;
    // the 32 x 32 engine skips the tiles of k_b = 8..23 (a >= 16 zeroes
    // them all); the wide and multi-pass kernels skip the mirror pairs of
    // outer classes j >= P/2 - d/2, whose bins are all zero
    const bool engine = (plan->use_row && plan->row_nb == 32) || plan->s.wide_P || plan->s.mp_P1;
    const int skip = (engine && a >= 16) ? 1 : 0;
    const int P = sparse_outer(plan->s);
    const int keep = P > 1 ? P / 2 - d / 2 : 0;
    return forward_impl(plan, u, nullptr, nullptr, k_f, y, B, H, N, workspace,
                        workspace_bytes, stream, skip, kMpChunkBytes, keep);
}

fftconv_status fftconv_forward_gated(fftconv_plan_t plan, const void* u,
                                     const void* w, const void* v,
                                     const void* k_f, void* y, size_t B,
                                     size_t H, size_t N, void* workspace,
                                     size_t workspace_bytes, void* stream) {
    if (B * H != 0 && (!w || !v)) return FFTCONV_ERR_INVALID_ARG;
    return forward_impl(plan, u, w, v, k_f, y, B, H, N, workspace,
                        workspace_bytes, stream, 0, kMpChunkBytes);
}

fftconv_status fftconv_backward(fftconv_plan_t plan, const void* u,
                                const void* dy, const void* k_f_adj, void* du,
                                float* dk, size_t B, size_t H, size_t N,
                                void* workspace, size_t workspace_bytes,
                                void* stream) {
    if (plan && plan->s.full) return FFTCONV_ERR_UNSUPPORTED;
    if (!plan || !plan->grad) return FFTCONV_ERR_INVALID_ARG;
    const Shape& s = plan->s;
    if (N != s.N) return FFTCONV_ERR_INVALID_ARG;
    if (!du && !dk) return FFTCONV_ERR_INVALID_ARG;
    const size_t rows = B * H;
    if (B != 0 && rows / B != H) return FFTCONV_ERR_INVALID_ARG;
    if (rows > 0x7fffffffULL || H > 0x7fffffffULL) return FFTCONV_ERR_UNSUPPORTED;
    const size_t esz = s.dtype == FFTCONV_F32 ? 4 : 2;
    const size_t io_bytes = rows * N * esz, dk_bytes = H * N * 4;
    if (dk) {
        if (!aligned16(dk)) return FFTCONV_ERR_ALIGNMENT;
        if (rows && (!u || !dy)) return FFTCONV_ERR_INVALID_ARG;
        if (rows && (!aligned16(u) || !aligned16(dy))) return FFTCONV_ERR_ALIGNMENT;
        if (overlap(dk, dk_bytes, u, io_bytes) || overlap(dk, dk_bytes, dy, io_bytes))
            return FFTCONV_ERR_INVALID_ARG;
        if (du && overlap(dk, dk_bytes, du, io_bytes)) return FFTCONV_ERR_INVALID_ARG;
        if (k_f_adj && overlap(dk, dk_bytes, k_f_adj, fftconv_spectrum_bytes(plan, H)))
            return FFTCONV_ERR_INVALID_ARG;
    }
    if (du && rows && u && overlap(du, io_bytes, u, io_bytes)) return FFTCONV_ERR_INVALID_ARG;
    const size_t ws_need = fftconv_backward_workspace_bytes(plan, B, H);
    if (rows && ws_need) {
        if (!workspace || workspace_bytes < ws_need) return FFTCONV_ERR_WORKSPACE;
        if (!aligned16(workspace)) return FFTCONV_ERR_ALIGNMENT;
        if ((u && overlap(workspace, ws_need, u, io_bytes)) ||
            (dy && overlap(workspace, ws_need, dy, io_bytes)) ||
            (du && overlap(workspace, ws_need, du, io_bytes)) ||
            (dk && overlap(workspace, ws_need, dk, dk_bytes)))
            return FFTCONV_ERR_INVALID_ARG;
    }
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return FFTCONV_ERR_HIP;
    if (dev != plan->device) return FFTCONV_ERR_INVALID_ARG;
    hipStream_t st = (hipStream_t)stream;
    // On the multi-pass engine both gradients start from the same forward
    // column pass of dy: dk's gradient pass only reads it, so du's inner and
    // inverse passes then run on that workspace in place of a second column
    // pass of dy of their own.
    const bool share_dy = du && dk && rows && !plan->kg && kgrad_on_mp(plan, B);
    // du = the adjoint operator applied to dy (the forward kernels with the
    // conjugate spectrum); validated like any forward call
    if (du) {
        const fftconv_status fs =
            share_dy ? forward_check(plan, dy, nullptr, nullptr, k_f_adj, du, B, H, N, workspace,
                                     workspace_bytes, kMpChunkBytes)
                     : forward_impl(plan, dy, nullptr, nullptr, k_f_adj, du, B, H, N, workspace,
                                    workspace_bytes, stream, 0, kMpChunkBytes);
        if (fs != FFTCONV_OK) return fs;
        if (share_dy && overlap(workspace, ws_need, k_f_adj, fftconv_spectrum_bytes(plan, H)))
            return FFTCONV_ERR_INVALID_ARG;
    }
    if (!dk || H == 0) return FFTCONV_OK;
    if (rows == 0) {
        // an empty batch contributes nothing: dk = 0
        return launch_scale_f32(dk, (long long)(H * N), 0.f, st) == hipSuccess
                   ? FFTCONV_OK : FFTCONV_ERR_HIP;
    }
    return backward_dk(plan->kg ? plan->kg : plan, u, dy, dk, B, H, N, workspace, st,
                       share_dy ? k_f_adj : nullptr, share_dy ? du : nullptr);
}

}  // extern "C"

namespace {

// dk of the causal convolution on the engine of `plan` (the caller's plan,
// or the one it delegates the kernel gradient to); arguments validated.
// With du set (multi-pass engine only), du = the adjoint spectrum k_f_adj
// applied to dy is computed from the same column pass of dy.
fftconv_status backward_dk(const fftconv_plan_s* plan, const void* u, const void* dy,
                           float* dk, size_t B, size_t H, size_t N, void* workspace,
                           hipStream_t st, const void* k_f_adj, void* du) {
    const Shape& s = plan->s;
    const size_t rows = B * H;
    const size_t esz = s.dtype == FFTCONV_F32 ? 4 : 2;
    const int io = (int)s.dtype;
    hipError_t e;
    if (kgrad_on_row(plan)) {
        KgRowParams R{};
        R.B = (int)B;
        R.H = (int)H;
        R.S = kgrad_row_slices(plan, B, H);
        R.u = u;
        R.dy = dy;
        R.part = (float*)workspace;
        R.dk = dk;
        R.f1b = plan->row.f1b;
        R.f2a = plan->row.f2a;
        R.i2b = plan->row.i2b;
        R.i1a = plan->row.i1a;
        R.twf = plan->row.twf;
        // accumulated 4 Z_g in unitary units: the inverse gets Z_g / sqrt(M),
        // the output takes back the factor M (see the generic path)
        R.pre = 0.25f / sqrtf((float)s.M);
        R.post = (float)s.M;
        e = launch_kgrad_row(io, R, st);
        return e == hipSuccess ? FFTCONV_OK : FFTCONV_ERR_HIP;
    }
    if (s.wide_P) {
        KgWideParams W{};
        W.B = (int)B;
        W.H = (int)H;
        W.S = kgrad_wide_slices(plan, B, H);
        W.u = u;
        W.dy = dy;
        W.part = (float*)workspace;
        W.dk = dk;
        W.f1b = plan->wide.f1b;
        W.f2a = plan->wide.f2a;
        W.i2b = plan->wide.i2b;
        W.i1a = plan->wide.i1a;
        W.twf = plan->wide.twf;
        W.two = plan->wide.two;
        W.pre = 0.25f / sqrtf((float)s.M);
        W.post = (float)s.M;
        e = launch_kgrad_wide(io, s.wide_P, W, st);
        return e == hipSuccess ? FFTCONV_OK : FFTCONV_ERR_HIP;
    }
    if (kgrad_on_mp(plan, B)) {
        const size_t bcm = kgrad_mp_batch(plan, B), hcm = kgrad_mp_channels(plan, B, H);
        const size_t per = bcm * hcm * s.M * 4;
        char* base = (char*)workspace;
        void* wsu = base;
        void* wsd = base + per;
        void* wsg = base + 2 * per;
        uint32_t* ctr = (uint32_t*)(base + 2 * per + hcm * s.M * 4);
        const MpInnerParams& T = plan->mp;
        const size_t row_bytes = H * N * esz;
        if (du && (long long)bcm * (long long)hcm * (T.Po / 2) > 0x7fffffffLL)
            return FFTCONV_ERR_UNSUPPORTED;
        e = hipSuccess;
        for (size_t h0 = 0; h0 < H && e == hipSuccess; h0 += hcm)
        for (size_t b0 = 0; b0 < B && e == hipSuccess; b0 += bcm) {
            const size_t hc = H - h0 < hcm ? H - h0 : hcm;
            const size_t bc = B - b0 < bcm ? B - b0 : bcm;
            const void* ub = (const char*)u + b0 * row_bytes;
            const void* dyb = (const char*)dy + b0 * row_bytes;
            e = mp_cols_fwd(plan, io, ub, wsu, ctr, bc, H, h0, hc, st);
            if (e == hipSuccess) e = mp_cols_fwd(plan, io, dyb, wsd, ctr, bc, H, h0, hc, st);
            if (e == hipSuccess) {
                KgMpParams P{};
                P.B = (int)bc;
                P.hc = (int)hc;
                P.M = (int)s.M;
                P.Po = T.Po;
                P.P1 = T.P1;
                P.P2 = T.P2;
                P.wsu = wsu;
                P.wsd = wsd;
                P.wsg = wsg;
                P.f1b = T.f1b;
                P.i1a = T.i1a;
                P.f2a = T.f2a;
                P.i2b = T.i2b;
                P.twf = T.twf;
                P.two = T.two;
                // accumulated 4 Z_g in unitary units (as the row engine)
                P.pre = 0.25f / sqrtf((float)s.M);
                e = launch_kgrad_mp(io, P, st);
            }
            if (e == hipSuccess && du) {
                // du: the forward call's inner and inverse passes on the
                // transformed dy rows, which the gradient pass left intact
                MpColParams C{};
                C.rows = (long long)bc * (long long)hc;
                C.H = (int)H;
                C.h0 = (int)h0;
                C.hc = (int)hc;
                C.M = (int)s.M;
                C.S = (int)(s.M / s.mp_P1);
                C.tw = plan->mp_tw1;
                C.y = (char*)du + b0 * row_bytes;
                C.ws = wsd;
                C.ctr = ctr;
                MpInnerParams I = T;
                I.skip_hi = 0;
                I.upr_active = I.Po / 2;
                I.B = (int)bc;
                I.H = (int)H;
                I.h0 = (int)h0;
                I.hc = (int)hc;
                I.ws = wsd;
                I.ctr = ctr;
                I.kf = k_f_adj;
                I.grid = mp_inner_grid(plan, C.rows * I.upr_active);
                e = mp_inner_inverse(plan, io, I, C, st);
            }
            if (e == hipSuccess) {
                // inverse column passes of the channels' result rows into
                // fp32 dk: the second level in place, then the first
                MpColParams C{};
                C.rows = (long long)hc;
                C.H = (int)H;
                C.h0 = (int)h0;
                C.hc = (int)hc;
                C.M = (int)s.M;
                C.ws = wsg;
                C.y = dk;
                C.ctr = ctr;
                C.post = (float)s.M;
                if (s.mp_P2 > 1) {
                    MpColParams C2 = C;
                    C2.S = 4096;
                    C2.tw = plan->mp_tw2;
                    e = launch_mp_col(io, s.mp_P2, 2, C2, st);
                }
                C.S = (int)(s.M / s.mp_P1);
                C.tw = plan->mp_tw1;
                if (e == hipSuccess) e = launch_mp_col(io, s.mp_P1, b0 == 0 ? 4 : 5, C, st);
            }
        }
        return e == hipSuccess ? FFTCONV_OK : FFTCONV_ERR_HIP;
    }
    const fftconv_plan_s* gp = plan->grad;
    const Shape& g = gp->s;
    KgradParams K{};
    K.B = (int)B;
    K.H = (int)H;
    K.scale = (float)g.M;
    K.u = u;
    K.dy = dy;
    K.dk = dk;
    const int lds = kgrad_lds(g);
    if (g.path == 0) {
        K.f = gp->fused;
        const int ns = kgrad_splits(plan, B, H);
        K.wsg = (float2*)workspace;
        e = launch_kgrad_fused(io, K, ns, lds, st);
        if (e == hipSuccess && ns > 1)
            e = launch_kgrad_reduce((const float*)workspace, dk, (long long)(H * N), ns, st);
    } else {
        float2* wsu = (float2*)workspace;
        float2* wsd = wsu + rows * g.M;
        float2* wsg = wsd + rows * g.M;
        FwdParams O = gp->outer;
        O.rows = (long long)rows;
        O.H = (int)H;
        O.u = u;
        O.ws = wsu;
        e = launch_outer_fwd(io, O, g.lds_outer, st);
        if (e == hipSuccess) {
            O.u = dy;
            O.ws = wsd;
            e = launch_outer_fwd(io, O, g.lds_outer, st);
        }
        if (e == hipSuccess) {
            K.f = gp->inner;
            K.wsu = wsu;
            K.wsd = wsd;
            K.wsg = wsg;
            e = launch_kgrad_inner(io, K, lds, st);
        }
        if (e == hipSuccess) {
            FwdParams OI = gp->outer;
            OI.rows = (long long)H;
            OI.H = (int)H;
            OI.ws = wsg;
            OI.y = dk;
            e = launch_outer_inv_f32out(io, OI, g.lds_outer, st);
        }
        if (e == hipSuccess) e = launch_scale_f32(dk, (long long)(H * N), (float)g.M, st);
    }
    return e == hipSuccess ? FFTCONV_OK : FFTCONV_ERR_HIP;
}

}  // namespace
