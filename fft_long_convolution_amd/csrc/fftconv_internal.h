// Internal declarations shared by the host planner (fftconv_host.cpp) and
// the gfx950 kernels (fftconv_kernels.hip).  Not part of the public ABI.
//
// Transform conventions (page "FlashFFTConv: Efficient Convolutions for
// Long Sequences with Tensor Cores", section 3.4):
//  * A row u[0:N] is packed into M = N complex points z[m] = u[2m] + i u[2m+1]
//    for m < N/2; z[m] = 0 for m >= N/2 is the causal zero padding, never
//    stored and never multiplied ("Implicit zero-padding").  Plans of the
//    circular operators at FFT size N ("full" plans) have M = N/2 and no
//    zero half: every packed point is loaded and every output stored.
//  * The M-point DFT is factored M = N_1 * ... * N_p (order-p Monarch).
//    Forward stage i (decimation in frequency, in place): within blocks of
//    S_i = N_i * ... * N_p points, each of the s_i = S_i / N_i columns gets an
//    N_i-point DFT over elements spaced s_i apart, followed by the twiddle
//    W_{S_i}^{k c} (k = output digit, c = column).  After stage p, position
//    pos = sum_i k_i s_i holds bin k = k_1 + N_1 k_2 + N_1 N_2 k_3 + ...
//  * Every stage DFT is scaled by 1/sqrt(N_i), so the whole transform is
//    unitary and fp16 operands cannot overflow.
//  * The inverse mirrors the stages (conjugate twiddle before each inverse
//    DFT), taking digit-reversed positions back to natural order.
//  * Between the transforms, bin k and its mirror bin (M - k) mod M are
//    combined as Z'[k] = alpha_k Z[k] + beta_k conj(Z[-k]); alpha/beta fold
//    the real-FFT unpack, the product with the kernel spectrum and the
//    repack of the one-stage decimation in time.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fftconv {

enum IoType : int { IO_F32 = 0, IO_F16 = 1, IO_BF16 = 2 };

constexpr int kMaxStages = 8;
constexpr int kWaveSize = 64;

// One regular (non-middle) Monarch stage, as seen by a kernel that keeps a
// "line" of complex points in LDS.  The line is made of outer units; each
// outer unit holds Cb consecutive batch columns (Cb = 1 unless several
// independent columns of a larger transform are processed together).
//   LDS index of (block b, digit d, column c, batch cb)
//        = ((b * Sb + d * sb + c) * Cb + cb)
//   twiddle index = d * tw_stride + c * tw_mul + tw_off + cb
struct StageDev {
    int n;          // radix N_i (8, 16 or 32)
    int Sb;         // block size in outer units
    int sb;         // stride between digits in outer units (= Sb / n)
    int Cb;         // batch columns per outer unit
    int ncols;      // number of n-point DFT columns on the line
    int tw_stride;  // s_i of the full transform
    int tw_mul;     // multiplier of c in the twiddle column
    int pad;
    const float2* tw;    // W_{S_i}^{k c}, S_i entries laid out [k][c], or null
    const void* mat_f;   // forward DFT matrix tiles (A operand, per lane)
    const void* mat_i;   // inverse DFT matrix tiles (A operand, per lane)
};

// The last (innermost) stage, fused with the bin pairing and the first
// inverse stage.
struct MidDev {
    int n;          // radix N_p (16 or 32)
    int Q;          // blocks per slab (slab length / n)
    int slab;       // slab length in points
    int pad;
    const int* digrev;   // block position of lower bin part q, [Q]
    const void* mat_f;   // forward matrix, rows permuted to pair bins in-lane
    const void* mat_i;   // inverse matrix, K ordered like the accumulators
};

struct FwdParams {
    // geometry
    int M;              // packed transform length (= N)
    int N;              // sequence length
    int nst;            // regular stages handled by this kernel
    int outer_half;     // stage 0 is the outermost stage with a zero half
                        // (0 on full plans: all of stage 0's inputs are
                        // loaded and all its outputs stored)
    StageDev st[kMaxStages];
    MidDev mid;
    // rows
    long long rows;     // B * H
    int H;
    int Qo;             // multi-pass: number of slabs (outer product)
    int ct;             // multi-pass outer passes: batch columns per tile
    int nunits;         // multi-pass inner pass: units per row
    int threads;        // threads per workgroup
    const int* digrev_o;   // multi-pass: slab index of outer bin part, [Qo]
    // data
    const void* u;
    void* y;
    const void* kf;     // alpha/beta, [H][M] entries
    float2* ws;         // multi-pass workspace, [rows][M]
    const void* w;      // input gate (layout of u) or null
    const void* v;      // output gate (layout of y) or null
};

// Kernel gradient of the causal convolution (LDS-staged kernels of a plan
// built for it): dk[h][j] = sum_b sum_{t>=j} dy[b,h,t] u[b,h,t-j].
struct KgradParams {
    FwdParams f;        // stages: the whole transform (fused) or the inner
                        // slabs (multi-pass: f.digrev_o, f.Qo, f.nunits)
    int B, H;
    float scale;        // sqrt(M): the unitary transforms' lost factor
    const void* u;      // [B][H][N], plan dtype (fused)
    const void* dy;
    float* dk;          // [H][N] fp32 (fused, one batch slice)
    const float2* wsu;  // multi-pass: outer-transformed rows [B*H][M]
    const float2* wsd;
    float2* wsg;        // multi-pass: per-channel result rows [H][M];
                        // fused with several slices: partial dk rows
};
// fused: grid H x nsplit batch slices; with nsplit > 1 the slices write
// partial rows to wsg ([nsplit][H][N] fp32) for launch_kgrad_reduce
hipError_t launch_kgrad_fused(int io, const KgradParams& p, int nsplit, int lds_bytes,
                              hipStream_t s);
hipError_t launch_kgrad_reduce(const float* part, float* dk, long long n, int nsplit,
                               hipStream_t s);
hipError_t launch_kgrad_inner(int io, const KgradParams& p, int lds_bytes,
                              hipStream_t s);
// outer inverse pass writing fp32 (the kernel gradient) whatever the plan's
// I/O type, and an in-place scale of n floats
hipError_t launch_outer_inv_f32out(int io, const FwdParams& p, int lds_bytes,
                                   hipStream_t s);
hipError_t launch_scale_f32(float* x, long long n, float a, hipStream_t s);
hipError_t launch_stream_copy(const void* src, void* dst, long long n16, int num_cu, hipStream_t s);

// Kernel gradient on the row engine (N = 1024, 16-bit I/O,
// fftconv_kgrad.hip): one wave per (channel, batch slice) accumulates the
// packed gradient spectrum over its rows into part ([S][H][64 lanes][32]
// fp32); one wave per channel sums the slices and inverts it into dk.
struct KgRowParams {
    int B, H, S;
    const void* u;
    const void* dy;
    float* part;
    float* dk;              // [H][1024] fp32
    const void* f1b;        // the row plan's tables
    const void* f2a;
    const void* i2b;
    const void* i1a;
    const uint32_t* twf;
    float pre, post;        // operand scale of the inverse, output scale
};
hipError_t launch_kgrad_row(int io, const KgRowParams& p, hipStream_t s);

// The same on the one-workgroup-per-row engine (N = P x 1024): a workgroup
// per (channel, batch slice); part is [S][H][P/2 waves][64 lanes][64] fp32.
struct KgWideParams {
    int B, H, S;
    const void* u;
    const void* dy;
    float* part;
    float* dk;              // [H][N] fp32
    const void* f1b;        // the wide plan's tables
    const void* f2a;
    const void* i2b;
    const void* i1a;
    const uint32_t* twf;
    const uint32_t* two;
    float pre, post;
};
hipError_t launch_kgrad_wide(int io, int P, const KgWideParams& p, hipStream_t s);

// Spectrum (alpha/beta) construction.
struct SpecParams {
    int M, N, L;
    int p;
    int factors[kMaxStages];
    int h0, hcount;     // channel chunk
    const float2* X;    // [hcount][L] fp32 spectra of the padded kernels
    void* kf;           // [H][M] alpha/beta
};

// Register-resident row kernel (N = 32 * NB, NB = 16 or 32, 16-bit I/O).
struct RowParams {
    int B, H, N;
    int skip_hi;             // band limit below M/4 (NB = 32): skip the
                             // matrix-core tiles of k_b = 8..23
    int full;                // FFT size 2M (circular operators): all 32 n_a
                             // in and out, rows of M 32-bit words
    long long rows_per_wg;   // contiguous slice of channel-major rows
    int grid;                // workgroups
    const void* u;
    void* y;
    const void* w;      // input gate (layout of u) or null
    const void* v;      // output gate (layout of y) or null
    const void* kf;     // alpha/beta, [H][M] (4 x f16 each)
    const void* f1b;    // first stage, B-operand tiles [n_a half][hi 4][lo 4][64]
    const void* f1h;    // first stage in f16 [n_a half][4][64] (gated rows)
    const void* i1a;    // last inverse stage, A-operand tiles [2 or 4][2][64]
    const void* f2a;    // inner forward stage, A-operand tiles
    const void* i2b;    // inner inverse stage, B-operand tiles
    const void* i2bs;   // the same with the band-limited K-step grouping
    const uint32_t* twf;  // per-lane forward twiddles (packed f16 re, im)
    const uint32_t* twi;  // per-lane inverse twiddles (packed f16 re, im)
};
hipError_t launch_row(int io, int nb, const RowParams& p, int lds_bytes,
                      hipStream_t s);
// Waves per row-kernel workgroup (one workgroup per CU); the LDS layout is
// sized for kRowWaves.
constexpr int kRowWaves = 16;
constexpr int kRowWavesGated = 12;

// Fused kernel for N = P * 1024 (P = 4, 8, 16, 16-bit I/O): one workgroup
// of P/2 wavefronts per row (fftconv_wide.hip).
// Row-claim counters of one call: 8 XCD groups, one 128-byte line each.
constexpr int kClaimWords = 256;
constexpr size_t kClaimBytes = kClaimWords * 4;

// The static scratch array of the allocation-free forward call
// (fftconv_scratch.hip): its device address on `device` (which must be the
// current device; looked up once per device) and its size in bytes.
hipError_t scratch_buffer(int device, void** ptr, size_t* bytes);

struct WideParams {
    int B, H, N;
    int grid;                // persistent workgroups, a multiple of 8
    uint32_t* ctr;           // claim counters, or null: static claims
    const void* u;
    void* y;
    const void* w;           // input gate (layout of u) or null
    const void* v;           // output gate (layout of y) or null
    const void* kf;          // coefficients, [H][P/2][2][2][4][64][2] (4 x f16)
    const void* f1b;         // 32-point stage over n_a, B tiles [ks 2][jt 4][64]
    const void* i1a;         // its inverse, A tiles [mt 4][ks 2][64]
    const void* f2a;         // 32-point stage over n_b, A tiles [mt 4][ks 2][64]
    const void* i2b;         // its inverse, B tiles [ks 2][jt 4][64]
    const void* i2bs;        // the same with the band-limited K-step grouping
    const uint32_t* twf;     // per-lane W_1024 twiddles (packed f16)
    const uint32_t* two;     // outer twiddles W_M^{n' k1}, [k1-1][thread][column]
    int skip_hi;             // band limit below M/4: skip the tiles of k_b = 8..23
    int pairs;               // mirror pairs of sub-rows computed (the rest
                             // hold only zeroed bins: their sub-rows are zero)
    int full;                // FFT size 2M (circular operators, P <= 16): all
                             // P sub-rows in and out, rows of M 32-bit words
};
hipError_t launch_wide(int io, int P, const WideParams& p, int lds_bytes,
                       hipStream_t s);

struct WideCoefParams {
    int M, L, P;
    int h0, hcount;
    const float2* X;         // [hcount][L] fp32 spectra of the padded kernels
    void* kf;
};
hipError_t launch_wide_coef(const WideCoefParams& p, hipStream_t s);

// Multi-pass path for N >= 32K, 16-bit I/O (fftconv_mp.hip): column passes
// over the outer factor P_o = P1 [* P2] and an inner pass over units of two
// 4096-point slabs; f16 complex workspace [rows][M].
struct MpColParams {
    long long rows;        // B * hc rows of the chunk: local row r -> channel
    int H, h0, hc;         //   h0 + r % hc of batch r / hc; workspace row r
    int M;
    int S;                 // columns per block (spacing of the P inputs)
    const float2* tw;      // W_{P S}^c, c < S
    const void* u;
    void* y;
    const void* w;         // input gate (layout of u) or null
    const void* v;         // output gate (layout of y) or null
    void* ws;
    uint32_t* ctr;         // first pass: clears the inner pass's counters
    float post;            // mode 4 (inverse, fp32 output): output scale
    int full;              // modes 0 and 3 at FFT size 2M: all P points of
                           // u / y, rows of M 32-bit words
};
// mode 0: forward first level from u; 1: forward second level (in place);
// 2: inverse second level (in place); 3: inverse first level into y (I/O
// type); 4: the same into fp32 rows y scaled by post; 5: added to them
hipError_t launch_mp_col(int io, int P, int mode, const MpColParams& p, hipStream_t s);

// Both outer levels of a two-level plan in one pass (tiles of 512 / P2
// columns with all P1 * P2 outer points; the level-1 results stay in LDS).
struct MpCol2Params {
    long long rows;        // B * hc rows of the chunk (as MpColParams)
    int H, h0, hc;
    int M;
    int grid;              // persistent workgroups (<= tiles)
    const float2* tw1;     // W_M^c, c < M / P1
    const float2* tw2;     // W_{M/P1}^c, c < 4096
    const void* u;
    void* y;
    const void* w;         // input gate (layout of u) or null
    const void* v;         // output gate (layout of y) or null
    void* ws;
    uint32_t* ctr;         // forward pass: clears the inner pass's counters
    int full;              // FFT size 2M: all P1 first-level points of u / y
    // matrix-core forward pass (P1 = P2 = 32)
    const uint4* a1;       // forward level-1 DFT A operands, [mt 4][hi/lo 2][64];
                           // inverse: level-1 inverse DFT, [mt 2][ks 2][hi/lo 2][64]
    const uint4* a2;       // level-2 (inverse) DFT A operands, [mt 4][ks 2][hi/lo 2][64]
    const float2* tm;      // [W_1024^{n2 k1} 1024][W_M^{32 i k1} 128 x 32][W_M^{c k1} 32 x 32]
                           // [W_M^{1024 i k2} 128 x 32][W_M^{32 c k2} 32 x 32]
};
long long mp_col2_tiles(int P2, long long rows);
// Forward two-level pass on the matrix cores for P1 = P2 = 32 (one
// workgroup of 512 threads per CU, 152 KB LDS).
constexpr int kCol2mLds = 128 * 1024 + 3 * 8 * 1024;
hipError_t launch_mp_col2m_fwd(int io, const MpCol2Params& p, hipStream_t s);
hipError_t launch_mp_col2m_inv(int io, const MpCol2Params& p, hipStream_t s);
hipError_t launch_mp_col2(int io, int P1, int P2, bool inv, const MpCol2Params& p, hipStream_t s);

struct MpInnerParams {
    int B, H, M;
    int h0, hc;            // channel chunk (workspace rows b * hc + h - h0)
    int Po, P1, P2;        // outer factor and its levels (P2 = 1: one level)
    int grid;              // persistent workgroups, a multiple of 8
    uint32_t* ctr;         // claim counters (end of the workspace)
    void* ws;
    const void* kf;        // coefficients, [H][P_o/2][4][2][2][4][64][2] (4 x f16)
    const void* f1b;
    const void* i1a;
    const void* f2a;
    const void* i2b;
    const void* i2bs;      // the same with the band-limited K-step grouping
    const uint32_t* twf;
    const uint32_t* two;   // W_4096^{n' m}, m = 0..4, [m][engine position of n'] (packed f16)
    int skip_hi;           // band limit below M/4: skip the tiles of k_b = 8..23
    int upr_active;        // units q < upr_active of a row are computed (the
                           // others hold only zeroed bins)
};
hipError_t launch_mp_inner(int io, const MpInnerParams& p, int lds_bytes, hipStream_t s);

// Kernel gradient on the multi-pass engine: one workgroup per (local
// channel, unit of two slabs); reads the outer-transformed rows of u and dy
// (workspace rows b * hc + hl) and writes the channel's packed gradient
// spectrum, inverse-transformed by the engine and the 4-point stage, to
// result row hl (the layout the inverse column passes read).
struct KgMpParams {
    int B, hc, M;
    int Po, P1, P2;
    const void* wsu;
    const void* wsd;
    void* wsg;
    const void* f1b;       // the multi-pass plan's engine tables
    const void* i1a;
    const void* f2a;
    const void* i2b;
    const uint32_t* twf;
    const uint32_t* two;
    float pre;             // scale of the accumulated 4 Z_g before the inverse
};
int kgrad_mp_lds();
hipError_t launch_kgrad_mp(int io, const KgMpParams& p, hipStream_t s);

struct MpCoefParams {
    int M, L, Po;
    int h0, hcount;
    const float2* X;       // [hcount][L] fp32 spectra of the padded kernels
    void* kf;
};
hipError_t launch_mp_coef(const MpCoefParams& p, hipStream_t s);

// Launchers (defined in fftconv_kernels.hip).  Return hipSuccess or the
// launch error.
hipError_t launch_fused(int io, const FwdParams& p, int lds_bytes,
                        hipStream_t s);
hipError_t launch_outer_fwd(int io, const FwdParams& p, int lds_bytes,
                            hipStream_t s);
hipError_t launch_inner(int io, const FwdParams& p, int lds_bytes,
                        hipStream_t s);
hipError_t launch_outer_inv(int io, const FwdParams& p, int lds_bytes,
                            hipStream_t s);
// X[h][0:L] = the L-periodic kernel of operator `kind` built from k[h][0:N]
// (L = 2N: every kind; L = N: the circular kinds at FFT size N)
hipError_t launch_kpad(const float* k, float2* X, int hcount, int N, int L, int kind,
                       hipStream_t s);
hipError_t launch_band_limit(float2* X, int hcount, int L, int F, hipStream_t s);
// Zero blocks along the transform's digits: frequencies f whose packed bin
// k = f mod M (or its mirror -k) has its top digit of 32 among the a
// middle values or its outer digit k mod P among the d classes nearest P/2.
hipError_t launch_block_mask(float2* X, int hcount, int L, int M, int P, int a, int d,
                             hipStream_t s);
// Zero the workspace slabs of the multi-pass units q in [q_from, Po/2)
// (slabs sigma(q) and sigma(Po - q) of every row).
hipError_t launch_mp_zero_units(void* ws, long long rows, int M, int Po, int P1, int P2,
                                int q_from, hipStream_t s);
hipError_t launch_stockham(const float2* in, float2* out, int hcount, int L,
                           int Ns, hipStream_t s);
hipError_t launch_alphabeta(int io, const SpecParams& p, hipStream_t s);

}  // namespace fftconv
