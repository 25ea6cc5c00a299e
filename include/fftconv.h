/*
 * fftconv.h -- C ABI of the MI355X (gfx950) causal FFT long-convolution
 * library (libfftconv.so).
 *
 * The operation (page "FlashFFTConv: Efficient Convolutions for Long
 * Sequences with Tensor Cores", section 3.4, convolution definition and the
 * convolution theorem with causal zero padding to 2N):
 *
 *     y[b,h,t] = sum_{s=0..t} u[b,h,s] * k[h,t-s],   t in [0, N)
 *
 * computed as the first N outputs of the 2N-point circular convolution of
 * the zero-padded sequences.  Internally the real 2N-point transforms are
 * packed into N-point complex ones (the one-stage decimation in time of
 * section 3.4, "The real-valued FFT optimization"), the zero half of the
 * padded input is never read or computed ("Implicit zero-padding for causal
 * convolutions"), and every DFT is an order-p Monarch factorisation
 * ("The Monarch FFT Decomposition"): small dense DFT-matrix products on the
 * matrix cores with twiddle multiplies between them.
 *
 * Conventions for every call:
 *  - All tensor pointers are DEVICE pointers (memory from hipMalloc or a
 *    torch CUDA tensor on the same device); sizes are element counts.
 *  - The caller owns u, k, k_f, y and the workspace.  A plan owns only its
 *    own device tables.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Launching calls are asynchronous on that stream; they never
 *    synchronise the host.  Faults inside kernels surface at the caller's
 *    next synchronisation.
 *  - Every argument is validated before anything is launched; on error the
 *    call returns a non-OK status, launches nothing and writes nothing.
 *    Nothing throws across this interface.
 *  - A plan is immutable after creation and may be used from several host
 *    threads and streams at once.
 */
#ifndef FFTCONV_H
#define FFTCONV_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fftconv_status {
    FFTCONV_OK = 0,
    FFTCONV_ERR_INVALID_ARG = 1,  /* null pointer, size mismatch, overlap   */
    FFTCONV_ERR_UNSUPPORTED = 2,  /* N, order or dtype not supported        */
    FFTCONV_ERR_ALIGNMENT = 3,    /* a tensor pointer is not 16-B aligned   */
    FFTCONV_ERR_WORKSPACE = 4,    /* workspace missing or too small         */
    FFTCONV_ERR_HIP = 5           /* the HIP runtime reported an error      */
} fftconv_status;

/* I/O element type of u and y.  k is always fp32. */
typedef enum fftconv_dtype {
    FFTCONV_F32 = 0,
    FFTCONV_F16 = 1,
    FFTCONV_BF16 = 2
} fftconv_dtype;

typedef struct fftconv_plan_s *fftconv_plan_t;

/* Description of what a plan does (filled without touching the device). */
typedef struct fftconv_plan_info {
    size_t N;                 /* sequence length                            */
    size_t M;                 /* packed complex transform length (N; N/2
                                 on a plan of fftconv_plan_circular)       */
    int order;                /* number of Monarch factors p                */
    int factors[8];           /* N_1 (outermost, sees the zero half) ...    */
    int path;                 /* 0 = fused (one launch per call),
                                 1 = multi-pass through the workspace       */
    int outer_factors;        /* multi-pass: factors done in the outer pass */
    fftconv_dtype dtype;
    size_t spectrum_bytes_per_channel;
    size_t workspace_bytes_per_row;
    double mfma_flops_per_row; /* algorithmic matrix-core flops per row     */
    int kernel_variant;       /* 0 = LDS-staged fused kernel,
                                 1 = register-resident row kernel (N = 32*16
                                     or 32*32, 16-bit I/O),
                                 2 = three-pass, LDS-staged (fp32 I/O),
                                 3 = one-workgroup-per-row kernel
                                     (N = P*1024, P = 4, 8, 16, 32, 16-bit
                                     I/O),
                                 4 = column passes + slab-pair inner pass
                                     (N >= 32K, 16-bit I/O)                */
    int sparse_outer;         /* outer factor P of the digit-block sparsity
                                 (fftconv_forward_blocksparse): P of the
                                 wide kernel, M/4096 on the multi-pass path,
                                 1 otherwise                                */
    int circular;             /* 1: a plan of fftconv_plan_circular (FFT
                                 size N, M = N/2, circular kinds only)     */
} fftconv_plan_info;

/* Predicted cost of one forward call (an MI355X analogue of the page's cost
 * model: "FlashFFTConv: Efficient Convolutions for Long Sequences with
 * Tensor Cores", section 3.4, "The GPU Cost Model for Order-p
 * Decompositions", Equation 2).  Each decomposition level's work is charged
 * to the unit that runs it: DFT-matrix products to the matrix cores
 * (2.5 PFLOP/s f16, 157.3 TFLOP/s fp32), butterfly stages, twiddles and the
 * spectrum pairing to the vector ALU (157.3 TFLOP/s packed f16, 78.6 fp32),
 * stage data and operand tables to LDS (128 B/clk per CU), the u, y and k_f
 * streams and any workspace round trips to HBM (5.2 TB/s, what a streaming
 * copy reaches).  Matrix, vector and LDS work share a wave's issue stream
 * and add up; HBM runs beside them:
 *     t_pred = max(t_hbm, t_mfma + t_valu + t_lds).
 * With p = 0 fftconv_plan picks the candidate (order and kernel family) of
 * lowest t_pred for N. */
typedef struct fftconv_estimate {
    int order;                /* p of the estimated plan                    */
    int factors[8];
    int path;                 /* as fftconv_plan_info                       */
    int kernel_variant;       /* as fftconv_plan_info                       */
    double hbm_bytes;         /* per call                                   */
    double mfma_flops;
    double valu_flops;
    double lds_bytes;
    double t_hbm, t_mfma, t_valu, t_lds, t_pred;   /* seconds per call      */
} fftconv_estimate;

/* Estimate the call over B x H rows of the plan (N, p, dtype) -- the plan
 * fftconv_plan builds (lds_staged = 0) or the same order on the LDS-staged
 * kernels (lds_staged = 1).  B = 0 gives the cost per H rows of a large
 * batch (the spectrum's one read amortised away), which is what the choice
 * for p = 0 compares.  No device access.  Errors as fftconv_plan_query;
 * out == NULL -> FFTCONV_ERR_INVALID_ARG. */
fftconv_status fftconv_plan_estimate(size_t N, int p, fftconv_dtype dtype, int lds_staged,
                                     size_t B, size_t H, fftconv_estimate *out);

/* Create a plan for length N, Monarch order p and I/O dtype.
 *  N: a power of two in [256, 4194304] (section 3.4 discusses lengths up to
 *     4M; section 4.2's tables span 256..4M).
 *  p: 0 picks the factorisation of lowest predicted time for N
 *     (fftconv_plan_estimate); p >= 2 requests exactly p
 *     factors and returns FFTCONV_ERR_UNSUPPORTED when N cannot be split
 *     that way.  For the LDS-staged kernels the factors are 8, 16 or 32 (the
 *     last one 16 or 32); 16-bit plans at N = 4K..32K use P x 32 x 32
 *     (P = N/1024, p = 3, fused) and at N >= 32K also the outer levels
 *     followed by 4 x 32 x 32 (multi-pass), whose order is fixed by N.
 * Builds the DFT matrices and twiddle tables in fp64 on the host, rounds
 * them to the kernel's operand types and uploads them synchronously.
 * On success *out receives the plan; on failure *out is set to NULL. */
fftconv_status fftconv_plan(size_t N, int p, fftconv_dtype dtype,
                            fftconv_plan_t *out);

/* Plan for the circular (non-causal) operators at FFT size N (page
 * "FlashFFTConv: Efficient Convolutions for Long Sequences with Tensor
 * Cores", section 5, "Convolution Micro-Benchmarks": the standard
 * convolutions of its Tables 3 and 4 transform the input at its own length
 * N, while the causal ones of Tables 13 and 14 pad it to twice that; the
 * real-valued FFT of section 3.4, "Domain-Specific Optimizations", packs the
 * N real points into M = N/2 complex ones).  The forward kernels of such a
 * plan load and store every packed point (none is padding) and run the
 * M-point transform: half the transform length of the 2N-point route that
 * fftconv_plan takes for the same kinds.
 *  N: a power of two in [512, 4194304]; M = N/2 picks the kernel family
 *     and factorisation exactly as fftconv_plan does for a transform of M
 *     points (p = 0: the family's own factors; p >= 2: exactly p factors
 *     of M, as there).
 * On such a plan fftconv_kernel_spectrum_kind accepts FFTCONV_CIRCULAR and
 * FFTCONV_CIRCULAR_ADJOINT (the causal kinds, fftconv_kernel_spectrum, the
 * band-limited and digit-block calls return FFTCONV_ERR_UNSUPPORTED);
 * fftconv_forward, fftconv_forward_noalloc and fftconv_forward_gated work
 * as on any plan; fftconv_backward returns FFTCONV_ERR_UNSUPPORTED (the
 * input gradient of a circular convolution is fftconv_forward with the
 * FFTCONV_CIRCULAR_ADJOINT spectrum; no kernel gradient is provided).
 * Errors and ownership as fftconv_plan. */
fftconv_status fftconv_plan_circular(size_t N, int p, fftconv_dtype dtype,
                                     fftconv_plan_t *out);

/* Describe the plan fftconv_plan_circular(N, p, dtype) would build,
 * without touching the device. */
fftconv_status fftconv_plan_circular_query(size_t N, int p, fftconv_dtype dtype,
                                           fftconv_plan_info *info);

/* Describe the plan fftconv_plan(N, p, dtype) would build, without
 * allocating anything on the device. */
fftconv_status fftconv_plan_query(size_t N, int p, fftconv_dtype dtype,
                                  fftconv_plan_info *info);

/* Describe an existing plan. */
fftconv_status fftconv_plan_get_info(fftconv_plan_t plan,
                                     fftconv_plan_info *info);

/* Free a plan's device tables.  NULL is accepted. */
void fftconv_plan_destroy(fftconv_plan_t plan);

/* Bytes of the k_f buffer for H channels (caller allocates). */
size_t fftconv_spectrum_bytes(fftconv_plan_t plan, size_t H);

/* Bytes of the workspace fftconv_forward needs for B x H rows; the caller
 * allocates it.  0 for the fused kernels (row, one-workgroup-per-row and
 * LDS-staged); for the 16-bit multi-pass
 * path one channel chunk of f16 complex rows (at most 1 GB unless a single
 * channel is larger) plus the counters; B*H rows of fp32 complex for the
 * fp32 multi-pass path.  A call owns its workspace until it completes: two
 * calls in flight at once need two workspaces. */
size_t fftconv_workspace_bytes(fftconv_plan_t plan, size_t B, size_t H);

/* Kernel spectrum, computed once per channel and reused for every batch
 * row (section 2, Equation 1: "Fk is often precomputed").
 *  k:   device, fp32, [H][N] contiguous (the causal kernel taps k[h, t]).
 *  k_f: device, fftconv_spectrum_bytes(plan, H) bytes, 16-B aligned.  Its
 *       layout is private to plans with the same N, factorisation and
 *       dtype: it holds, per packed frequency bin, the two coefficients
 *       that combine the bin and its mirror bin with the kernel's
 *       spectrum (the real-FFT unpack, pointwise product and repack folded
 *       together), stored in the order the kernels visit the bins.
 * Asynchronous on `stream`; it allocates a temporary fp32 transform
 * buffer with stream-ordered allocation (hipMallocAsync). */
fftconv_status fftconv_kernel_spectrum(fftconv_plan_t plan, const float *k,
                                       size_t H, void *k_f, void *stream);

/* Which operator a spectrum makes fftconv_forward (and the gated call)
 * compute, for kernel taps k[h, 0:N] (page "FlashFFTConv: Efficient
 * Convolutions for Long Sequences with Tensor Cores": the convolution
 * definition and theorem of section 3.4, "The FFT Convolution and Its
 * Hardware Mismatch"; the non-causal convolutions of its
 * benchmark tables use an FFT of size N, i.e. a circular convolution; the
 * gradients multiply by the conjugate spectrum):
 *   FFTCONV_CAUSAL            y[t] = sum_{s<=t} u[s] k[t-s]
 *   FFTCONV_CAUSAL_ADJOINT    y[s] = sum_{t>=s} u[t] k[t-s]
 *                             (the transpose: du from dy)
 *   FFTCONV_CIRCULAR          y[t] = sum_s u[s] k[(t-s) mod N]
 *   FFTCONV_CIRCULAR_ADJOINT  y[s] = sum_t u[t] k[(t-s) mod N]
 * On a plan of fftconv_plan every kind runs the same kernels at the same
 * cost: each is the first N outputs of a 2N-point circular convolution of
 * the zero-padded input with a 2N-periodic kernel built from k (k followed
 * by zeros; k[0] and the reversed taps; k twice; k reversed twice).  A plan
 * of fftconv_plan_circular computes the two circular kinds at FFT size N
 * (the N-periodic kernel k, or k reversed). */
typedef enum fftconv_kernel_kind {
    FFTCONV_CAUSAL = 0,
    FFTCONV_CAUSAL_ADJOINT = 1,
    FFTCONV_CIRCULAR = 2,
    FFTCONV_CIRCULAR_ADJOINT = 3
} fftconv_kernel_kind;

/* fftconv_kernel_spectrum for the operator `kind` (FFTCONV_CAUSAL gives
 * exactly fftconv_kernel_spectrum).  Arguments, layout and errors as
 * there; an unknown kind -> FFTCONV_ERR_INVALID_ARG. */
fftconv_status fftconv_kernel_spectrum_kind(fftconv_plan_t plan, const float *k,
                                            size_t H, fftconv_kernel_kind kind,
                                            void *k_f, void *stream);

/* Frequency-sparse (band-limited) kernel spectrum (page "FlashFFTConv:
 * Efficient Convolutions for Long Sequences with Tensor Cores", section 3:
 * zeroing part of the frequency-domain kernel, the convolutional analogue
 * of low-pass filtering, lets the kernels skip the matrix-product blocks
 * whose bins are all zero).  The causal kernel's 2N-point spectrum is kept
 * at frequencies f with min(f, 2N - f) <= cutoff and zeroed elsewhere
 * (sparsity 1 - (2 cutoff + 1) / 2N for cutoff < N; cutoff = N keeps
 * everything).  cutoff > N -> FFTCONV_ERR_INVALID_ARG; otherwise as
 * fftconv_kernel_spectrum. */
fftconv_status fftconv_kernel_spectrum_lowpass(fftconv_plan_t plan, const float *k,
                                               size_t H, size_t cutoff, void *k_f,
                                               void *stream);

/* Causal long convolution y = (u * k)[0:N] for all B x H rows.
 *  u: device, plan dtype, [B][H][N] contiguous, 16-B aligned.
 *  k_f: device, from fftconv_kernel_spectrum with the same plan and H.
 *  y: device, plan dtype, [B][H][N], 16-B aligned; must not overlap u or
 *     k_f (checked: FFTCONV_ERR_INVALID_ARG).
 *  N: must equal the plan's N.
 *  workspace, workspace_bytes: device scratch of at least
 *     fftconv_workspace_bytes(plan, B, H) bytes, 16-B aligned (may be NULL
 *     with size 0 when that is 0); too small -> FFTCONV_ERR_WORKSPACE.
 * Asynchronous on `stream`, no host synchronisation.  B*H == 0 is a valid
 * no-op.  The calling thread's current HIP device must be the plan's. */
fftconv_status fftconv_forward(fftconv_plan_t plan, const void *u,
                               const void *k_f, void *y, size_t B, size_t H,
                               size_t N, void *workspace,
                               size_t workspace_bytes, void *stream);

/* fftconv_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The workspace is a static
 * device array of the library (64 MiB; each GPU the library runs on holds
 * its own copy from the first call on it until the process ends); the call
 * itself allocates nothing.  The multi-pass path (16-bit I/O, N >= 32K) runs
 * its channel chunks sized to that array, so any B and H fit; an fp32 plan
 * at N >= 32K needs B*H*N*8 bytes in one piece, and a call needing more
 * than the array holds returns FFTCONV_ERR_WORKSPACE before launching
 * anything.  Every call on one GPU uses the same array and leaves its
 * contents behind (the counters that must start at zero are cleared by each
 * call's own kernels): calls that overlap in time on one GPU (on different
 * streams or host threads) race and must not be issued.  Arguments,
 * results and the other errors as fftconv_forward. */
fftconv_status fftconv_forward_noalloc(fftconv_plan_t plan, const void *u,
                                       const void *k_f, void *y, size_t B, size_t H,
                                       size_t N, void *stream);

/* fftconv_forward for a spectrum from fftconv_kernel_spectrum_lowpass with
 * the same cutoff: the frequency-sparse convolution.  Kernels may skip the
 * blocks whose bins the cutoff zeroes: with 16-bit data at N = 1024 and at
 * N >= 4096, the 32 x 32 matrix-core stage (the whole transform at 1024,
 * the innermost one at larger N) skips half of its second forward product,
 * of its pairing work and of its first inverse product when cutoff < N/4;
 * other kernels, and larger cutoffs, compute the zero bins.  A spectrum built with
 * a larger cutoff (or none) is not valid here.  Arguments and errors as
 * fftconv_forward; cutoff > N -> FFTCONV_ERR_INVALID_ARG. */
fftconv_status fftconv_forward_lowpass(fftconv_plan_t plan, const void *u,
                                       const void *k_f, size_t cutoff, void *y,
                                       size_t B, size_t H, size_t N, void *workspace,
                                       size_t workspace_bytes, void *stream);

/* Frequency-sparse convolution with zero blocks along the transform's
 * digits (page "FlashFFTConv: Efficient Convolutions for Long Sequences
 * with Tensor Cores", section 3.4, "Frequency-sparse convolutions": the
 * kernel spectrum reshaped along the decomposition's factors with whole
 * rows zeroed along each, so that whole blocks of the transform can be
 * skipped).  The 2N-point spectrum is used through N packed bins (f and
 * f + N share bin f mod N); a bin k = k_out + P k_in (P = the plan's
 * sparse_outer, k_out < P) is zeroed when
 *   - its top digit of 32, floor(32 k_in P / N), is one of the a middle
 *     values 16 - a/2 .. 15 + a/2 (a even, 0..32), or
 *   - its outer digit k_out is one of the d classes nearest P/2
 *     (0 < |k_out - P/2| <= d/2, and P/2 itself when d is odd; d < P),
 * or when its mirror bin -k mod N is (so the output stays real).  The
 * sparsity is about 1 - (32 - a)(P - d) / (32 P).
 * fftconv_kernel_spectrum_blocksparse builds that spectrum (arguments as
 * fftconv_kernel_spectrum); fftconv_forward_blocksparse convolves with it
 * (arguments as fftconv_forward, a and d as given to the spectrum), skipping
 * the work of zero blocks: the matrix-core tiles of the top digit's middle
 * 16 values when a >= 16 (1024-point row kernel, wide and multi-pass
 * engines), and the whole engine passes of the outer classes' mirror pairs
 * (wide kernel: pairs of sub-rows; multi-pass: units of two slabs).  Bad a
 * or d -> FFTCONV_ERR_INVALID_ARG. */
fftconv_status fftconv_kernel_spectrum_blocksparse(fftconv_plan_t plan, const float *k,
                                                   size_t H, int a, int d, void *k_f,
                                                   void *stream);
fftconv_status fftconv_forward_blocksparse(fftconv_plan_t plan, const void *u,
                                           const void *k_f, int a, int d, void *y,
                                           size_t B, size_t H, size_t N, void *workspace,
                                           size_t workspace_bytes, void *stream);

/* Gated causal long convolution, y = v (.) ((u (.) w) * k)[0:N], for all
 * B x H rows: the input gate w multiplies u element-wise before the
 * convolution and the output gate v multiplies its result (page
 * "FlashFFTConv: Efficient Convolutions for Long Sequences with Tensor
 * Cores", section 3, "Domain-Specific Optimizations": the gating of
 * H3/Hyena-style layers fused into the convolution kernel, so neither
 * u (.) w nor the ungated result makes a round trip through HBM).
 *  u, w, v: device, plan dtype, [B][H][N] contiguous, 16-B aligned; both
 *     gates are required (a tensor of ones stands for an absent gate).
 *  y: as in fftconv_forward; must not overlap u, w, v or k_f (checked:
 *     FFTCONV_ERR_INVALID_ARG).  w and v may alias u or each other.
 *  All other arguments, the workspace and the error behaviour are those of
 *  fftconv_forward.  Products are formed in fp32 (exact for 16-bit
 *  inputs); with 16-bit I/O the gated input enters the first transform
 *  stage as f16, and the output gate multiplies the fp32 result before the
 *  one rounding to the I/O type (f16 rows of N = 4K..32K multiply in
 *  packed f16, as that stage computes). */
fftconv_status fftconv_forward_gated(fftconv_plan_t plan, const void *u,
                                     const void *w, const void *v,
                                     const void *k_f, void *y, size_t B,
                                     size_t H, size_t N, void *workspace,
                                     size_t workspace_bytes, void *stream);

/* Bytes of the workspace fftconv_backward needs for B x H rows: the larger
 * of the forward call's and the kernel gradient's.  The gradient needs
 * per-slice partial spectra on the row and wide engines (N = 1K..16K,
 * 16-bit I/O), for N >= 32K with 16-bit I/O the outer-transformed rows of
 * u and dy of one chunk of channels x batch rows plus one result row per
 * channel (f16 complex, at most 1 GB per buffer), and for fp32 plans two
 * B*H x N and one H x N fp32 complex rows (0 when fused). */
size_t fftconv_backward_workspace_bytes(fftconv_plan_t plan, size_t B, size_t H);

/* Backward pass of the causal convolution y = (u * k)[0:N] (page
 * "FlashFFTConv: Efficient Convolutions for Long Sequences with Tensor
 * Cores", section 3: the gradients of an FFT convolution are products with
 * conjugate spectra, and the spectra of the inputs are recomputed rather
 * than kept from the forward pass):
 *   du[b,h,s] = sum_{t>=s} dy[b,h,t] k[h,t-s]
 *   dk[h,j]   = sum_b sum_{t>=j} dy[b,h,t] u[b,h,t-j]
 *  u, dy: device, plan dtype, [B][H][N], 16-B aligned (u only needed for dk).
 *  k_f_adj: from fftconv_kernel_spectrum_kind(..., FFTCONV_CAUSAL_ADJOINT)
 *     of the same plan and k (only needed for du).
 *  du: device, plan dtype, [B][H][N], or NULL to skip the input gradient.
 *  dk: device, fp32, [H][N], 16-B aligned, overwritten (not accumulated),
 *     or NULL to skip the kernel gradient; not both NULL.
 *  workspace: fftconv_backward_workspace_bytes(plan, B, H) bytes.
 * du runs the forward kernels on dy with the adjoint spectrum (the same
 * cost as a forward call); dk recomputes the spectra of u and dy,
 * accumulates conj(U) DY over the batch per channel in fp32 registers and
 * runs one inverse transform per channel: on the matrix-core engine of the
 * forward kernels for 16-bit I/O (the row kernel's at N = 1024, the wide
 * kernel's at 4K..16K, the multi-pass column and inner passes at N >= 32K
 * -- at 32K the forward call is the fused wide kernel and dk still runs on
 * the multi-pass engine --
 * batch chunks adding their share to dk), on the LDS-staged kernels for
 * fp32 plans.  When both gradients are requested on the multi-pass engine,
 * du's inner and inverse passes start from dk's forward column pass of dy
 * (one column pass fewer; the same bits as two separate calls), and
 * k_f_adj must not overlap any part of the workspace.  B = 0 gives dk = 0.
 * The input
 * gradient of the other kinds is fftconv_forward with the matching adjoint
 * spectrum.  Errors as fftconv_forward. */
fftconv_status fftconv_backward(fftconv_plan_t plan, const void *u,
                                const void *dy, const void *k_f_adj, void *du,
                                float *dk, size_t B, size_t H, size_t N,
                                void *workspace, size_t workspace_bytes,
                                void *stream);

/* Static, human-readable text for a status code. */
const char *fftconv_status_string(fftconv_status status);

/* Version string of the library build. */
const char *fftconv_version(void);

/* Measurement aid, not part of the convolution: copies `bytes` (a multiple
 * of 16; src and dst device pointers, 16-B aligned, not overlapping) with
 * 16-byte non-temporal loads and stores on the current device, the access
 * pattern the convolution kernels stream their rows with.  Its rate is the
 * practical HBM roof of the part, and its byte counters calibrate the
 * kernels' (bench.py --copy-calibration).  Asynchronous on `stream`.
 * Errors: null or misaligned pointers, a size not a multiple of 16, or
 * overlap -> FFTCONV_ERR_INVALID_ARG / FFTCONV_ERR_ALIGNMENT. */
fftconv_status fftconv_stream_copy(const void *src, void *dst, size_t bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FFTCONV_H */
