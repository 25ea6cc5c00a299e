/*
 * oracle.c -- plain fp64 CPU reference for the causal long convolution.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or constant with
 * the GPU library.
 *
 * What it computes (page "FlashFFTConv: Efficient Convolutions for Long
 * Sequences with Tensor Cores", section 3.4, "The FFT Convolution and Its
 * Hardware Mismatch"):
 *
 *   convolution definition:  (u * k)[i] = sum_j u[j] k[i - j]
 *   causal form used here:   y[b,h,t] = sum_{s=0..t} u[b,h,s] k[h,t-s],
 *                            t in [0, N)   (kernel as long as the input)
 *
 * and, as an independent second route, the convolution theorem of the same
 * section (u * k = F^-1(Fu . Fk)) with both sequences zero-padded to 2N so
 * the circular result has no wrap-around, truncated back to N.  The FFT is
 * the textbook iterative radix-2 Cooley-Tukey transform (bit reversal, then
 * log2(L) butterfly stages).  Twiddles are taken from libm cos/sin of
 * 2*pi*j/len for every index (no recurrence).  There is no real-to-complex
 * packing and no matrix (Monarch) factoring here: this file deliberately
 * computes the plain definitions so it can be checked by eye.
 *
 * Further operators of the same family (same page, section 3: the
 * non-causal convolutions of its benchmark tables use an FFT of size N, a
 * circular convolution; training needs the gradients of the causal one,
 * which section 3.4, "Recomputation in the backward pass", writes as
 * products with the conjugate spectra):
 *
 *   kind 0  causal             y[t] = sum_{s<=t} u[s] k[t-s]
 *   kind 1  causal adjoint     y[s] = sum_{t>=s} u[t] k[t-s]
 *                              (the transpose of kind 0: du from dy)
 *   kind 2  circular           y[t] = sum_s u[s] k[(t-s) mod N]
 *   kind 3  circular adjoint   y[s] = sum_t u[t] k[(t-s) mod N]
 *
 *   kernel gradient  dk[h][j] = sum_{rows r of channel h} sum_t
 *                               dy[r][t] u[r][t-j]   (t-j taken mod N for
 *                               the circular kinds, t-j >= 0 otherwise)
 *
 * each by its definition and, independently, through the convolution
 * theorem (2N zero padding for the causal kinds, size N for the circular
 * ones; the adjoints multiply by the conjugate spectrum).
 *
 * Frequency-sparse (low-pass) convolution (same page, section 3:
 * zeroing part of the kernel spectrum, a band limit that discards the high
 * frequencies): the causal route above with the 2N-point kernel spectrum
 * set to zero at every frequency f whose distance min(f, 2N - f) from
 * zero exceeds the cutoff F.
 *
 * All arithmetic is fp64.  Rows are independent; OpenMP splits them.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef M_PI
#define M_PI 3.14159265358979323846
#endif

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Direct causal convolution by the definition.  u and y are [R][N];
 * kern is [Hk][N]; row r uses kernel row hidx[r].  O(N^2) per row. */
void oracle_conv_direct(const double *u, const double *kern, const long *hidx,
                        double *y, long R, long N)
{
    long r;
#pragma omp parallel for schedule(dynamic, 1)
    for (r = 0; r < R; ++r) {
        const double *ur = u + r * N;
        const double *kr = kern + hidx[r] * N;
        double *yr = y + r * N;
        for (long t = 0; t < N; ++t) {
            double acc = 0.0;
            for (long s = 0; s <= t; ++s)
                acc += ur[s] * kr[t - s];
            yr[t] = acc;
        }
    }
}

/* Selected outputs by the definition: out[i] = y[rows[i], ts[i]]. */
void oracle_conv_points(const double *u, const double *kern, const long *hidx,
                        long N, const long *rows, const long *ts, long count,
                        double *out)
{
    long i;
#pragma omp parallel for schedule(dynamic, 16)
    for (i = 0; i < count; ++i) {
        const double *ur = u + rows[i] * N;
        const double *kr = kern + hidx[rows[i]] * N;
        long t = ts[i];
        double acc = 0.0;
        for (long s = 0; s <= t; ++s)
            acc += ur[s] * kr[t - s];
        out[i] = acc;
    }
}

/* In-place iterative radix-2 DFT of length n (a power of two).
 * sign = -1: X[k] = sum_j x[j] exp(-2 pi i jk/n)   (forward, unnormalised)
 * sign = +1: x[j] = sum_k X[k] exp(+2 pi i jk/n)   (no 1/n here)          */
static void fft_radix2(double *re, double *im, long n, int sign)
{
    /* bit-reversal permutation */
    long j = 0;
    for (long i = 1; i < n; ++i) {
        long bit = n >> 1;
        while (j & bit) {
            j ^= bit;
            bit >>= 1;
        }
        j ^= bit;
        if (i < j) {
            double t = re[i]; re[i] = re[j]; re[j] = t;
            t = im[i]; im[i] = im[j]; im[j] = t;
        }
    }
    /* butterfly stages */
    for (long len = 2; len <= n; len <<= 1) {
        long half = len >> 1;
        for (long q = 0; q < half; ++q) {
            double ang = sign * 2.0 * M_PI * (double)q / (double)len;
            double wr = cos(ang), wi = sin(ang);
            for (long b = 0; b < n; b += len) {
                long p0 = b + q, p1 = b + q + half;
                double xr = re[p1] * wr - im[p1] * wi;
                double xi = re[p1] * wi + im[p1] * wr;
                re[p1] = re[p0] - xr;
                im[p1] = im[p0] - xi;
                re[p0] += xr;
                im[p0] += xi;
            }
        }
    }
}

/* Exposed for the oracle's own pins.  inverse != 0 applies sign +1 and
 * the 1/n normalisation, so oracle_fft(oracle_fft(x), inverse) == x. */
void oracle_fft(double *re, double *im, long n, int inverse)
{
    fft_radix2(re, im, n, inverse ? +1 : -1);
    if (inverse) {
        double s = 1.0 / (double)n;
        for (long i = 0; i < n; ++i) {
            re[i] *= s;
            im[i] *= s;
        }
    }
}

/* Spectrum of the zero-padded kernel rows: kre/kim are [Hk][2N]. */
void oracle_kernel_spectrum(const double *kern, long Hk, long N,
                            double *kre, double *kim)
{
    long L = 2 * N, h;
#pragma omp parallel for schedule(dynamic, 1)
    for (h = 0; h < Hk; ++h) {
        double *re = kre + h * L, *im = kim + h * L;
        for (long t = 0; t < L; ++t) {
            re[t] = t < N ? kern[h * N + t] : 0.0;
            im[t] = 0.0;
        }
        fft_radix2(re, im, L, -1);
    }
}

/* Causal convolution through the convolution theorem with 2N zero padding:
 *   U = FFT_2N(pad(u)),  K = FFT_2N(pad(k)),  y = IFFT_2N(U.K)[0:N] (real).
 * u, y: [R][N]; kern: [Hk][N]; row r uses kernel row hidx[r].
 * The kernel spectra are computed once per call (Hk of them). */
int oracle_conv_fft(const double *u, const double *kern, const long *hidx,
                    double *y, long R, long Hk, long N)
{
    long L = 2 * N;
    double *kre = (double *)malloc(sizeof(double) * (size_t)(Hk * L));
    double *kim = (double *)malloc(sizeof(double) * (size_t)(Hk * L));
    if (!kre || !kim) {
        free(kre);
        free(kim);
        return -1;
    }
    oracle_kernel_spectrum(kern, Hk, N, kre, kim);
    int fail = 0;
#pragma omp parallel
    {
        double *re = (double *)malloc(sizeof(double) * (size_t)L);
        double *im = (double *)malloc(sizeof(double) * (size_t)L);
        if (!re || !im) {
#pragma omp atomic write
            fail = 1;
        } else {
            long r;
#pragma omp for schedule(dynamic, 1)
            for (r = 0; r < R; ++r) {
                const double *ur = u + r * N;
                const double *Kr = kre + hidx[r] * L, *Ki = kim + hidx[r] * L;
                for (long t = 0; t < L; ++t) {
                    re[t] = t < N ? ur[t] : 0.0;
                    im[t] = 0.0;
                }
                fft_radix2(re, im, L, -1);
                for (long f = 0; f < L; ++f) {
                    double a = re[f], b = im[f];
                    re[f] = a * Kr[f] - b * Ki[f];
                    im[f] = a * Ki[f] + b * Kr[f];
                }
                fft_radix2(re, im, L, +1);
                double s = 1.0 / (double)L;
                double *yr = y + r * N;
                for (long t = 0; t < N; ++t)
                    yr[t] = re[t] * s;
            }
        }
        free(re);
        free(im);
    }
    free(kre);
    free(kim);
    return fail ? -1 : 0;
}


/* ---------------------------------------------------------------------
 * The operator family (kinds 0..3 above) and the kernel gradient.
 * ------------------------------------------------------------------- */

/* k index of the term pairing output position a with input position b of
 * operator `kind`, or -1 when the term is absent. */
static long op_tap(int kind, long a, long b, long N)
{
    switch (kind) {
    case 0: return b <= a ? a - b : -1;              /* y[a] += u[b] k[a-b] */
    case 1: return b >= a ? b - a : -1;              /* y[a] += u[b] k[b-a] */
    case 2: return ((a - b) % N + N) % N;            /* k[(a-b) mod N]      */
    default: return ((b - a) % N + N) % N;           /* k[(b-a) mod N]      */
    }
}

/* Operator `kind` by its definition; u, y [R][N], kern [Hk][N]. */
void oracle_op_direct(const double *u, const double *kern, const long *hidx,
                      double *y, long R, long N, int kind)
{
    long r;
#pragma omp parallel for schedule(dynamic, 1)
    for (r = 0; r < R; ++r) {
        const double *ur = u + r * N;
        const double *kr = kern + hidx[r] * N;
        for (long a = 0; a < N; ++a) {
            double acc = 0.0;
            for (long b = 0; b < N; ++b) {
                long j = op_tap(kind, a, b, N);
                if (j >= 0)
                    acc += ur[b] * kr[j];
            }
            y[r * N + a] = acc;
        }
    }
}

/* Single outputs out[i] = y[rows[i]][ts[i]] of operator `kind`. */
void oracle_op_points(const double *u, const double *kern, const long *hidx,
                      long N, const long *rows, const long *ts, long n,
                      int kind, double *out)
{
    long i;
#pragma omp parallel for schedule(dynamic, 16)
    for (i = 0; i < n; ++i) {
        const double *ur = u + rows[i] * N;
        const double *kr = kern + hidx[rows[i]] * N;
        double acc = 0.0;
        for (long b = 0; b < N; ++b) {
            long j = op_tap(kind, ts[i], b, N);
            if (j >= 0)
                acc += ur[b] * kr[j];
        }
        out[i] = acc;
    }
}

/* Operator `kind` through the convolution theorem: transform length
 * L = 2N (zero padded) for the causal kinds, N for the circular ones;
 * Y = U . K (kinds 0, 2) or U . conj(K) (kinds 1, 3); y = IFFT(Y)[0:N]. */
int oracle_op_fft(const double *u, const double *kern, const long *hidx,
                  double *y, long R, long Hk, long N, int kind)
{
    const long L = kind < 2 ? 2 * N : N;
    const double csign = (kind == 1 || kind == 3) ? -1.0 : 1.0;
    double *kre = (double *)malloc(sizeof(double) * (size_t)(Hk * L));
    double *kim = (double *)malloc(sizeof(double) * (size_t)(Hk * L));
    if (!kre || !kim) {
        free(kre);
        free(kim);
        return -1;
    }
    long h;
#pragma omp parallel for schedule(dynamic, 1)
    for (h = 0; h < Hk; ++h) {
        for (long t = 0; t < L; ++t) {
            kre[h * L + t] = t < N ? kern[h * N + t] : 0.0;
            kim[h * L + t] = 0.0;
        }
        fft_radix2(kre + h * L, kim + h * L, L, -1);
    }
    int fail = 0;
#pragma omp parallel
    {
        double *re = (double *)malloc(sizeof(double) * (size_t)L);
        double *im = (double *)malloc(sizeof(double) * (size_t)L);
        if (!re || !im) {
#pragma omp atomic write
            fail = 1;
        } else {
            long r;
#pragma omp for schedule(dynamic, 1)
            for (r = 0; r < R; ++r) {
                const double *Kr = kre + hidx[r] * L, *Ki = kim + hidx[r] * L;
                for (long t = 0; t < L; ++t) {
                    re[t] = t < N ? u[r * N + t] : 0.0;
                    im[t] = 0.0;
                }
                fft_radix2(re, im, L, -1);
                for (long f = 0; f < L; ++f) {
                    double a = re[f], b = im[f], c = Kr[f], d = csign * Ki[f];
                    re[f] = a * c - b * d;
                    im[f] = a * d + b * c;
                }
                fft_radix2(re, im, L, +1);
                for (long t = 0; t < N; ++t)
                    y[r * N + t] = re[t] / (double)L;
            }
        }
        free(re);
        free(im);
    }
    free(kre);
    free(kim);
    return fail ? -1 : 0;
}

/* Kernel gradient by its definition: dk [Hk][N] (overwritten). Causal
 * kinds (0, 1 -- the gradient of kind 0): dk[h][j] = sum_r sum_{t>=j}
 * dy[r][t] u[r][t-j]; circular kinds (2, 3): t-j taken mod N. */
void oracle_kgrad_direct(const double *u, const double *dy, const long *hidx,
                         double *dk, long R, long Hk, long N, int kind)
{
    long h;
#pragma omp parallel for schedule(dynamic, 1)
    for (h = 0; h < Hk; ++h) {
        for (long j = 0; j < N; ++j)
            dk[h * N + j] = 0.0;
        for (long r = 0; r < R; ++r) {
            if (hidx[r] != h)
                continue;
            const double *ur = u + r * N, *dr = dy + r * N;
            for (long j = 0; j < N; ++j) {
                double acc = 0.0;
                for (long t = 0; t < N; ++t) {
                    long s = t - j;
                    if (kind >= 2)
                        s = (s % N + N) % N;
                    else if (s < 0)
                        continue;
                    acc += dr[t] * ur[s];
                }
                dk[h * N + j] += acc;
            }
        }
    }
}

/* Kernel gradient through the convolution theorem: per row
 * G = conj(FFT(u)) . FFT(dy) (length 2N zero padded for the causal kinds,
 * N for the circular ones), summed over the rows of each channel, then
 * dk = IFFT(G)[0:N]. */
int oracle_kgrad_fft(const double *u, const double *dy, const long *hidx,
                     double *dk, long R, long Hk, long N, int kind)
{
    const long L = kind < 2 ? 2 * N : N;
    int fail = 0;
    long h;
#pragma omp parallel for schedule(dynamic, 1)
    for (h = 0; h < Hk; ++h) {
        double *gre = (double *)calloc((size_t)L, sizeof(double));
        double *gim = (double *)calloc((size_t)L, sizeof(double));
        double *are = (double *)malloc(sizeof(double) * (size_t)L);
        double *aim = (double *)malloc(sizeof(double) * (size_t)L);
        double *bre = (double *)malloc(sizeof(double) * (size_t)L);
        double *bim = (double *)malloc(sizeof(double) * (size_t)L);
        if (!gre || !gim || !are || !aim || !bre || !bim) {
#pragma omp atomic write
            fail = 1;
        } else {
            for (long r = 0; r < R; ++r) {
                if (hidx[r] != h)
                    continue;
                for (long t = 0; t < L; ++t) {
                    are[t] = t < N ? u[r * N + t] : 0.0;
                    bre[t] = t < N ? dy[r * N + t] : 0.0;
                    aim[t] = bim[t] = 0.0;
                }
                fft_radix2(are, aim, L, -1);
                fft_radix2(bre, bim, L, -1);
                for (long f = 0; f < L; ++f) {
                    /* conj(A) . B */
                    gre[f] += are[f] * bre[f] + aim[f] * bim[f];
                    gim[f] += are[f] * bim[f] - aim[f] * bre[f];
                }
            }
            fft_radix2(gre, gim, L, +1);
            for (long j = 0; j < N; ++j)
                dk[h * N + j] = gre[j] / (double)L;
        }
        free(gre);
        free(gim);
        free(are);
        free(aim);
        free(bre);
        free(bim);
    }
    return fail ? -1 : 0;
}

/* Single kernel-gradient entries out[i] = dk[hs[i]][js[i]] by the
 * definition. */
void oracle_kgrad_points(const double *u, const double *dy, const long *hidx,
                         long R, long N, const long *hs, const long *js,
                         long n, int kind, double *out)
{
    long i;
#pragma omp parallel for schedule(dynamic, 1)
    for (i = 0; i < n; ++i) {
        double acc = 0.0;
        for (long r = 0; r < R; ++r) {
            if (hidx[r] != hs[i])
                continue;
            const double *ur = u + r * N, *dr = dy + r * N;
            for (long t = 0; t < N; ++t) {
                long s = t - js[i];
                if (kind >= 2)
                    s = (s % N + N) % N;
                else if (s < 0)
                    continue;
                acc += dr[t] * ur[s];
            }
        }
        out[i] = acc;
    }
}


/* Frequency-sparse causal convolution: y = IFFT_2N(U . K_F)[0:N] with
 * K_F[f] = K[f] if min(f, 2N - f) <= F, else 0. */
int oracle_lowpass_fft(const double *u, const double *kern, const long *hidx,
                       double *y, long R, long Hk, long N, long F)
{
    const long L = 2 * N;
    double *kre = (double *)malloc(sizeof(double) * (size_t)(Hk * L));
    double *kim = (double *)malloc(sizeof(double) * (size_t)(Hk * L));
    if (!kre || !kim) {
        free(kre);
        free(kim);
        return -1;
    }
    oracle_kernel_spectrum(kern, Hk, N, kre, kim);
    for (long h = 0; h < Hk; ++h)
        for (long f = 0; f < L; ++f) {
            long dist = f < L - f ? f : L - f;
            if (dist > F) {
                kre[h * L + f] = 0.0;
                kim[h * L + f] = 0.0;
            }
        }
    int fail = 0;
#pragma omp parallel
    {
        double *re = (double *)malloc(sizeof(double) * (size_t)L);
        double *im = (double *)malloc(sizeof(double) * (size_t)L);
        if (!re || !im) {
#pragma omp atomic write
            fail = 1;
        } else {
            long r;
#pragma omp for schedule(dynamic, 1)
            for (r = 0; r < R; ++r) {
                const double *Kr = kre + hidx[r] * L, *Ki = kim + hidx[r] * L;
                for (long t = 0; t < L; ++t) {
                    re[t] = t < N ? u[r * N + t] : 0.0;
                    im[t] = 0.0;
                }
                fft_radix2(re, im, L, -1);
                for (long f = 0; f < L; ++f) {
                    double a = re[f], b = im[f];
                    re[f] = a * Kr[f] - b * Ki[f];
                    im[f] = a * Ki[f] + b * Kr[f];
                }
                fft_radix2(re, im, L, +1);
                for (long t = 0; t < N; ++t)
                    y[r * N + t] = re[t] / (double)L;
            }
        }
        free(re);
        free(im);
    }
    free(kre);
    free(kim);
    return fail ? -1 : 0;
}

/* Causal convolution with a masked kernel spectrum: y = IFFT_2N(U . K m)[0:N]
 * with m[f] in {0, 1} given for every f in [0, 2N) (mask[f] != 0 keeps the
 * frequency).  The frequency-sparse convolutions are such masks. */
int oracle_masked_fft(const double *u, const double *kern, const long *hidx,
                      double *y, long R, long Hk, long N, const double *mask)
{
    const long L = 2 * N;
    double *kre = (double *)malloc(sizeof(double) * (size_t)(Hk * L));
    double *kim = (double *)malloc(sizeof(double) * (size_t)(Hk * L));
    if (!kre || !kim) {
        free(kre);
        free(kim);
        return -1;
    }
    oracle_kernel_spectrum(kern, Hk, N, kre, kim);
    for (long h = 0; h < Hk; ++h)
        for (long f = 0; f < L; ++f) {
            kre[h * L + f] *= mask[f];
            kim[h * L + f] *= mask[f];
        }
    int fail = 0;
#pragma omp parallel
    {
        double *re = (double *)malloc(sizeof(double) * (size_t)L);
        double *im = (double *)malloc(sizeof(double) * (size_t)L);
        if (!re || !im) {
#pragma omp atomic write
            fail = 1;
        } else {
            long r;
#pragma omp for schedule(dynamic, 1)
            for (r = 0; r < R; ++r) {
                const double *Kr = kre + hidx[r] * L, *Ki = kim + hidx[r] * L;
                for (long t = 0; t < L; ++t) {
                    re[t] = t < N ? u[r * N + t] : 0.0;
                    im[t] = 0.0;
                }
                fft_radix2(re, im, L, -1);
                for (long f = 0; f < L; ++f) {
                    double a = re[f], b = im[f];
                    re[f] = a * Kr[f] - b * Ki[f];
                    im[f] = a * Ki[f] + b * Kr[f];
                }
                fft_radix2(re, im, L, +1);
                for (long t = 0; t < N; ++t)
                    y[r * N + t] = re[t] / (double)L;
            }
        }
        free(re);
        free(im);
    }
    free(kre);
    free(kim);
    return fail ? -1 : 0;
}
