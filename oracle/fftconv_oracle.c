/*
 * fftconv_oracle.c -- CPU oracle for the exact causal long FFT convolution.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the package smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or helper with
 * the HIP library.
 *
 * What it computes (FlashFFTConv summary page, "Summary" and "Key results":
 * the method computes the *exact* FFT convolution, with gating fused into the
 * kernel ("Measured effects" row on fused gating), with partial (short) filters
 * and with frequency-sparse filters whose zeroed frequency-domain entries are
 * skipped ("Approach"):
 *
 *     y[b,h,t] = v[b,h,t] * sum_{s=0}^{min(t, L-1)} k[h,s] * u[b,h,t-s] * w[b,h,t-s]
 *
 * for t in [0, N).  Exactness of the convolution theorem makes this equal to
 *     v * irfft( rfft(pad(u*w, 2N)) * rfft(pad(k, 2N)) )[:N]
 * which is route F below.  w == NULL or v == NULL means that gate is absent.
 *
 * Frequency-sparse reading (the pages give only the fraction of zeroed
 * entries): the 2N-point real spectrum's bins f in [0, N] are split in 128
 * blocks of G = N/128 bins, the Nyquist bin N joining block 127; mask[h, blk]
 * = 0 zeroes those bins of the filter spectrum and their Hermitian mirrors
 * 2N - f.  The masked result is no longer a causal linear convolution: it is
 * the circular convolution (length 2N) of the zero-padded input with
 * k' = IFFT(mask * FFT(pad(k, 2N))), truncated to t < N.
 *
 * Everything is float64.  All routines are plain loops; the only threading is
 * an OpenMP loop over independent (b, h) sequences.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_PI 3.14159265358979323846264338327950288

static int pick_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#else
    nthreads = 1;
#endif
    return nthreads;
}

int oracle_max_threads(void) { return pick_threads(0); }

/* ------------------------------------------------------------------------ */
/* Complex FFT: iterative radix-2 decimation in time (textbook Cooley-Tukey). */
/* sign = -1: X[f] = sum_n x[n] exp(-2 pi i f n / M)  (forward)               */
/* sign = +1: the same with exp(+...), no 1/M scaling (unnormalised inverse). */
/* M must be a power of two.  Each twiddle is computed directly from cos/sin  */
/* of its own angle in double, with no recurrence.                            */
/* ------------------------------------------------------------------------ */
int oracle_fft(double *re, double *im, int64_t M, int sign)
{
    if (M < 1 || (M & (M - 1)) != 0) return 1;
    if (sign != 1 && sign != -1) return 1;
    /* bit-reversal permutation */
    int64_t j = 0;
    for (int64_t i = 0; i < M - 1; ++i) {
        if (i < j) {
            double tr = re[i]; re[i] = re[j]; re[j] = tr;
            double ti = im[i]; im[i] = im[j]; im[j] = ti;
        }
        int64_t bit = M >> 1;
        while (j & bit) { j ^= bit; bit >>= 1; }
        j |= bit;
    }
    /* butterflies: sub-transforms of length len combine into 2*len */
    for (int64_t len = 1; len < M; len <<= 1) {
        for (int64_t p = 0; p < len; ++p) {
            double ang = (double)sign * ORACLE_PI * (double)p / (double)len;
            double wr = cos(ang), wi = sin(ang);
            for (int64_t s = p; s < M; s += 2 * len) {
                int64_t q = s + len;
                double br = re[q] * wr - im[q] * wi;
                double bi = re[q] * wi + im[q] * wr;
                re[q] = re[s] - br; im[q] = im[s] - bi;
                re[s] = re[s] + br; im[s] = im[s] + bi;
            }
        }
    }
    return 0;
}

/* Mask lookup for rfft bin f in [0, N]: blocks of N/128 bins, Nyquist -> last. */
int64_t oracle_mask_blocks(int64_t N) { (void)N; return 128; }

static int bin_kept(const uint8_t *mask_row, int64_t nblk, int64_t N, int64_t f)
{
    int64_t G = N / nblk;
    int64_t b = f / G;
    if (b > nblk - 1) b = nblk - 1;
    return mask_row[b] != 0;
}

/* ------------------------------------------------------------------------ */
/* Route D: direct causal convolution, the definition written out.           */
/* ------------------------------------------------------------------------ */
static void direct_one(const double *u, const double *w, const double *v,
                       const double *k, int64_t N, int64_t L, double *y)
{
    for (int64_t t = 0; t < N; ++t) {
        int64_t smax = t < L - 1 ? t : L - 1;
        double acc = 0.0;
        for (int64_t s = 0; s <= smax; ++s) {
            double x = u[t - s] * (w ? w[t - s] : 1.0);
            acc += k[s] * x;
        }
        y[t] = (v ? v[t] : 1.0) * acc;
    }
}

int oracle_direct(const double *u, const double *w, const double *v,
                  const double *k, int64_t B, int64_t H, int64_t N, int64_t L,
                  double *y, int nthreads)
{
    if (B < 0 || H < 0 || N < 1 || L < 1 || L > N) return 1;
    int64_t S = B * H;
    nthreads = pick_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t s = 0; s < S; ++s) {
        int64_t h = s % H;
        direct_one(u + s * N, w ? w + s * N : NULL, v ? v + s * N : NULL,
                   k + h * L, N, L, y + s * N);
    }
    return 0;
}

/* Route D at sampled outputs: pts holds (b, h, t) triples. */
int oracle_direct_points(const double *u, const double *w, const double *v,
                         const double *k, int64_t B, int64_t H, int64_t N,
                         int64_t L, const int64_t *pts, int64_t npts,
                         double *out, int nthreads)
{
    if (B < 0 || H < 0 || N < 1 || L < 1 || L > N) return 1;
    nthreads = pick_threads(nthreads);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 16) num_threads(nthreads) reduction(| : bad)
    for (int64_t p = 0; p < npts; ++p) {
        int64_t b = pts[3 * p], h = pts[3 * p + 1], t = pts[3 * p + 2];
        if (b < 0 || b >= B || h < 0 || h >= H || t < 0 || t >= N) { bad = 1; continue; }
        const double *us = u + (b * H + h) * N;
        const double *ws = w ? w + (b * H + h) * N : NULL;
        int64_t smax = t < L - 1 ? t : L - 1;
        double acc = 0.0;
        for (int64_t s = 0; s <= smax; ++s)
            acc += k[h * L + s] * (us[t - s] * (ws ? ws[t - s] : 1.0));
        out[p] = (v ? v[(b * H + h) * N + t] : 1.0) * acc;
    }
    return bad;
}

/* ------------------------------------------------------------------------ */
/* Route F: convolution theorem with the oracle's own FFT, FFT size M >= 2N. */
/* Optional frequency mask (H x 128 uint8, see the file header).             */
/* max_imag (optional) returns max over sequences of max|Im z| / max|z|.     */
/* ------------------------------------------------------------------------ */
int oracle_fft_conv(const double *u, const double *w, const double *v,
                    const double *k, int64_t B, int64_t H, int64_t N, int64_t L,
                    const uint8_t *mask, int64_t M, double *y, double *max_imag,
                    int nthreads)
{
    if (B < 0 || H < 0 || N < 1 || L < 1 || L > N) return 1;
    if (M < 2 * N || (M & (M - 1)) != 0) return 1;
    if (mask && (M != 2 * N || N < 128)) return 1; /* mask is defined on the 2N-point spectrum */
    int64_t S = B * H;
    int64_t nblk = oracle_mask_blocks(N);
    double worst = 0.0;
    nthreads = pick_threads(nthreads);
    int fail = 0;
#pragma omp parallel num_threads(nthreads) reduction(max : worst) reduction(| : fail)
    {
        double *xr = (double *)malloc(sizeof(double) * (size_t)M);
        double *xi = (double *)malloc(sizeof(double) * (size_t)M);
        double *kr = (double *)malloc(sizeof(double) * (size_t)M);
        double *ki = (double *)malloc(sizeof(double) * (size_t)M);
        if (!xr || !xi || !kr || !ki) fail = 1;
        int64_t cached_h = -1;
#pragma omp for schedule(dynamic, 1)
        for (int64_t s = 0; s < S; ++s) {
            if (fail) continue;
            int64_t h = s % H;
            if (h != cached_h) {
                /* K = FFT_M(pad(k[h, :L])), then the optional mask */
                for (int64_t n = 0; n < M; ++n) { kr[n] = n < L ? k[h * L + n] : 0.0; ki[n] = 0.0; }
                oracle_fft(kr, ki, M, -1);
                if (mask) {
                    for (int64_t f = 0; f < M; ++f) {
                        int64_t fr = f <= N ? f : M - f; /* Hermitian mirror into [0, N] */
                        if (!bin_kept(mask + h * nblk, nblk, N, fr)) { kr[f] = 0.0; ki[f] = 0.0; }
                    }
                }
                cached_h = h;
            }
            const double *us = u + s * N;
            const double *ws = w ? w + s * N : NULL;
            for (int64_t n = 0; n < M; ++n) {
                xr[n] = n < N ? us[n] * (ws ? ws[n] : 1.0) : 0.0;
                xi[n] = 0.0;
            }
            oracle_fft(xr, xi, M, -1);
            for (int64_t f = 0; f < M; ++f) {
                double a = xr[f], bq = xi[f];
                xr[f] = a * kr[f] - bq * ki[f];
                xi[f] = a * ki[f] + bq * kr[f];
            }
            oracle_fft(xr, xi, M, +1);
            double zmax = 0.0, imax = 0.0;
            for (int64_t t = 0; t < M; ++t) {
                double ar = fabs(xr[t]) / (double)M, ai = fabs(xi[t]) / (double)M;
                if (ar > zmax) zmax = ar;
                if (ai > zmax) zmax = ai;
                if (ai > imax) imax = ai;
            }
            double ratio = zmax > 0.0 ? imax / zmax : 0.0;
            if (ratio > worst) worst = ratio;
            const double *vs = v ? v + s * N : NULL;
            for (int64_t t = 0; t < N; ++t)
                y[s * N + t] = (vs ? vs[t] : 1.0) * (xr[t] / (double)M);
        }
        free(xr); free(xi); free(kr); free(ki);
    }
    if (max_imag) *max_imag = worst;
    return fail ? 2 : 0;
}

/* ------------------------------------------------------------------------ */
/* Masked filter in the time domain: kp[0..2N) = Re IFFT(mask * FFT(pad(k))). */
/* Used for sampled masked outputs through the circular form.                */
/* ------------------------------------------------------------------------ */
int oracle_masked_filter(const double *k_row, int64_t L, int64_t N,
                         const uint8_t *mask_row, double *kp)
{
    if (N < 128 || L < 1 || L > N) return 1;
    int64_t M = 2 * N, nblk = oracle_mask_blocks(N);
    double *re = (double *)malloc(sizeof(double) * (size_t)M);
    double *im = (double *)malloc(sizeof(double) * (size_t)M);
    if (!re || !im) { free(re); free(im); return 2; }
    for (int64_t n = 0; n < M; ++n) { re[n] = n < L ? k_row[n] : 0.0; im[n] = 0.0; }
    oracle_fft(re, im, M, -1);
    for (int64_t f = 0; f < M; ++f) {
        int64_t fr = f <= N ? f : M - f;
        if (!bin_kept(mask_row, nblk, N, fr)) { re[f] = 0.0; im[f] = 0.0; }
    }
    oracle_fft(re, im, M, +1);
    for (int64_t n = 0; n < M; ++n) kp[n] = re[n] / (double)M;
    free(re); free(im);
    return 0;
}

/* Circular-form output at sampled points of ONE sequence:                    */
/* y[t] = g_v[t] * sum_{s=0}^{2N-1} kp[s] * x[(t - s) mod 2N], x zero beyond N.  */
int oracle_circular_points(const double *u, const double *w, const double *v,
                           const double *kp, int64_t N, const int64_t *ts,
                           int64_t nts, double *out)
{
    int64_t M = 2 * N;
    for (int64_t p = 0; p < nts; ++p) {
        int64_t t = ts[p];
        if (t < 0 || t >= N) return 1;
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n) { /* x[n] nonzero only for n < N */
            int64_t s = (t - n) % M;
            if (s < 0) s += M;
            acc += kp[s] * u[n] * (w ? w[n] : 1.0);
        }
        out[p] = (v ? v[t] : 1.0) * acc;
    }
    return 0;
}
