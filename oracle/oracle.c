/*
 * oracle.c -- plain, slow fp64 CPU reference for conv2d -> BatchNorm -> SiLU.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it. It shares no code, header, table or constant with
 * the HIP library.
 *
 * What it computes (the plain definition; the fused kernels must reach the
 * same numbers up to rounding):
 *   - "Fusing an Epilogue" (teenygrad docs), section "The problem": a
 *     convolution, then batch normalisation, then SiLU, where batch norm is a
 *     per-channel multiply-and-add and SiLU is v times sigmoid(v); fusing the
 *     three changes where the data lives, not the arithmetic.
 *   - Same page, section "The shape of it": the result of the convolution is
 *     scaled and shifted per output channel, then multiplied by its own
 *     sigmoid, before the single store.
 * Readings of what the pages leave open (all pinned by the CPU tests):
 *   - the convolution is a cross-correlation (no kernel flip) with symmetric
 *     zero padding of x, dilation 1, one group, no conv bias;
 *   - output extent P = floor((H + 2 pad - kh) / stride) + 1, same for Q;
 *   - layouts: x NHWC [N][H][W][C_in], w OHWI [C_out][kh][kw][C_in],
 *     output NHWC [N][P][Q][C_out];
 *   - batch norm is the inference form with running statistics, written out
 *     unfolded: gamma * (t - mean) / sqrt(var + eps) + beta, eps inside the
 *     root;
 *   - sigmoid is the logistic function 1 / (1 + exp(-v)).
 *
 * Arithmetic is IEEE double with no contraction (built with
 * -ffp-contract=off, no fast-math), summation order r, s, c for every output.
 * Threads own disjoint (n, p) output rows, so the result does not depend on
 * the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL 1
#define ORACLE_ENOMEM 2

/* Output extent along one axis; 0 when the padded input is smaller than the
 * window. Reading: floor((in + 2 pad - k) / stride) + 1. */
long long oracle_out_extent(long long in, long long k, long long stride, long long pad)
{
    if (in < 1 || k < 1 || stride < 1 || pad < 0 || in + 2 * pad < k)
        return 0;
    return (in + 2 * pad - k) / stride + 1;
}

typedef struct {
    const double *x, *w;
    int N, H, W, C_in, C_out, kh, kw, stride, pad;
    long long P, Q;
} conv_geom;

/* One output value of the convolution: the sum over the window of x times w,
 * with x taken as zero outside [0,H) x [0,W). */
static double conv_point(const conv_geom *g, long long n, long long p, long long q, long long k)
{
    double acc = 0.0;
    for (int r = 0; r < g->kh; ++r) {
        long long ih = p * g->stride - g->pad + r;
        if (ih < 0 || ih >= g->H)
            continue;
        for (int s = 0; s < g->kw; ++s) {
            long long iw = q * g->stride - g->pad + s;
            if (iw < 0 || iw >= g->W)
                continue;
            const double *xp = g->x + ((n * g->H + ih) * g->W + iw) * g->C_in;
            const double *wp = g->w + ((k * g->kh + r) * g->kw + s) * g->C_in;
            for (int c = 0; c < g->C_in; ++c)
                acc += xp[c] * wp[c];
        }
    }
    return acc;
}

/* Batch normalisation, inference form, one value of channel k. */
static double bn_point(double t, double gamma, double beta, double mean, double var, double eps)
{
    return gamma * (t - mean) / sqrt(var + eps) + beta;
}

/* SiLU: v * sigmoid(v), sigmoid(v) = 1 / (1 + exp(-v)). For v -> -inf the
 * exponential overflows to +inf, sigmoid -> 0 and the result is -0. */
static double silu_point(double v)
{
    double sig = 1.0 / (1.0 + exp(-v));
    return v * sig;
}

typedef struct {
    const conv_geom *g;
    const double *gamma, *beta, *mean, *var;
    double eps;
    int stage; /* 0: conv only, 1: conv -> bn -> silu */
    double *out;
    int tid, nthreads;
} row_job;

static void *row_worker(void *arg)
{
    row_job *j = (row_job *)arg;
    const conv_geom *g = j->g;
    long long rows = (long long)g->N * g->P;
    for (long long row = j->tid; row < rows; row += j->nthreads) {
        long long n = row / g->P, p = row % g->P;
        for (long long q = 0; q < g->Q; ++q) {
            double *o = j->out + ((n * g->P + p) * g->Q + q) * g->C_out;
            for (long long k = 0; k < g->C_out; ++k) {
                double v = conv_point(g, n, p, q, k);
                if (j->stage == 1)
                    v = silu_point(bn_point(v, j->gamma[k], j->beta[k], j->mean[k], j->var[k], j->eps));
                o[k] = v;
            }
        }
    }
    return NULL;
}

static int check_geom(int N, int H, int W, int C_in, int C_out, int kh, int kw, int stride, int pad)
{
    if (N < 1 || H < 1 || W < 1 || C_in < 1 || C_out < 1 || kh < 1 || kw < 1 || stride < 1 || pad < 0)
        return ORACLE_EINVAL;
    if (oracle_out_extent(H, kh, stride, pad) == 0 || oracle_out_extent(W, kw, stride, pad) == 0)
        return ORACLE_EINVAL;
    return ORACLE_OK;
}

static int run_rows(const conv_geom *g, const double *gamma, const double *beta, const double *mean,
                    const double *var, double eps, int stage, double *out, int nthreads)
{
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    pthread_t th[256];
    row_job jobs[256];
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        row_job tmp = {g, gamma, beta, mean, var, eps, stage, out, t, nthreads};
        jobs[t] = tmp;
    }
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&th[t], NULL, row_worker, &jobs[t]) != 0)
            break;
        started = t;
    }
    /* Rows of threads that failed to start are done here, in order. */
    for (int t = started + 1; t < nthreads; ++t)
        row_worker(&jobs[t]);
    row_worker(&jobs[0]);
    for (int t = 1; t <= started; ++t)
        pthread_join(th[t], NULL);
    return ORACLE_OK;
}

/* Convolution alone: out[n][p][q][k]. */
int oracle_conv2d(const double *x, const double *w, int N, int H, int W, int C_in, int C_out, int kh,
                  int kw, int stride, int pad, double *out, int nthreads)
{
    int rc = check_geom(N, H, W, C_in, C_out, kh, kw, stride, pad);
    if (rc)
        return rc;
    conv_geom g = {x, w, N, H, W, C_in, C_out, kh, kw, stride, pad,
                   oracle_out_extent(H, kh, stride, pad), oracle_out_extent(W, kw, stride, pad)};
    return run_rows(&g, NULL, NULL, NULL, NULL, 0.0, 0, out, nthreads);
}

/* Batch normalisation alone over a channels-last tensor of n_pix pixels. */
void oracle_batchnorm(const double *t, long long n_pix, int C, const double *gamma, const double *beta,
                      const double *mean, const double *var, double eps, double *out)
{
    for (long long i = 0; i < n_pix; ++i)
        for (int k = 0; k < C; ++k)
            out[i * C + k] = bn_point(t[i * C + k], gamma[k], beta[k], mean[k], var[k], eps);
}

/* SiLU alone, elementwise. */
void oracle_silu(const double *t, long long n, double *out)
{
    for (long long i = 0; i < n; ++i)
        out[i] = silu_point(t[i]);
}

/* The whole path, element by element: silu(bn(conv(x, w))). */
int oracle_conv_bn_silu(const double *x, const double *w, int N, int H, int W, int C_in, int C_out,
                        int kh, int kw, int stride, int pad, const double *gamma, const double *beta,
                        const double *mean, const double *var, double eps, double *out, int nthreads)
{
    int rc = check_geom(N, H, W, C_in, C_out, kh, kw, stride, pad);
    if (rc)
        return rc;
    conv_geom g = {x, w, N, H, W, C_in, C_out, kh, kw, stride, pad,
                   oracle_out_extent(H, kh, stride, pad), oracle_out_extent(W, kw, stride, pad)};
    return run_rows(&g, gamma, beta, mean, var, eps, 1, out, nthreads);
}

/* The whole path at selected flat output indices (into [N][P][Q][C_out]),
 * for outputs of shapes too large to compute in full. */
int oracle_conv_bn_silu_at(const double *x, const double *w, int N, int H, int W, int C_in, int C_out,
                           int kh, int kw, int stride, int pad, const double *gamma, const double *beta,
                           const double *mean, const double *var, double eps, const long long *idx,
                           long long n_idx, double *out)
{
    int rc = check_geom(N, H, W, C_in, C_out, kh, kw, stride, pad);
    if (rc)
        return rc;
    conv_geom g = {x, w, N, H, W, C_in, C_out, kh, kw, stride, pad,
                   oracle_out_extent(H, kh, stride, pad), oracle_out_extent(W, kw, stride, pad)};
    long long total = (long long)N * g.P * g.Q * C_out;
    for (long long j = 0; j < n_idx; ++j) {
        long long i = idx[j];
        if (i < 0 || i >= total)
            return ORACLE_EINVAL;
        long long k = i % C_out, pix = i / C_out;
        long long q = pix % g.Q, p = (pix / g.Q) % g.P, n = pix / (g.Q * g.P);
        double v = conv_point(&g, n, p, q, k);
        out[j] = silu_point(bn_point(v, gamma[k], beta[k], mean[k], var[k], eps));
    }
    return ORACLE_OK;
}
