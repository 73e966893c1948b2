/* Driver for a sanitizer build of oracle/oracle.c (AddressSanitizer and
 * UndefinedBehaviorSanitizer): every exported function on small random
 * shapes -- strides 1..3, padding 0..2, windows up to the padded input,
 * 1..5 threads -- plus the geometry checks that must reject. Results are
 * checked for self-consistency (the fused entry equals the composed stages;
 * the sampled entry equals the full one; the thread count changes nothing).
 * The sanitizers abort on the first out-of-bounds access, use after free
 * or undefined behaviour. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

long long oracle_out_extent(long long in, long long k, long long stride, long long pad);
int oracle_conv2d(const double *x, const double *w, int N, int H, int W, int C_in, int C_out,
                  int kh, int kw, int stride, int pad, double *out, int nthreads);
void oracle_batchnorm(const double *t, long long n_pix, int C, const double *gamma,
                      const double *beta, const double *mean, const double *var, double eps,
                      double *out);
void oracle_silu(const double *t, long long n, double *out);
int oracle_conv_bn_silu(const double *x, const double *w, int N, int H, int W, int C_in,
                        int C_out, int kh, int kw, int stride, int pad, const double *gamma,
                        const double *beta, const double *mean, const double *var, double eps,
                        double *out, int nthreads);
int oracle_conv_bn_silu_at(const double *x, const double *w, int N, int H, int W, int C_in,
                           int C_out, int kh, int kw, int stride, int pad, const double *gamma,
                           const double *beta, const double *mean, const double *var,
                           double eps, const long long *idx, long long n_idx, double *out);

static unsigned long long rng = 88172645463325252ULL;
static double urand(void) {
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (double)(rng >> 11) / 9007199254740992.0;
}
static int irand(int lo, int hi) { return lo + (int)(urand() * (hi - lo + 1)); }

static double *fill(size_t n, double lo, double hi) {
    double *a = (double *)malloc((n ? n : 1) * sizeof(double));
    for (size_t i = 0; i < n; ++i) a[i] = lo + (hi - lo) * urand();
    return a;
}

int main(void) {
    int failures = 0, cases = 0;
    for (int it = 0; it < 200; ++it) {
        int N = irand(1, 2), H = irand(1, 9), W = irand(1, 9), Ci = irand(1, 5), Co = irand(1, 6);
        int kh = irand(1, 5), kw = irand(1, 5), s = irand(1, 3), p = irand(0, 2);
        long long P = oracle_out_extent(H, kh, s, p), Q = oracle_out_extent(W, kw, s, p);
        double *x = fill((size_t)N * H * W * Ci, -1, 1), *w = fill((size_t)Co * kh * kw * Ci, -1, 1);
        double *g = fill(Co, 0.5, 1.5), *b = fill(Co, -0.3, 0.3), *m = fill(Co, -0.3, 0.3);
        double *v = fill(Co, 0.5, 2.0);
        if (P == 0 || Q == 0) {
            double dummy;
            if (oracle_conv2d(x, w, N, H, W, Ci, Co, kh, kw, s, p, &dummy, 2) == 0) ++failures;
        } else {
            size_t n = (size_t)N * P * Q * Co;
            double *c = (double *)malloc(n * sizeof(double)), *bn = (double *)malloc(n * sizeof(double));
            double *y1 = (double *)malloc(n * sizeof(double)), *y2 = (double *)malloc(n * sizeof(double));
            double *ys = (double *)malloc(n * sizeof(double));
            long long *idx = (long long *)malloc(n * sizeof(long long));
            int th = irand(1, 5);
            if (oracle_conv2d(x, w, N, H, W, Ci, Co, kh, kw, s, p, c, th)) ++failures;
            oracle_batchnorm(c, (long long)N * P * Q, Co, g, b, m, v, 1e-5, bn);
            oracle_silu(bn, (long long)n, y1);
            if (oracle_conv_bn_silu(x, w, N, H, W, Ci, Co, kh, kw, s, p, g, b, m, v, 1e-5, y2, th))
                ++failures;
            for (size_t i = 0; i < n; ++i) idx[i] = (long long)(n - 1 - i);
            if (oracle_conv_bn_silu_at(x, w, N, H, W, Ci, Co, kh, kw, s, p, g, b, m, v, 1e-5, idx,
                                       (long long)n, ys))
                ++failures;
            for (size_t i = 0; i < n; ++i) {
                if (memcmp(&y1[i], &y2[i], sizeof(double)) != 0) ++failures;
                if (memcmp(&ys[i], &y2[n - 1 - i], sizeof(double)) != 0) ++failures;
            }
            idx[0] = (long long)n;  /* out of range: rejected */
            if (oracle_conv_bn_silu_at(x, w, N, H, W, Ci, Co, kh, kw, s, p, g, b, m, v, 1e-5, idx,
                                       1, ys) == 0)
                ++failures;
            free(c); free(bn); free(y1); free(y2); free(ys); free(idx);
            ++cases;
        }
        free(x); free(w); free(g); free(b); free(m); free(v);
    }
    double big[4] = {-1e4, -800.0, 0.0, 800.0}, out[4];
    oracle_silu(big, 4, out);
    if (!(out[0] == 0.0 && out[2] == 0.0 && out[3] == 800.0)) ++failures;
    if (oracle_out_extent(0, 1, 1, 0) != 0 || oracle_out_extent(4, 3, 0, 0) != 0) ++failures;
    printf("oracle_driver: %d cases, %d failures\n", cases, failures);
    return failures == 0 ? 0 : 1;
}
