/*
 * Test infrastructure (not part of the library): drives every function of
 * the fp64 oracle (oracle/hc_oracle.c) on small seeded inputs, so that a
 * build with AddressSanitizer and UndefinedBehaviorSanitizer sees each of
 * them read and write its buffers.  Every buffer is allocated at exactly
 * the size the function's contract names, so an access one element past it
 * is reported.  Exit status 0 when every call returned as documented.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

double hco_bf16_to_double(uint16_t b);
uint16_t hco_round_bf16(double v);
void hco_round_bf16_array(const double *v, int64_t n, uint16_t *out);
void hco_mixes(const uint16_t *R, const float *W, int64_t n, int hc, int d, double norm_eps, double *mixes);
int hco_split_sinkhorn(const double *mixes, const float *scale, const float *base, int64_t n, int hc, int iters,
                       double eps, double *pre, double *post, double *comb);
void hco_pre(const uint16_t *R, const double *pre, int64_t n, int hc, int d, uint16_t *h);
void hco_post(const uint16_t *x, const uint16_t *R, const double *post, const double *comb, int64_t n, int hc,
              int d, uint16_t *Rout);
void hco_diag_scale(const uint16_t *h, const uint16_t *D, int64_t n, int d, uint16_t *x);
void hco_rmsnorm(const uint16_t *h, const float *gamma, int64_t n, int d, double norm_eps, uint16_t *y);
void hco_post_backward(const uint16_t *x, const uint16_t *R, const double *post, const double *comb,
                       const uint16_t *gRout, int64_t n, int hc, int d, double *gx, double *gpost, double *gcomb,
                       double *gR);
void hco_pre_backward(const uint16_t *R, const double *pre, const uint16_t *gh, int64_t n, int hc, int d,
                      double *gpre, double *gR);
int hco_split_sinkhorn_backward(const double *mixes, const float *scale, const float *base, const double *gpre,
                                const double *gpost, const double *gcomb, int64_t n, int hc, int iters, double eps,
                                double *gmixes, double *gscale_tok, double *gbase_tok);
void hco_mixes_backward(const uint16_t *R, const float *W, const double *gmixes, int64_t n, int hc, int d,
                        double norm_eps, double *gR, double *gW);
int hco_num_threads(void);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static double unif(void) {                   /* splitmix64, mapped to [-1, 1) */
    uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (double)(z >> 11) / (double)(1ull << 52) - 1.0;
}
static void *xmalloc(size_t bytes) {         /* exact size; 1 byte for empty arrays */
    void *p = malloc(bytes ? bytes : 1);
    if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
    return p;
}
static uint16_t *bf16s(int64_t count) {
    uint16_t *p = xmalloc(sizeof(uint16_t) * (size_t)count);
    for (int64_t i = 0; i < count; ++i) p[i] = hco_round_bf16(unif() * 2.0);
    return p;
}
static float *f32s(int64_t count, double lo, double hi) {
    float *p = xmalloc(sizeof(float) * (size_t)count);
    for (int64_t i = 0; i < count; ++i) p[i] = (float)(lo + (hi - lo) * (unif() + 1.0) * 0.5);
    return p;
}
static double *f64s(int64_t count, double lo, double hi) {
    double *p = xmalloc(sizeof(double) * (size_t)count);
    for (int64_t i = 0; i < count; ++i) p[i] = lo + (hi - lo) * (unif() + 1.0) * 0.5;
    return p;
}

static int run(int64_t n, int hc, int d, int iters) {
    const int M = (2 + hc) * hc;
    const int64_t K = (int64_t)hc * d;
    int bad = 0;
    uint16_t *R = bf16s(n * K), *x = bf16s(n * d), *D = bf16s(d), *gh = bf16s(n * d), *gRout = bf16s(n * K);
    float *W = f32s((int64_t)M * K, -0.01, 0.01), *scale = f32s(3, 0.5, 2.0), *base = f32s(M, -1.0, 1.0);
    float *gamma = f32s(d, 0.5, 1.5);
    double *mixes = xmalloc(sizeof(double) * (size_t)(n * M));
    double *pre = xmalloc(sizeof(double) * (size_t)(n * hc)), *post = xmalloc(sizeof(double) * (size_t)(n * hc));
    double *comb = xmalloc(sizeof(double) * (size_t)(n * hc * hc));
    uint16_t *h = xmalloc(sizeof(uint16_t) * (size_t)(n * d)), *y = xmalloc(sizeof(uint16_t) * (size_t)(n * d));
    uint16_t *xs = xmalloc(sizeof(uint16_t) * (size_t)(n * d)), *Rout = xmalloc(sizeof(uint16_t) * (size_t)(n * K));

    hco_mixes(R, W, n, hc, d, 1e-20, mixes);
    bad |= hco_split_sinkhorn(mixes, scale, base, n, hc, iters, 1e-6, pre, post, comb) != 0;
    hco_pre(R, pre, n, hc, d, h);
    hco_post(x, R, post, comb, n, hc, d, Rout);
    hco_diag_scale(h, D, n, d, xs);
    hco_rmsnorm(h, gamma, n, d, 1e-20, y);
    hco_rmsnorm(h, gamma, n, d, 0.0, y);

    double *gx = xmalloc(sizeof(double) * (size_t)(n * d)), *gpost = xmalloc(sizeof(double) * (size_t)(n * hc));
    double *gcomb = xmalloc(sizeof(double) * (size_t)(n * hc * hc)), *gR = xmalloc(sizeof(double) * (size_t)(n * K));
    double *gpre = xmalloc(sizeof(double) * (size_t)(n * hc)), *gR2 = xmalloc(sizeof(double) * (size_t)(n * K));
    double *gmixes = xmalloc(sizeof(double) * (size_t)(n * M)), *gsc = xmalloc(sizeof(double) * (size_t)(n * 3));
    double *gba = xmalloc(sizeof(double) * (size_t)(n * M)), *gR3 = xmalloc(sizeof(double) * (size_t)(n * K));
    double *gW = xmalloc(sizeof(double) * (size_t)M * (size_t)K);
    double *gp = f64s(n * hc, -1.0, 1.0), *gq = f64s(n * hc, -1.0, 1.0), *gc = f64s(n * hc * hc, -1.0, 1.0);
    hco_post_backward(x, R, post, comb, gRout, n, hc, d, gx, gpost, gcomb, gR);
    hco_pre_backward(R, pre, gh, n, hc, d, gpre, gR2);
    bad |= hco_split_sinkhorn_backward(mixes, scale, base, gp, gq, gc, n, hc, iters, 1e-6, gmixes, gsc, gba) != 0;
    hco_mixes_backward(R, W, gmixes, n, hc, d, 1e-20, gR3, gW);

    /* the documented refusals */
    bad |= hco_split_sinkhorn(mixes, scale, base, n, hc, 0, 1e-6, pre, post, comb) != -1;
    bad |= hco_split_sinkhorn(mixes, scale, base, n, 0, iters, 1e-6, pre, post, comb) != -1;

    free(R); free(x); free(D); free(gh); free(gRout); free(W); free(scale); free(base); free(gamma);
    free(mixes); free(pre); free(post); free(comb); free(h); free(y); free(xs); free(Rout);
    free(gx); free(gpost); free(gcomb); free(gR); free(gpre); free(gR2); free(gmixes); free(gsc); free(gba);
    free(gR3); free(gW); free(gp); free(gq); free(gc);
    if (bad) fprintf(stderr, "a call returned other than documented at n=%lld hc=%d d=%d\n", (long long)n, hc, d);
    return bad;
}

int main(void) {
    int bad = 0;
    double v[5] = {0.0, -1.5, 3.0e38, 1e-40, 65504.0};
    uint16_t out[5];
    hco_round_bf16_array(v, 5, out);
    bad |= hco_bf16_to_double(out[1]) != -1.5;
    bad |= hco_num_threads() < 1;
    const int64_t ns[] = {0, 1, 3};
    const int hcs[] = {1, 2, 4, 8};
    const int ds[] = {8, 24};
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 4; ++j)
            for (int k = 0; k < 2; ++k) bad |= run(ns[i], hcs[j], ds[k], 3);
    bad |= run(2, 4, 64, 20);
    printf(bad ? "FAIL\n" : "ok\n");
    return bad;
}
