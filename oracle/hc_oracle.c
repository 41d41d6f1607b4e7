/*
 * hc_oracle.c -- plain, slow, fp64 CPU oracle for hyper-connection residual
 * mixing (mix projection, split into pre/post/comb with epsilon-Sinkhorn,
 * hc_pre collapse, hc_post expansion).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the correctness reference that the
 * GPU library is checked against.  Only the test suite, the package smoke
 * check and the benchmark's CPU-baseline leg may build, load or call it; the
 * product path never does.  It shares no code, header or constant with the
 * GPU library.
 *
 * Sources it follows (the pages' own titles and listings):
 *   [MP]  "DeepSeek V4.1 - Mix projection" page: the mix formula
 *         m = x^f W^T / sqrt(mean((x^f)^2) + eps), eps = 1e-20, float32 in the
 *         model; and the Block.hc_mixes / hc_pre / hc_post listing.
 *   [RW]  "DeepSeek V4.1 - Reading weights" page: the learned-pre formula and
 *         the hc_split_sinkhorn kernel listing (split, row softmax + eps,
 *         column normalisation, then alternating row/column normalisations).
 *   [AT]  "DeepSeek V4.1 attention" page, config.json: hc_mult 4,
 *         hc_sinkhorn_iters 20, hc_eps 1e-6, norm_eps 1e-20, dim 5120.
 *
 * Conventions:
 *   - bf16 tensors are passed as their 16-bit patterns (uint16_t); fp32
 *     parameters as float; every computation is done in double.
 *   - R is [n][hc][d] (stream-major flattening: element (k,c) at k*d + c,
 *     as x.flatten(2) in [MP]); x and h are [n][d]; W is [(2+hc)*hc][hc*d];
 *     mixes is [n][(2+hc)*hc]; pre/post [n][hc]; comb [n][hc][hc] with
 *     comb[j][k] at j*hc + k.
 *   - bf16 outputs are rounded once, directly from the double value, to
 *     nearest with ties to even; overflow gives +-inf (see hco_round_bf16).
 *
 * Parity status: every function here is pinned by tests against closed
 * forms, invariants, special cases, an independent library routine or a
 * high-precision brute force in a different formulation; none is
 * "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define HCO_MAX_HC 16

/* bf16 pattern -> double, exact (a bf16 value is the top half of a float). */
double hco_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * Round a double to bf16 (8 significant bits, float's exponent range) once,
 * to nearest, ties to even.  Written out from the definition: pick the
 * spacing of representable bf16 values around |v|, scale so that those
 * values are integers, round that to the nearest integer (ties to even, the
 * default rounding mode of nearbyint) and scale back.  Results at or beyond
 * 2^128 overflow to infinity; NaN maps to the canonical quiet NaN.
 */
uint16_t hco_round_bf16(double v)
{
    if (isnan(v))
        return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isinf(a))
        return sign | 0x7F80;
    if (a == 0.0)
        return sign;
    int e;
    (void)frexp(a, &e);         /* a = f * 2^e with f in [0.5, 1) */
    int lead = e - 1;           /* a in [2^lead, 2^(lead+1)) */
    if (lead < -126)
        lead = -126;            /* subnormal bf16: fixed spacing 2^-133 */
    double q = ldexp(a, 7 - lead);          /* spacing becomes 1 */
    double r = nearbyint(q);                /* ties to even */
    double y = ldexp(r, lead - 7);
    if (y >= 0x1p128)
        return sign | 0x7F80;
    float f = (float)y;                     /* exact: <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return sign | (uint16_t)(u >> 16);
}

/* Logistic function, evaluated without overflow for either sign. */
static double sigmoid(double z)
{
    if (z >= 0.0)
        return 1.0 / (1.0 + exp(-z));
    double ez = exp(z);
    return ez / (1.0 + ez);
}

/*
 * [MP] mix formula: per token, over the flattened hc*d stream,
 *   r = 1 / sqrt( sum_i x_i^2 / K + norm_eps ),   m_j = r * sum_i x_i W[j][i].
 * One statistic per token; the dot product is taken first and then scaled,
 * as F.linear(x, hc_fn) * rsqrt does.
 */
void hco_mixes(const uint16_t *R, const float *W, int64_t n, int hc, int d,
               double norm_eps, double *mixes)
{
    const int64_t K = (int64_t)hc * d;
    const int M = (2 + hc) * hc;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        const uint16_t *x = R + t * K;
        double ss = 0.0;
        for (int64_t i = 0; i < K; ++i) {
            double v = hco_bf16_to_double(x[i]);
            ss += v * v;
        }
        double r = 1.0 / sqrt(ss / (double)K + norm_eps);
        for (int j = 0; j < M; ++j) {
            const float *w = W + (int64_t)j * K;
            double acc = 0.0;
            for (int64_t i = 0; i < K; ++i)
                acc += hco_bf16_to_double(x[i]) * (double)w[i];
            mixes[t * M + j] = acc * r;
        }
    }
}

/* comb[j][k] /= (sum_k' comb[j][k'] + eps)  -- a row normalisation. */
static void row_normalise(double C[HCO_MAX_HC][HCO_MAX_HC], int hc, double eps)
{
    for (int j = 0; j < hc; ++j) {
        double s = 0.0;
        for (int k = 0; k < hc; ++k)
            s += C[j][k];
        for (int k = 0; k < hc; ++k)
            C[j][k] = C[j][k] / (s + eps);
    }
}

/* comb[j][k] /= (sum_j' comb[j'][k] + eps)  -- a column normalisation. */
static void col_normalise(double C[HCO_MAX_HC][HCO_MAX_HC], int hc, double eps)
{
    for (int k = 0; k < hc; ++k) {
        double s = 0.0;
        for (int j = 0; j < hc; ++j)
            s += C[j][k];
        for (int j = 0; j < hc; ++j)
            C[j][k] = C[j][k] / (s + eps);
    }
}

/*
 * [RW] split and epsilon-Sinkhorn, in the listing's order:
 *   pre_j  = sigmoid(s0 * m_j + b_j) + eps                     (j < hc)
 *   post_j = 2 * sigmoid(s1 * m_{hc+j} + b_{hc+j})
 *   L_jk   = s2 * m_{2hc + j*hc + k} + b_{2hc + j*hc + k}
 *   C = softmax over each row of L, plus eps on every entry;
 *   C = C / (column sums + eps);
 *   then (iters - 1) times: C = C / (row sums + eps); C = C / (column sums + eps).
 * The scale index follows the listing (hc_scale[0] for pre, [1] for post,
 * [2] for comb); the page's formula writes the pre scale as s_1, read as
 * 1-based.  The row maximum is subtracted inside the softmax only for
 * numerical safety; the softmax itself is the plain one.  Returns 0, or -1
 * if hc is out of range or iters < 1.
 */
int hco_split_sinkhorn(const double *mixes, const float *scale,
                       const float *base, int64_t n, int hc, int iters,
                       double eps, double *pre, double *post, double *comb)
{
    if (hc < 1 || hc > HCO_MAX_HC || iters < 1)
        return -1;
    const int M = (2 + hc) * hc;
    const double s0 = scale[0], s1 = scale[1], s2 = scale[2];
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        const double *m = mixes + t * M;
        double C[HCO_MAX_HC][HCO_MAX_HC];
        for (int j = 0; j < hc; ++j)
            pre[t * hc + j] = sigmoid(s0 * m[j] + (double)base[j]) + eps;
        for (int j = 0; j < hc; ++j)
            post[t * hc + j] =
                2.0 * sigmoid(s1 * m[hc + j] + (double)base[hc + j]);
        for (int j = 0; j < hc; ++j)
            for (int k = 0; k < hc; ++k)
                C[j][k] = s2 * m[2 * hc + j * hc + k] +
                          (double)base[2 * hc + j * hc + k];
        /* row softmax, then + eps */
        for (int j = 0; j < hc; ++j) {
            double mx = C[j][0];
            for (int k = 1; k < hc; ++k)
                if (C[j][k] > mx)
                    mx = C[j][k];
            double s = 0.0;
            for (int k = 0; k < hc; ++k) {
                C[j][k] = exp(C[j][k] - mx);
                s += C[j][k];
            }
            for (int k = 0; k < hc; ++k)
                C[j][k] = C[j][k] / s + eps;
        }
        col_normalise(C, hc, eps);
        for (int it = 1; it < iters; ++it) {
            row_normalise(C, hc, eps);
            col_normalise(C, hc, eps);
        }
        for (int j = 0; j < hc; ++j)
            for (int k = 0; k < hc; ++k)
                comb[(t * hc + j) * hc + k] = C[j][k];
    }
    return 0;
}

/*
 * [MP] Block.hc_pre: h_c = bf16( sum_k pre_k * R_{k,c} ), the streams
 * collapsed with the pre weights and cast back to the residual's dtype.
 */
void hco_pre(const uint16_t *R, const double *pre, int64_t n, int hc, int d,
             uint16_t *h)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        for (int c = 0; c < d; ++c) {
            double y = 0.0;
            for (int k = 0; k < hc; ++k)
                y += pre[t * hc + k] *
                     hco_bf16_to_double(R[(t * hc + k) * (int64_t)d + c]);
            h[t * (int64_t)d + c] = hco_round_bf16(y);
        }
    }
}

/*
 * [MP] Block.hc_post: output stream k is
 *   R'_{k,c} = bf16( post_k * x_c + sum_j comb[j][k] * R_{j,c} ),
 * i.e. column k of comb feeds output stream k (comb is broadcast over the
 * last axis, the residual over the second-to-last, and the sum runs over
 * the first stream axis).
 */
void hco_post(const uint16_t *x, const uint16_t *R, const double *post,
              const double *comb, int64_t n, int hc, int d, uint16_t *Rout)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        for (int k = 0; k < hc; ++k) {
            for (int c = 0; c < d; ++c) {
                double y = post[t * hc + k] *
                           hco_bf16_to_double(x[t * (int64_t)d + c]);
                for (int j = 0; j < hc; ++j)
                    y += comb[(t * hc + j) * hc + k] *
                         hco_bf16_to_double(R[(t * hc + j) * (int64_t)d + c]);
                Rout[(t * hc + k) * (int64_t)d + c] = hco_round_bf16(y);
            }
        }
    }
}

/*
 * Stand-in sublayer of the chained-stack workload: x_c = bf16(h_c * D_c),
 * a fixed per-layer diagonal scale applied to the hc_pre output.
 */
void hco_diag_scale(const uint16_t *h, const uint16_t *D, int64_t n, int d,
                    uint16_t *x)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t)
        for (int c = 0; c < d; ++c)
            x[t * (int64_t)d + c] = hco_round_bf16(
                hco_bf16_to_double(h[t * (int64_t)d + c]) *
                hco_bf16_to_double(D[c]));
}

/* Number of OpenMP threads a parallel region would use (for reporting). */
int hco_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
