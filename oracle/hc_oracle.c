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
 * high-precision brute force in a different formulation (the backward
 * functions: finite differences of the forward in fp64 and in 40-digit
 * arithmetic, chain-rule identities, scale and shift invariances, and the
 * closed form at W = 0); none is "parity unpinned".
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

/* hco_round_bf16 over an array. */
void hco_round_bf16_array(const double *v, int64_t n, uint16_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = hco_round_bf16(v[i]);
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

/*
 * The pre-sublayer RMSNorm of [MP] Block.__init__ (attn_norm / ffn_norm,
 * RMSNorm(dim, norm_eps)), applied to the bf16 output h of hc_pre.  The
 * pages construct it but print no formula; this is the reading the rest of
 * them supports: the same root-mean-square normalisation as the mix formula
 * (x * rsqrt(mean(x^2) + norm_eps), over the last axis, in float), times a
 * learned per-feature weight gamma[d], the result in h's dtype:
 *   r   = 1 / sqrt( sum_c h_c^2 / d + norm_eps )
 *   y_c = bf16( h_c * r * gamma_c )
 * h_c is the bf16 value (the norm sees hc_pre's stored output); everything
 * is double here and rounded once.
 */
void hco_rmsnorm(const uint16_t *h, const float *gamma, int64_t n, int d,
                 double norm_eps, uint16_t *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        double ss = 0.0;
        for (int c = 0; c < d; ++c) {
            const double v = hco_bf16_to_double(h[t * (int64_t)d + c]);
            ss += v * v;
        }
        const double r = 1.0 / sqrt(ss / (double)d + norm_eps);
        for (int c = 0; c < d; ++c)
            y[t * (int64_t)d + c] = hco_round_bf16(
                hco_bf16_to_double(h[t * (int64_t)d + c]) * r * (double)gamma[c]);
    }
}

/* ====================================================================
 * Backward pass (gradients of a scalar loss through one sublayer's
 * mixing).  The pages give the forward only; its gradient is defined by
 * the chain rule over the forward's steps, taken here in reverse order.
 * The bf16 roundings of h and R' are outputs' storage, not steps of the
 * function: the gradient is that of the real-valued forward (each output
 * before its rounding).  Inputs that the GPU holds in bf16 (R, x and the
 * incoming gradients gRout, gh) come as bf16 patterns; coefficients as
 * double; every result is double.
 * ==================================================================== */

/*
 * Backward of [MP] Block.hc_post, R'_{k,c} = post_k x_c + sum_j comb[j][k] R_{j,c}:
 *   gx[t][c]       = sum_k post_k gRout_{k,c}
 *   gpost[t][k]    = sum_c x_c gRout_{k,c}
 *   gcomb[t][j][k] = sum_c R_{j,c} gRout_{k,c}
 *   gR[t][j][c]    = sum_k comb[j][k] gRout_{k,c}     (hc_post's share of dL/dR)
 */
void hco_post_backward(const uint16_t *x, const uint16_t *R, const double *post,
                       const double *comb, const uint16_t *gRout, int64_t n,
                       int hc, int d, double *gx, double *gpost, double *gcomb,
                       double *gR)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        const uint16_t *xt = x + t * (int64_t)d;
        const uint16_t *Rt = R + t * (int64_t)hc * d;
        const uint16_t *gt = gRout + t * (int64_t)hc * d;
        const double *pt = post + t * hc, *ct = comb + t * hc * hc;
        for (int c = 0; c < d; ++c) {
            double a = 0.0;
            for (int k = 0; k < hc; ++k)
                a += pt[k] * hco_bf16_to_double(gt[(int64_t)k * d + c]);
            gx[t * (int64_t)d + c] = a;
        }
        for (int k = 0; k < hc; ++k) {
            double a = 0.0;
            for (int c = 0; c < d; ++c)
                a += hco_bf16_to_double(xt[c]) *
                     hco_bf16_to_double(gt[(int64_t)k * d + c]);
            gpost[t * hc + k] = a;
        }
        for (int j = 0; j < hc; ++j)
            for (int k = 0; k < hc; ++k) {
                double a = 0.0;
                for (int c = 0; c < d; ++c)
                    a += hco_bf16_to_double(Rt[(int64_t)j * d + c]) *
                         hco_bf16_to_double(gt[(int64_t)k * d + c]);
                gcomb[(t * hc + j) * hc + k] = a;
            }
        for (int j = 0; j < hc; ++j)
            for (int c = 0; c < d; ++c) {
                double a = 0.0;
                for (int k = 0; k < hc; ++k)
                    a += ct[j * hc + k] *
                         hco_bf16_to_double(gt[(int64_t)k * d + c]);
                gR[(t * hc + j) * (int64_t)d + c] = a;
            }
    }
}

/*
 * Backward of [MP] Block.hc_pre, h_c = sum_k pre_k R_{k,c}:
 *   gpre[t][k]  = sum_c gh_c R_{k,c}
 *   gR[t][k][c] = pre_k gh_c                          (hc_pre's share of dL/dR)
 */
void hco_pre_backward(const uint16_t *R, const double *pre, const uint16_t *gh,
                      int64_t n, int hc, int d, double *gpre, double *gR)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        const uint16_t *ght = gh + t * (int64_t)d;
        for (int k = 0; k < hc; ++k) {
            const uint16_t *Rk = R + (t * hc + k) * (int64_t)d;
            double a = 0.0;
            for (int c = 0; c < d; ++c)
                a += hco_bf16_to_double(ght[c]) * hco_bf16_to_double(Rk[c]);
            gpre[t * hc + k] = a;
            for (int c = 0; c < d; ++c)
                gR[(t * hc + k) * (int64_t)d + c] =
                    pre[t * hc + k] * hco_bf16_to_double(ght[c]);
        }
    }
}

/*
 * Backward of one normalisation step Y = X / (s + eps), s the sum of X
 * along the step's axis (rows: axis 1, columns: axis 0).  With Y and the
 * denominators D = s + eps of the forward step:
 *   dY_jk / dX_jl = (delta_kl - Y_jk) / D_j     (a row step; columns alike)
 * so gX = (gY - sum_along(gY * Y)) / D.  g holds gY on entry, gX on exit.
 */
static void normalise_backward(double g[HCO_MAX_HC][HCO_MAX_HC],
                               const double Y[HCO_MAX_HC][HCO_MAX_HC],
                               const double *D, int hc, int rows)
{
    for (int a = 0; a < hc; ++a) {
        double dot = 0.0;
        for (int b = 0; b < hc; ++b)
            dot += rows ? g[a][b] * Y[a][b] : g[b][a] * Y[b][a];
        for (int b = 0; b < hc; ++b) {
            if (rows)
                g[a][b] = (g[a][b] - dot) / D[a];
            else
                g[b][a] = (g[b][a] - dot) / D[a];
        }
    }
}

static double sigmoid_slope(double z)
{
    double s = sigmoid(z);
    return s * (1.0 - s);
}

/*
 * Backward of the [RW] split and epsilon-Sinkhorn (hco_split_sinkhorn),
 * per token.  The forward's matrices after each step are recomputed and
 * kept; then, in reverse order:
 *   each normalisation step: normalise_backward;
 *   "+ eps": the identity;
 *   row softmax P = softmax(L): gL_jk = P_jk (gP_jk - sum_k' gP_jk' P_jk');
 *   the gates and logits, z = s * m + b: gm = s gz, gs = m gz, gb = gz,
 *   with gz = gpre sigma'(z) for pre, gpost * 2 sigma'(z) for post, and
 *   gz = gL for the comb logits.
 * Outputs: gmixes[t][M], and each token's contributions to the scale and
 * base gradients, gscale_tok[t][3] and gbase_tok[t][M] (their sums over
 * tokens are the gradients of hc_scale and hc_base).  Returns 0, or -1 if
 * hc is out of range or iters < 1.
 */
int hco_split_sinkhorn_backward(const double *mixes, const float *scale,
                                const float *base, const double *gpre,
                                const double *gpost, const double *gcomb,
                                int64_t n, int hc, int iters, double eps,
                                double *gmixes, double *gscale_tok,
                                double *gbase_tok)
{
    if (hc < 1 || hc > HCO_MAX_HC || iters < 1)
        return -1;
    const int M = (2 + hc) * hc;
    const double s[3] = {scale[0], scale[1], scale[2]};
    /* normalisation steps after the softmax: one column step, then
     * (iters - 1) pairs of a row and a column step */
    const int nsteps = 2 * iters - 1;
    int bad = 0;
#pragma omp parallel
    {
        /* forward states: Ys[k] after normalisation step k, Ds[k] its denominators */
        double (*Ys)[HCO_MAX_HC][HCO_MAX_HC] =
            malloc(sizeof(*Ys) * (size_t)nsteps);
        double *Ds = malloc(sizeof(double) * (size_t)nsteps * HCO_MAX_HC);
        if (!Ys || !Ds) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(static)
        for (int64_t t = 0; t < n; ++t) {
            if (!Ys || !Ds)
                continue;
            const double *m = mixes + t * M;
            double *gm = gmixes + t * M, *gs = gscale_tok + t * 3,
                   *gb = gbase_tok + t * M;
            gs[0] = gs[1] = gs[2] = 0.0;
            /* gates */
            for (int j = 0; j < hc; ++j) {
                double z = s[0] * m[j] + (double)base[j];
                double gz = gpre[t * hc + j] * sigmoid_slope(z);
                gm[j] = s[0] * gz;
                gs[0] += m[j] * gz;
                gb[j] = gz;
                double y = s[1] * m[hc + j] + (double)base[hc + j];
                double gy = gpost[t * hc + j] * 2.0 * sigmoid_slope(y);
                gm[hc + j] = s[1] * gy;
                gs[1] += m[hc + j] * gy;
                gb[hc + j] = gy;
            }
            /* forward of the comb, keeping every step */
            double P[HCO_MAX_HC][HCO_MAX_HC], X[HCO_MAX_HC][HCO_MAX_HC];
            for (int j = 0; j < hc; ++j) {
                double L[HCO_MAX_HC], mx = -INFINITY, z = 0.0;
                for (int k = 0; k < hc; ++k) {
                    L[k] = s[2] * m[2 * hc + j * hc + k] +
                           (double)base[2 * hc + j * hc + k];
                    if (L[k] > mx)
                        mx = L[k];
                }
                for (int k = 0; k < hc; ++k) {
                    P[j][k] = exp(L[k] - mx);
                    z += P[j][k];
                }
                for (int k = 0; k < hc; ++k) {
                    P[j][k] /= z;
                    X[j][k] = P[j][k] + eps;
                }
            }
            for (int st = 0; st < nsteps; ++st) {
                /* step 0 is a column step; then rows and columns alternate */
                const int rows = st % 2 == 1;
                double *D = Ds + (size_t)st * HCO_MAX_HC;
                for (int a = 0; a < hc; ++a) {
                    double sum = 0.0;
                    for (int b = 0; b < hc; ++b)
                        sum += rows ? X[a][b] : X[b][a];
                    D[a] = sum + eps;
                    for (int b = 0; b < hc; ++b) {
                        if (rows)
                            X[a][b] = X[a][b] / D[a];
                        else
                            X[b][a] = X[b][a] / D[a];
                    }
                }
                memcpy(Ys[st], X, sizeof(X));
            }
            /* reverse */
            double g[HCO_MAX_HC][HCO_MAX_HC];
            for (int j = 0; j < hc; ++j)
                for (int k = 0; k < hc; ++k)
                    g[j][k] = gcomb[(t * hc + j) * hc + k];
            for (int st = nsteps - 1; st >= 0; --st)
                normalise_backward(g, Ys[st], Ds + (size_t)st * HCO_MAX_HC,
                                   hc, st % 2 == 1);
            /* g is now the gradient of P (the "+ eps" passes it through) */
            for (int j = 0; j < hc; ++j) {
                double dot = 0.0;
                for (int k = 0; k < hc; ++k)
                    dot += g[j][k] * P[j][k];
                for (int k = 0; k < hc; ++k) {
                    const int i = 2 * hc + j * hc + k;
                    double gL = P[j][k] * (g[j][k] - dot);
                    gm[i] = s[2] * gL;
                    gs[2] += m[i] * gL;
                    gb[i] = gL;
                }
            }
        }
        free(Ys);
        free(Ds);
    }
    return bad ? -1 : 0;
}

/*
 * Backward of the [MP] mix formula, m_j = r dot_j with dot_j = sum_i W_ji X_i
 * and r = (sum_i X_i^2 / K + norm_eps)^(-1/2), r and dot recomputed from R:
 *   gdot_j = r gm_j
 *   dr/dss = -r^3 / (2K), so gss = -(r^3 / (2K)) sum_j gm_j dot_j
 *   gR[t][i] = sum_j gdot_j W_ji + 2 X_i gss        (the projection's share of dL/dR)
 *   gW[j][i] = sum_t gdot_tj X_ti                   (summed over tokens in order)
 * gR is [n][hc*d] (flattened like the forward), gW is [M][hc*d].
 */
void hco_mixes_backward(const uint16_t *R, const float *W, const double *gmixes,
                        int64_t n, int hc, int d, double norm_eps, double *gR,
                        double *gW)
{
    const int64_t K = (int64_t)hc * d;
    const int M = (2 + hc) * hc;
    double *gdot = malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * M);
    if (!gdot)
        return;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        const uint16_t *x = R + t * K;
        double ss = 0.0;
        for (int64_t i = 0; i < K; ++i) {
            double v = hco_bf16_to_double(x[i]);
            ss += v * v;
        }
        const double r = 1.0 / sqrt(ss / (double)K + norm_eps);
        double gr = 0.0;
        for (int j = 0; j < M; ++j) {
            double dot = 0.0;
            for (int64_t i = 0; i < K; ++i)
                dot += (double)W[(int64_t)j * K + i] * hco_bf16_to_double(x[i]);
            gr += gmixes[t * M + j] * dot;
            gdot[t * M + j] = r * gmixes[t * M + j];
        }
        const double gss = gr * (-(r * r * r) / (2.0 * (double)K));
        for (int64_t i = 0; i < K; ++i) {
            double a = 0.0;
            for (int j = 0; j < M; ++j)
                a += gdot[t * M + j] * (double)W[(int64_t)j * K + i];
            gR[t * K + i] = a + 2.0 * hco_bf16_to_double(x[i]) * gss;
        }
    }
#pragma omp parallel for schedule(static)
    for (int64_t ji = 0; ji < (int64_t)M * K; ++ji) {
        const int j = (int)(ji / K);
        const int64_t i = ji - (int64_t)j * K;
        double a = 0.0;
        for (int64_t t = 0; t < n; ++t)
            a += gdot[t * M + j] * hco_bf16_to_double(R[t * K + i]);
        gW[ji] = a;
    }
    free(gdot);
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
