// hc_backward.hip -- the backward pass of one sublayer's mixing for four
// streams: gradients of a scalar loss through hc_post, hc_pre, the split +
// epsilon-Sinkhorn and the mix projection ("Mix projection" page, the mix
// formula and Block.hc_pre / Block.hc_post; "Reading weights" page, the
// split + Sinkhorn listing).  The pages give the forward; its gradient is the
// chain rule over the forward's steps in reverse order, taken on the
// real-valued forward (the bf16 roundings of h and R' are storage, not
// steps).
//
//  * k_post_bwd (hc_post_backward): one wave per token.  dL/dx (bf16, the
//    exact sum of post_k dL/dR'_k rounded once), and the token's dL/dpost
//    and dL/dcomb, sums over the d features accumulated in double.
//  * k_pre_bwd: one wave per token.  dL/dpre and the sum of squares of the
//    stream (double), then the split + Sinkhorn backward in float: the
//    forward's steps are replayed with the forward kernels' own operations
//    (so pre and comb come out bitwise as the forward's), each step's matrix
//    and reciprocal denominator kept in LDS, and the steps are run backwards.
//    Writes per token the coefficients the next kernel needs (pre, comb,
//    dL/ddot = r dL/dm, and dL/d(sum of squares)) and the token's
//    contributions to dL/dscale and dL/dbase.
//  * k_mix_bwd: dL/dR = sum_k comb[j][k] dL/dR'_k + pre_j dL/dh
//    + sum_m dL/ddot_m W[m][i] + 2 x_i dL/dss, in float, rounded once to
//    bf16; and per token group the partial sums of dL/dW[m][i] =
//    sum_t dL/ddot_tm x_ti.  A workgroup owns 128 features of every stream
//    (wave j: stream j) and walks a contiguous range of tokens; each thread
//    keeps its 2 x 24 weights and 2 x 24 partial sums in registers.
//  * k_gw_reduce, k_sb_partial + k_sb_final: the partial sums over token groups, and the
//    per-token scale and base contributions over tokens, each added in one
//    fixed order (double), so the results are deterministic.
#include "hc_device.hpp"
#include "hc_launch.hpp"

namespace hc {

namespace {

constexpr int kCoef = 48;                   // floats per token in the coefficient record
constexpr int kCPre = 0, kCComb = 4, kCDot = 20, kCSs = 44;
constexpr int kSB = 28;                     // floats per token: dL/dscale (3), dL/dbase (24), pad
constexpr int kBwdMaxIters = 64;
constexpr int kBwdSteps = 2 * kBwdMaxIters - 1;
constexpr int kMixFeat = 128;               // features per stream owned by a k_mix_bwd workgroup
constexpr int kMaxTokenGroups = 32;

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// ------------------------------------------------------------ hc_post bwd
// One wave per token; lane l takes the 8-feature chunks l, l + 64, ...
__global__ __launch_bounds__(256) void k_post_bwd(const u32x4* __restrict__ x, const u32x4* __restrict__ R,
                                                  const float* __restrict__ post, const float* __restrict__ comb,
                                                  const u32x4* __restrict__ gRo, u32x4* __restrict__ gx,
                                                  float* __restrict__ gpost, float* __restrict__ gcomb, int64_t n,
                                                  int d) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= n) return;
    const int d8 = d / 8;
    const double q0 = post[t * kHC], q1 = post[t * kHC + 1], q2 = post[t * kHC + 2], q3 = post[t * kHC + 3];
    double ap[kHC], ac[kHC][kHC];
#pragma unroll
    for (int k = 0; k < kHC; ++k) {
        ap[k] = 0.0;
#pragma unroll
        for (int j = 0; j < kHC; ++j) ac[j][k] = 0.0;
    }
    for (int c8 = lane; c8 < d8; c8 += 64) {
        const u32x4 xv = x[t * d8 + c8];
        u32x4 rv[kHC], gv[kHC];
#pragma unroll
        for (int k = 0; k < kHC; ++k) {
            rv[k] = R[(t * kHC + k) * d8 + c8];
            gv[k] = gRo[(t * kHC + k) * d8 + c8];
        }
        u32x4 out;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t o2[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                auto v = [&](uint32_t word) { return (double)(e ? bf_hi(word) : bf_lo(word)); };
                const double g0 = v(gv[0][w]), g1 = v(gv[1][w]), g2 = v(gv[2][w]), g3 = v(gv[3][w]);
                // dL/dx: exact products in double, one rounding
                double y = q0 * g0;
                y = __builtin_fma(q1, g1, y);
                y = __builtin_fma(q2, g2, y);
                y = __builtin_fma(q3, g3, y);
                o2[e] = bf16_rn_f64(y);
                const double xe = v(xv[w]);
                const double g[kHC] = {g0, g1, g2, g3};
#pragma unroll
                for (int k = 0; k < kHC; ++k) ap[k] = __builtin_fma(xe, g[k], ap[k]);
#pragma unroll
                for (int j = 0; j < kHC; ++j) {
                    const double rj = v(rv[j][w]);
#pragma unroll
                    for (int k = 0; k < kHC; ++k) ac[j][k] = __builtin_fma(rj, g[k], ac[j][k]);
                }
            }
            out[w] = pack2(o2[0], o2[1]);
        }
        gx[t * d8 + c8] = out;
    }
#pragma unroll
    for (int k = 0; k < kHC; ++k) ap[k] = wave_sum_f64(ap[k]);
#pragma unroll
    for (int j = 0; j < kHC; ++j)
#pragma unroll
        for (int k = 0; k < kHC; ++k) ac[j][k] = wave_sum_f64(ac[j][k]);
    if (lane < kHC) {
        double v = ap[0];
#pragma unroll
        for (int k = 1; k < kHC; ++k) v = lane == k ? ap[k] : v;
        gpost[t * kHC + lane] = (float)v;
    }
    if (lane < kHC * kHC) {
        double v = 0.0;
#pragma unroll
        for (int j = 0; j < kHC; ++j)
#pragma unroll
            for (int k = 0; k < kHC; ++k) v = lane == j * kHC + k ? ac[j][k] : v;
        gcomb[t * kHC * kHC + lane] = (float)v;
    }
}

// ------------------------------------------ hc_pre + split + Sinkhorn bwd
struct PreBwdArgs {
    const u32x4* R;
    const u32x4* gh;
    const float* mixes;
    const float* scale;
    const float* base;
    const float* gpost;
    const float* gcomb;
    float* coef;        // [n][kCoef]
    float* sb;          // [n][kSB]
    float* gmixes;      // [n][24] or null
    int64_t n;
    int d;
    int iters;
    float eps;
    float norm_eps;
};

// One wave per token: dL/dpre and the sum of squares over the d features
// (double), then the split + Sinkhorn backward of the token in every 16-lane
// row of the wave (the rows compute the same values; row 0 writes).
__global__ __launch_bounds__(256) void k_pre_bwd(PreBwdArgs a) {
    __shared__ float2 st[4][kBwdSteps][16];     // per wave: each step's value and 1 / (sum + eps)
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + wv;
    if (t >= a.n) return;
    const int d8 = a.d / 8;
    double gp[kHC] = {0.0, 0.0, 0.0, 0.0}, ss = 0.0;
    for (int c8 = lane; c8 < d8; c8 += 64) {
        const u32x4 hv = a.gh[t * d8 + c8];
#pragma unroll
        for (int k = 0; k < kHC; ++k) {
            const u32x4 rv = a.R[(t * kHC + k) * d8 + c8];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const double r0 = bf_lo(rv[w]), r1 = bf_hi(rv[w]);
                gp[k] = __builtin_fma((double)bf_lo(hv[w]), r0, gp[k]);
                gp[k] = __builtin_fma((double)bf_hi(hv[w]), r1, gp[k]);
                ss = __builtin_fma(r0, r0, ss);
                ss = __builtin_fma(r1, r1, ss);
            }
        }
    }
#pragma unroll
    for (int k = 0; k < kHC; ++k) gp[k] = wave_sum_f64(gp[k]);
    ss = wave_sum_f64(ss);

    // split + Sinkhorn, forward replayed with the forward kernels' operations
    const int e = lane & 15, j4 = e & 3;
    const float* m = a.mixes + t * kMix;
    const float s0 = a.scale[0], s1 = a.scale[1], s2 = a.scale[2];
    const float* base = a.base;
    const float mp = m[j4], mq = m[kHC + j4], mc = m[2 * kHC + e];
    const float sg_pre = sigmoidf_(mp * s0 + base[j4]);
    const float pre = sg_pre + a.eps;                            // pre_gate's value
    const float sg_post = sigmoidf_(mq * s1 + base[kHC + j4]);
    float c = mc * s2 + base[2 * kHC + e];
    const float mx = quad_max(c);
    const float ex = expf(c - mx);
    const float rsum = quad_sum(ex);
    const float P = ex / rsum;
    c = P + a.eps;
    const int nsteps = 2 * a.iters - 1;
    float2* S = &st[wv][0][0];
    {
        const float r = __builtin_amdgcn_rcpf(col4_sum(c) + a.eps);
        c = c * r;
        S[e] = make_float2(c, r);
    }
    for (int it = 1; it < a.iters; ++it) {
        float r = __builtin_amdgcn_rcpf(quad_sum(c) + a.eps);
        c = c * r;
        S[(2 * it - 1) * 16 + e] = make_float2(c, r);
        r = __builtin_amdgcn_rcpf(col4_sum(c) + a.eps);
        c = c * r;
        S[(2 * it) * 16 + e] = make_float2(c, r);
    }
    const float comb = c;
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");     // the wave reads back its own LDS writes
    // backward through the normalisations: gX = (gY - sum_along(gY Y)) / D
    float g = a.gcomb[t * kHC * kHC + e];
    for (int s = nsteps - 1; s >= 0; --s) {
        const float2 yr = S[s * 16 + e];
        const float gy = g * yr.x;
        const float dot = (s & 1) ? quad_sum(gy) : col4_sum(gy);     // odd steps are row steps
        g = (g - dot) * yr.y;
    }
    // "+ eps" passes the gradient through; the row softmax:
    // gL = P (gP - sum_k gP P)
    const float gL = P * (g - quad_sum(g * P));
    // gates: pre = sigma(z) + eps, post = 2 sigma(z); z = s m + b
    double gpe = gp[0];
#pragma unroll
    for (int k = 1; k < kHC; ++k) gpe = j4 == k ? gp[k] : gpe;
    const float gz_pre = (float)gpe * (sg_pre * (1.0f - sg_pre));
    const float gz_post = a.gpost[t * kHC + j4] * (2.0f * (sg_post * (1.0f - sg_post)));
    const float gm_pre = s0 * gz_pre, gm_post = s1 * gz_post, gm_c = s2 * gL;
    // dL/dm . m over the 24 mixes, and the scale contributions
    const bool lo4 = e < kHC;
    const float dm = gm_c * mc + (lo4 ? gm_pre * mp + gm_post * mq : 0.0f);
    const float sum_dm = col4_sum(quad_sum(dm));
    const float gs0 = col4_sum(quad_sum(lo4 ? mp * gz_pre : 0.0f));
    const float gs1 = col4_sum(quad_sum(lo4 ? mq * gz_post : 0.0f));
    const float gs2 = col4_sum(quad_sum(mc * gL));
    // r = (ss / K + norm_eps)^-1/2; m = r dot, so dL/ddot = r dL/dm and
    // dL/dss = -(r^3 / 2K) sum_j dL/dm_j dot_j = -(r^2 / 2K) sum_j dL/dm_j m_j
    const double Kd = (double)(kHC * a.d);
    const double r2 = 1.0 / (ss / Kd + (double)a.norm_eps);
    const float r = (float)__builtin_sqrt(r2);
    const float gss = (float)(-(r2 / (2.0 * Kd)) * (double)sum_dm);
    if (lane < 16) {
        float* cf = a.coef + t * kCoef;
        cf[kCComb + e] = comb;
        cf[kCDot + 2 * kHC + e] = r * gm_c;
        float* sb = a.sb + t * kSB;
        sb[3 + 2 * kHC + e] = gL;
        if (a.gmixes) a.gmixes[t * kMix + 2 * kHC + e] = gm_c;
        if (lo4) {
            cf[kCPre + e] = pre;
            cf[kCDot + e] = r * gm_pre;
            cf[kCDot + kHC + e] = r * gm_post;
            sb[3 + e] = gz_pre;
            sb[3 + kHC + e] = gz_post;
            if (a.gmixes) {
                a.gmixes[t * kMix + e] = gm_pre;
                a.gmixes[t * kMix + kHC + e] = gm_post;
            }
        }
        if (e == 0) {
            cf[kCSs] = gss;
            sb[0] = gs0;
            sb[1] = gs1;
            sb[2] = gs2;
        }
    }
}

// --------------------------------------------------- projection bwd (dL/dR)
struct MixBwdArgs {
    const uint32_t* R;      // bf16 pairs
    const uint32_t* gh;
    const uint32_t* gRo;
    const float* W;
    const float* coef;
    uint32_t* gR;
    float* part;            // [NTG][24][K] partial dL/dW
    int64_t n;
    int d;
    int ntg;                // token groups
};

// Workgroup (feature block fb, token group tg): wave j owns features
// fb * 128 + 2 lane, +1 of stream j.
__global__ __launch_bounds__(256) void k_mix_bwd(MixBwdArgs a) {
    const int nfb = a.d / kMixFeat;
    const int fb = blockIdx.x % nfb, tg = blockIdx.x / nfb;
    const int j = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int c0 = fb * kMixFeat + 2 * lane;
    const int64_t K = (int64_t)kHC * a.d;
    const int64_t i0 = (int64_t)j * a.d + c0;
    const int64_t per = (a.n + a.ntg - 1) / a.ntg;
    const int64_t t0 = per * tg, t1 = t0 + per < a.n ? t0 + per : a.n;
    float w[kMix][2], acc[kMix][2];
#pragma unroll
    for (int mm = 0; mm < kMix; ++mm) {
        const float2 wv = *reinterpret_cast<const float2*>(a.W + mm * K + i0);
        w[mm][0] = wv.x;
        w[mm][1] = wv.y;
        acc[mm][0] = acc[mm][1] = 0.0f;
    }
    const int d2 = a.d / 2;          // bf16 pairs per row
    for (int64_t t = t0; t < t1; ++t) {
        const float* cf = a.coef + t * kCoef;
        const uint32_t xw = a.R[(t * kHC + j) * d2 + c0 / 2];
        const uint32_t hw = a.gh[t * d2 + c0 / 2];
        uint32_t gw[kHC];
#pragma unroll
        for (int k = 0; k < kHC; ++k) gw[k] = a.gRo[(t * kHC + k) * d2 + c0 / 2];
        const float pj = cf[kCPre + j], gss2 = 2.0f * cf[kCSs];
        float cb[kHC];
#pragma unroll
        for (int k = 0; k < kHC; ++k) cb[k] = cf[kCComb + j * kHC + k];
        float gd[kMix];
#pragma unroll
        for (int mm = 0; mm < kMix; ++mm) gd[mm] = cf[kCDot + mm];
        uint32_t o[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            auto v = [&](uint32_t word) { return e ? bf_hi(word) : bf_lo(word); };
            const float xe = v(xw);
            float y = cb[0] * v(gw[0]);
#pragma unroll
            for (int k = 1; k < kHC; ++k) y = __builtin_fmaf(cb[k], v(gw[k]), y);
            y = __builtin_fmaf(pj, v(hw), y);
#pragma unroll
            for (int mm = 0; mm < kMix; ++mm) y = __builtin_fmaf(gd[mm], w[mm][e], y);
            y = __builtin_fmaf(gss2, xe, y);
            o[e] = bf16_rn(y);
#pragma unroll
            for (int mm = 0; mm < kMix; ++mm) acc[mm][e] = __builtin_fmaf(gd[mm], xe, acc[mm][e]);
        }
        a.gR[(t * kHC + j) * d2 + c0 / 2] = pack2(o[0], o[1]);
    }
    float* P = a.part + (int64_t)tg * kMix * K;
#pragma unroll
    for (int mm = 0; mm < kMix; ++mm)
        *reinterpret_cast<float2*>(P + mm * K + i0) = make_float2(acc[mm][0], acc[mm][1]);
}

// dL/dW[m][i] = sum over token groups of the partials, in group order.
__global__ __launch_bounds__(256) void k_gw_reduce(const float* __restrict__ part, float* __restrict__ gW,
                                                   int64_t total, int ntg) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        double s = 0.0;
        for (int g = 0; g < ntg; ++g) s += (double)part[(int64_t)g * total + i];
        gW[i] = (float)s;
    }
}

// The per-token [n][kSB] scale and base contributions summed over tokens,
// in two fixed-order stages: block b stages its contiguous range of up to
// 256 tokens in LDS (every load in flight at once) and lane c adds column c
// over them in token order; then one wave adds the blocks' sums in block
// order.
constexpr int kSbBlocks = 256;
__global__ __launch_bounds__(256) void k_sb_partial(const float* __restrict__ sb, double* __restrict__ part,
                                                    int64_t n) {
    __shared__ __attribute__((aligned(16))) float rows[256][kSB];
    const int64_t per = (n + kSbBlocks - 1) / kSbBlocks;
    const int64_t t0 = per * blockIdx.x, t1 = t0 + per < n ? t0 + per : n;
    double s = 0.0;
    for (int64_t c0 = t0; c0 < t1; c0 += 256) {
        const int cnt = (int)(t1 - c0 < 256 ? t1 - c0 : 256);
        if ((int)threadIdx.x < cnt) {
            const f32x4* src = reinterpret_cast<const f32x4*>(sb + (c0 + threadIdx.x) * kSB);
#pragma unroll
            for (int q = 0; q < kSB / 4; ++q) *reinterpret_cast<f32x4*>(&rows[threadIdx.x][4 * q]) = src[q];
        }
        __syncthreads();
        if ((int)threadIdx.x < kSB)
            for (int i = 0; i < cnt; ++i) s += (double)rows[i][threadIdx.x];
        __syncthreads();
    }
    if ((int)threadIdx.x < kSB) part[blockIdx.x * kSB + threadIdx.x] = s;
}
__global__ __launch_bounds__(256) void k_sb_final(const double* __restrict__ part, float* __restrict__ gscale,
                                                  float* __restrict__ gbase) {
    __shared__ double sums[kSbBlocks][kSB];
    for (int i = threadIdx.x; i < kSbBlocks * kSB; i += 256) (&sums[0][0])[i] = part[i];
    __syncthreads();
    const int c = threadIdx.x;
    if (c >= 3 + kMix) return;
    double s = 0.0;
    for (int b = 0; b < kSbBlocks; ++b) s += sums[b][c];
    if (c < 3) gscale[c] = (float)s;
    else gbase[c - 3] = (float)s;
}

int token_groups(int64_t n) {
    int64_t g = (n + 255) / 256;
    if (g > kMaxTokenGroups) g = kMaxTokenGroups;
    return (int)(g < 1 ? 1 : g);
}

size_t al256(size_t b) { return (b + 255) & ~(size_t)255; }

}  // namespace

bool bwd_supported(int hc_, int d, int iters) {
    return hc_ == kHC && d > 0 && d % kMixFeat == 0 && iters >= 1 && iters <= kBwdMaxIters;
}

size_t bwd_ws_bytes(int64_t n, int d) {
    const int64_t K = (int64_t)kHC * d;
    return al256((size_t)n * kCoef * 4) + al256((size_t)n * kSB * 4) +
           al256((size_t)token_groups(n) * kMix * K * 4) + al256((size_t)kSbBlocks * kSB * 8);
}

int launch_post_bwd(const void* x, const void* R, const float* post, const float* comb, const void* gRo, void* gx,
                    float* gpost, float* gcomb, int64_t n, int d, hipStream_t s) {
    const int64_t blocks = (n + 3) / 4;
    k_post_bwd<<<(unsigned)blocks, 256, 0, s>>>((const u32x4*)x, (const u32x4*)R, post, comb, (const u32x4*)gRo,
                                                (u32x4*)gx, gpost, gcomb, n, d);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_mix_pre_bwd(const void* R, const float* W, const float* scale, const float* base, const float* mixes,
                       const void* gh, const void* gRo, const float* gpost, const float* gcomb, void* gR, float* gW,
                       float* gscale, float* gbase, float* gmixes, void* ws, int64_t n, int d, int iters, float eps,
                       float norm_eps, hipStream_t s) {
    const int64_t K = (int64_t)kHC * d;
    char* w = static_cast<char*>(ws);
    float* coef = reinterpret_cast<float*>(w);
    float* sb = reinterpret_cast<float*>(w + al256((size_t)n * kCoef * 4));
    float* part = reinterpret_cast<float*>(w + al256((size_t)n * kCoef * 4) + al256((size_t)n * kSB * 4));
    double* sbp = reinterpret_cast<double*>(w + al256((size_t)n * kCoef * 4) + al256((size_t)n * kSB * 4) +
                                            al256((size_t)token_groups(n) * kMix * K * 4));
    PreBwdArgs pa{(const u32x4*)R, (const u32x4*)gh, mixes, scale, base, gpost, gcomb, coef, sb, gmixes, n, d,
                  iters, eps, norm_eps};
    k_pre_bwd<<<(unsigned)((n + 3) / 4), 256, 0, s>>>(pa);
    if (hipGetLastError() != hipSuccess) return -1;
    const int ntg = token_groups(n);
    MixBwdArgs ma{(const uint32_t*)R, (const uint32_t*)gh, (const uint32_t*)gRo, W, coef, (uint32_t*)gR, part, n, d,
                  ntg};
    k_mix_bwd<<<(unsigned)((d / kMixFeat) * ntg), 256, 0, s>>>(ma);
    if (hipGetLastError() != hipSuccess) return -1;
    const int64_t total = kMix * K;
    int64_t blocks = (total + 255) / 256;
    if (blocks > (int64_t)num_cus() * 8) blocks = (int64_t)num_cus() * 8;
    k_gw_reduce<<<(unsigned)blocks, 256, 0, s>>>(part, gW, total, ntg);
    if (hipGetLastError() != hipSuccess) return -1;
    k_sb_partial<<<kSbBlocks, 256, 0, s>>>(sb, sbp, n);
    if (hipGetLastError() != hipSuccess) return -1;
    k_sb_final<<<1, 256, 0, s>>>(sbp, gscale, gbase);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace hc
