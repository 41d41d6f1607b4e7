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
//    sum_t dL/ddot_tm x_ti.  Both sums over the mixes run on the matrix
//    cores from exact bf16 pieces of the fp32 operands; a workgroup owns 128
//    features of every stream and walks a contiguous range of tokens in
//    rounds of 32.
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
constexpr int kMixFeat = 128;               // the backward takes widths d that are multiples of this
constexpr int kMaxTokenGroups = 32;
constexpr int kBufDword3 = 0x00020000;      // raw buffer resource, dword 3
constexpr int kBufOOB = 0x7FFFFFF0;         // buffer offset past every resource: loads read 0

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
    // the next chunk's loads are in flight while this one is computed
    // (non-temporal: every input is read once); past the row's end the last
    // chunk is loaded again, with no branch around the loads
    struct Chunk {
        u32x4 xv, rv[kHC], gv[kHC];
    };
    auto fetch = [&](int c8, Chunk& C) {
        const int c = c8 < d8 ? c8 : d8 - 1;
        C.xv = __builtin_nontemporal_load(x + t * d8 + c);
#pragma unroll
        for (int k = 0; k < kHC; ++k) {
            C.rv[k] = __builtin_nontemporal_load(R + (t * kHC + k) * d8 + c);
            C.gv[k] = __builtin_nontemporal_load(gRo + (t * kHC + k) * d8 + c);
        }
    };
    Chunk cur, nxt;
    if (lane < d8) fetch(lane, cur);
    for (int c8 = lane; c8 < d8; c8 += 64) {
        fetch(c8 + 64, nxt);
        const u32x4 xv = cur.xv;
        const u32x4(&rv)[kHC] = cur.rv;
        const u32x4(&gv)[kHC] = cur.gv;
        // dL/dx: exact products in double, one rounding (through the float
        // rounding unless a lane of the wave hit a halfway point)
        double ys[4][2];
        float fs[4][2];
        bool mid = false;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                auto v = [&](uint32_t word) { return (double)(e ? bf_hi(word) : bf_lo(word)); };
                const double g0 = v(gv[0][w]), g1 = v(gv[1][w]), g2 = v(gv[2][w]), g3 = v(gv[3][w]);
                double y = q0 * g0;
                y = __builtin_fma(q1, g1, y);
                y = __builtin_fma(q2, g2, y);
                y = __builtin_fma(q3, g3, y);
                ys[w][e] = y;
                fs[w][e] = f32_mid(y, mid);
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
        }
        u32x4 out;
        if (__builtin_amdgcn_ballot_w64(mid)) {
#pragma unroll
            for (int w = 0; w < 4; ++w) out[w] = pack2(bf16_rn_f64(ys[w][0]), bf16_rn_f64(ys[w][1]));
        } else {
#pragma unroll
            for (int w = 0; w < 4; ++w) out[w] = pack2(bf16_rn(fs[w][0]), bf16_rn(fs[w][1]));
        }
        __builtin_nontemporal_store(out, gx + t * d8 + c8);
        cur = nxt;
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
    // the next chunk's loads are in flight while this one is summed (few
    // waves fit beside the step table in LDS, so latency would show);
    // non-temporal, and past the row's end the last chunk is loaded again
    struct Chunk {
        u32x4 hv, rv[kHC];
    };
    auto fetch = [&](int c8, Chunk& C) {
        const int c = c8 < d8 ? c8 : d8 - 1;
        C.hv = __builtin_nontemporal_load(a.gh + t * d8 + c);
#pragma unroll
        for (int k = 0; k < kHC; ++k) C.rv[k] = __builtin_nontemporal_load(a.R + (t * kHC + k) * d8 + c);
    };
    Chunk cur, nxt;
    if (lane < d8) fetch(lane, cur);
    for (int c8 = lane; c8 < d8; c8 += 64) {
        fetch(c8 + 64, nxt);
        const u32x4 hv = cur.hv;
#pragma unroll
        for (int k = 0; k < kHC; ++k) {
            const u32x4 rv = cur.rv[k];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const double r0 = bf_lo(rv[w]), r1 = bf_hi(rv[w]);
                gp[k] = __builtin_fma((double)bf_lo(hv[w]), r0, gp[k]);
                gp[k] = __builtin_fma((double)bf_hi(hv[w]), r1, gp[k]);
                ss = __builtin_fma(r0, r0, ss);
                ss = __builtin_fma(r1, r1, ss);
            }
        }
        cur = nxt;
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
    const uint16_t* R;
    const uint16_t* gh;
    const uint16_t* gRo;
    const float* W;
    const float* coef;
    uint16_t* gR;
    float* part;            // [NTG][24][K] partial dL/dW
    int64_t n;
    int d;
    int ntg;                // token groups
};

// The two contractions over the 24 mixes run on the matrix cores
// (v_mfma_f32_16x16x32_bf16, mixes padded to 32 with zeros): fp32 operands
// are split exactly into three bf16 pieces (a float's 24-bit significand is
// three 8-bit ones), so every product below is an exact product of pieces.
//  * sum_m dL/ddot[t][m] W[m][i]: rows = 16 tokens, columns = 16 features,
//    reduction = the mixes.  Both operands are split; the six products of
//    pieces whose weight is at least 2^-16 of the leading one are summed,
//    the three dropped ones are below 2^-23 of it.
//  * dL/dW[m][i] += sum_t dL/ddot[t][m] x[t][i]: rows = 16 mixes, columns =
//    16 features, reduction = the round's 32 tokens; x is bf16 already, so
//    the three pieces of dL/ddot give the products exactly.
// A workgroup owns F features of every stream (F = 128: 256-byte row
// segments) and walks its token group in rounds of kMbT tokens.  Per round: every thread has loaded (two
// rounds ahead) one 8-feature chunk of one token from each stream of R and
// dL/dR' and from dL/dh; the round's residual goes to LDS transposed
// (feature-major, the MFMA operand order for a reduction over tokens) with
// its coefficient records; each thread puts its chunk's four-term comb sum,
// pre_j dL/dh and 2 x dL/dss in LDS (after which its registers take the
// loads of the round two ahead); each wave adds the products of one
// stream's 64 features to those sums on the matrix cores; then each thread
// stores its chunk's dL/dR, rounded once to bf16.
constexpr int kMbT = 32;                         // tokens per round
constexpr int kXtRow = 80;                       // bytes per feature row of the transposed residual (32 tokens + pad)

// H = 1 or 2: a workgroup of 256 H threads owns F = 64 H features of every
// stream; wave w runs the products of stream w % 4, features 64 (w / 4) ..
template <int H>
struct MbGeo {
    static constexpr int F = 64 * H;                        // features per stream of a workgroup
    static constexpr int kThreads = 256 * H;
    static constexpr int kXtStream = F * kXtRow + 16 * (F / 8);   // one stream, with a 16-byte skew per 8 features
    static constexpr int kDrTok = kHC * F + 4;              // floats per token row of the matrix-core sums (+ pad)
    static constexpr int kCfLoads = (kMbT * kCoef / 4 + kThreads - 1) / kThreads;   // record float4s per thread
};

template <int H>
struct MbLds {
    uint8_t xt[kHC * MbGeo<H>::kXtStream];       // x transposed: [stream][feature][token] bf16
    float cf[2][kMbT][kCoef];                    // the round's coefficient records (by round parity)
    float dr[kMbT][MbGeo<H>::kDrTok];            // the round's sum_m dL/ddot_m W[m][i], fp32
};

// Byte offset of (stream j, feature f, token t) in MbLds::xt.  The pad and
// the skew keep both the transposing 2-byte stores (8 chunks x 8 tokens of
// a wave) and the 16-byte operand reads (16 features) on distinct banks.
template <int H>
__device__ __forceinline__ int xt_off(int j, int f, int t) {
    return j * MbGeo<H>::kXtStream + f * kXtRow + (f >> 3) * 16 + 2 * t;
}

// v = hi + mid + lo exactly, each piece bf16.
__device__ __forceinline__ void split3(const float (&v)[8], bf16x8& hi, bf16x8& mid, bf16x8& lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const __bf16 h = (__bf16)v[e];
        const float r1 = v[e] - (float)h;
        const __bf16 m = (__bf16)r1;
        hi[e] = h;
        mid[e] = m;
        lo[e] = (__bf16)(r1 - (float)m);
    }
}

// A barrier for LDS only: this wave's LDS accesses complete, then the
// workgroup barrier; global loads issued before it stay in flight.  In
// assembly with a memory clobber, so the compiler moves no memory access
// across it (an LDS-scoped fence pair around the barrier builtin let the
// stores of MFMA results sink below the barrier).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One round's global inputs for one thread: chunk ic of token it.
template <int H>
struct MbIo {
    u32x4 x[kHC], g[kHC], h;
    f32x4 c[MbGeo<H>::kCfLoads];                 // the round's coefficient float4s tid, tid + threads, ..
};

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Workgroup (feature block fb, token group tg).
template <int H>
__global__ __launch_bounds__(256 * H, H == 1 ? 2 : 1) void k_mix_bwd(MixBwdArgs a) {
    using G = MbGeo<H>;
    constexpr int kMbF = G::F, kDrTok = G::kDrTok;
    __shared__ __attribute__((aligned(16))) MbLds<H> L;
    const int nfb = a.d / kMbF;
    const int fb = blockIdx.x % nfb, tg = blockIdx.x / nfb;
    const int tid = threadIdx.x, l = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = wv & 3, mc = 64 * (wv >> 2);   // matrix-core work: stream j, features mc .. mc + 63
    const int row = l & 15, grp = l >> 4;
    const int col0 = fb * kMbF;
    const int d = a.d;
    const int64_t K = (int64_t)kHC * d;
    const int64_t per = (a.n + a.ntg - 1) / a.ntg;
    const int64_t t0 = per * tg, t1 = t0 + per < a.n ? t0 + per : a.n;
    const int nr = t1 > t0 ? (int)((t1 - t0 + kMbT - 1) / kMbT) : 0;

    // stream j's weights for features col0 + mc .. + 63 as B fragments:
    // column tile ct, lane (row, grp) = feature 16 ct + row, mixes 8 grp ..
    bf16x8 wh[4], wm[4], wl[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
        const int64_t i = (int64_t)j * d + col0 + mc + 16 * ct + row;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int m = 8 * grp + e;
            v[e] = m < kMix ? a.W[m * K + i] : 0.0f;
        }
        split3(v, wh[ct], wm[ct], wl[ct]);
    }
    f32x4 gw[2][4];                              // dL/dW sums: mix tile, column tile
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) gw[mt][ct] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const int it = tid / (8 * H), ic = tid % (8 * H);   // streaming item: token it of the round, features 8 ic ..
    // the round's rows as buffer resources: tokens r0 .. r0 + 31 of the
    // group; rows past the group's end lie outside the resource, so their
    // loads return zeros and their stores are dropped
    auto rows = [&](const void* base, int64_t tok_bytes, int64_t r0) {
        int64_t valid = t1 - r0;
        valid = valid < 0 ? 0 : (valid > kMbT ? kMbT : valid);
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(static_cast<const char*>(base)) + r0 * tok_bytes,
                                                 0, (int)(valid * tok_bytes), kBufDword3);
    };
    const int ox = (it * kHC * d + col0 + 8 * ic) * 2;          // stream 0 of the item in a round of R, dL/dR'
    const int oh = (it * d + col0 + 8 * ic) * 2;                // the item in a round of dL/dh
    auto load = [&](MbIo<H>& io, int64_t r0) {
        const __amdgpu_buffer_rsrc_t rx = rows(a.R, (int64_t)kHC * d * 2, r0);
        const __amdgpu_buffer_rsrc_t rg = rows(a.gRo, (int64_t)kHC * d * 2, r0);
        const __amdgpu_buffer_rsrc_t rh = rows(a.gh, (int64_t)d * 2, r0);
        const __amdgpu_buffer_rsrc_t rc = rows(a.coef, kCoef * 4, r0);
        // the streams non-temporal (aux 2): each is read once; the records
        // are read by every feature block and stay cached
#pragma unroll
        for (int k = 0; k < kHC; ++k) {
            io.x[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, ox, k * d * 2, 2));
            io.g[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, ox, k * d * 2, 2));
        }
        io.h = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rh, oh, 0, 2));
#pragma unroll
        for (int u = 0; u < G::kCfLoads; ++u) {
            const int q = tid + G::kThreads * u;                 // float4 q of the round's records
            io.c[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    rc, q < kMbT * kCoef / 4 ? 16 * q : kBufOOB, 0, 0));
        }
    };
    // stage A: the round's residual transposed into xt, its records into cf
    auto stage_a = [&](const MbIo<H>& io, int pb) {
#pragma unroll
        for (int k = 0; k < kHC; ++k)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t word = io.x[k][w];
                *reinterpret_cast<uint16_t*>(&L.xt[xt_off<H>(k, 8 * ic + 2 * w, it)]) = (uint16_t)word;
                *reinterpret_cast<uint16_t*>(&L.xt[xt_off<H>(k, 8 * ic + 2 * w + 1, it)]) = (uint16_t)(word >> 16);
            }
#pragma unroll
        for (int u = 0; u < G::kCfLoads; ++u) {
            const int q = tid + G::kThreads * u;
            if (q < kMbT * kCoef / 4) *reinterpret_cast<f32x4*>(&L.cf[pb][q / 12][4 * (q % 12)]) = io.c[u];
        }
    };
    // stage B: the item's terms outside the matrix cores, for every stream
    // j: sum_k comb[j][k] dL/dR'_k + pre_j dL/dh + 2 dL/dss x_j, into dr
    auto stage_b = [&](const MbIo<H>& io, int pb) {
        const float* c = &L.cf[pb][it][0];
        const float gss2 = 2.0f * c[kCSs];
#pragma unroll
        for (int jj = 0; jj < kHC; ++jj) {
            const float pj = c[kCPre + jj];
            float cb[kHC];
#pragma unroll
            for (int k = 0; k < kHC; ++k) cb[k] = c[kCComb + jj * kHC + k];
            float y[8];
#pragma unroll
            for (int w = 0; w < 4; ++w)
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    auto v = [&](uint32_t word) { return e ? bf_hi(word) : bf_lo(word); };
                    float acc = cb[0] * v(io.g[0][w]);
#pragma unroll
                    for (int k = 1; k < kHC; ++k) acc = __builtin_fmaf(cb[k], v(io.g[k][w]), acc);
                    acc = __builtin_fmaf(pj, v(io.h[w]), acc);
                    y[2 * w + e] = __builtin_fmaf(gss2, v(io.x[jj][w]), acc);
                }
            *reinterpret_cast<f32x4*>(&L.dr[it][jj * kMbF + 8 * ic]) = f32x4{y[0], y[1], y[2], y[3]};
            *reinterpret_cast<f32x4*>(&L.dr[it][jj * kMbF + 8 * ic + 4]) = f32x4{y[4], y[5], y[6], y[7]};
        }
    };
    auto mma = [&](int pb) {
        // dr += sum_m dL/ddot[t][m] W[m][i]: A = 16 tokens x mixes 8 grp .. 8 grp + 7
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            float v[8];
            if (grp < 3) {
                const float* src = &L.cf[pb][16 * tt + row][kCDot + 8 * grp];
                const f32x4 lo4 = *reinterpret_cast<const f32x4*>(src), hi4 = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[e] = lo4[e];
                    v[4 + e] = hi4[e];
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = 0.0f;
            }
            bf16x8 ah, am, al;
            split3(v, ah, am, al);
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                float* dst = &L.dr[16 * tt + 4 * grp][j * kMbF + mc + 16 * ct + row];
                f32x4 c;
#pragma unroll
                for (int i = 0; i < 4; ++i) c[i] = dst[i * kDrTok];
                c = mfma16(am, wm[ct], c);
                c = mfma16(al, wh[ct], c);
                c = mfma16(ah, wl[ct], c);
                c = mfma16(am, wh[ct], c);
                c = mfma16(ah, wm[ct], c);
                c = mfma16(ah, wh[ct], c);
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[i * kDrTok] = c[i];
            }
        }
        // dL/dW[m][i] += sum_t dL/ddot[t][m] x[t][i]: A = mixes 16 mt + row x
        // tokens 8 grp .. 8 grp + 7, B = the transposed residual
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const int mix = 16 * mt + row;
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = mix < kMix ? L.cf[pb][8 * grp + e][kCDot + mix] : 0.0f;
            bf16x8 gh_, gm_, gl_;
            split3(v, gh_, gm_, gl_);
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                const bf16x8 xb = *reinterpret_cast<const bf16x8*>(&L.xt[xt_off<H>(j, mc + 16 * ct + row, 8 * grp)]);
                gw[mt][ct] = mfma16(gl_, xb, gw[mt][ct]);
                gw[mt][ct] = mfma16(gm_, xb, gw[mt][ct]);
                gw[mt][ct] = mfma16(gh_, xb, gw[mt][ct]);
            }
        }
    };
    // dL/dR of the item, rounded once to bf16
    auto emit = [&](int64_t r0) {
        const __amdgpu_buffer_rsrc_t ro = rows(a.gR, (int64_t)kHC * d * 2, r0);
#pragma unroll
        for (int jj = 0; jj < kHC; ++jj) {
            const f32x4 d0 = *reinterpret_cast<const f32x4*>(&L.dr[it][jj * kMbF + 8 * ic]);
            const f32x4 d1 = *reinterpret_cast<const f32x4*>(&L.dr[it][jj * kMbF + 8 * ic + 4]);
            const u32x2 o0 = u32x2{bf16x2_rn(d0[0], d0[1]), bf16x2_rn(d0[2], d0[3])};
            const u32x2 o1 = u32x2{bf16x2_rn(d1[0], d1[1]), bf16x2_rn(d1[2], d1[3])};
            // two 8-byte stores, not one of 16: with the wider store, a
            // 64-bit move into its data registers a few instructions later
            // (the compiler's loop code) was seen to reach the data of lanes
            // 12..15 of every 16 before the store had read it.  The data
            // registers are also held, unwritten, through a few wait states.
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((__vector_size__(8))) int, o0), ro,
                                                  ox, jj * d * 2, 2);
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((__vector_size__(8))) int, o1), ro,
                                                  ox + 8, jj * d * 2, 2);
            asm volatile("s_nop 7" ::"v"(o0), "v"(o1) : "memory");     // (stores non-temporal: written once)
        }
    };
    // round r: its inputs (loaded two rounds ahead) go to LDS and are
    // consumed there, so their registers take round r + 2's loads at once;
    // then the products, then the outputs.  LDS: xt and cf (by parity) are
    // rewritten only after the barrier that follows the products reading
    // them; dr after the first barrier of the next round, which follows the
    // outputs reading it.  Every round issues the same memory instructions
    // (rounds past the group's end lie outside their resources: zeros in,
    // stores dropped), so the loop body is straight-line and the compiler's
    // memory-counter waits let the next round's loads stay in flight.
    auto round = [&](MbIo<H>& io, int r, int pb) {
        stage_a(io, pb);
        lds_barrier();
        stage_b(io, pb);
        load(io, t0 + (int64_t)(r + 2) * kMbT);
        lds_barrier();
        mma(pb);
        lds_barrier();
        emit(t0 + (int64_t)r * kMbT);
    };
    // stores outside every resource, in the order of a round's outputs:
    // the prologue issues what a round issues, so the loop entry and its
    // back edge present the same sequence of outstanding memory operations
    auto no_emit = [&]() {
        const __amdgpu_buffer_rsrc_t ro = rows(a.gR, (int64_t)kHC * d * 2, t1);
        const u32x2 z = u32x2{0u, 0u};
#pragma unroll
        for (int jj = 0; jj < kHC; ++jj) {
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((__vector_size__(8))) int, z), ro,
                                                  ox, jj * d * 2, 0);
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((__vector_size__(8))) int, z), ro,
                                                  ox + 8, jj * d * 2, 0);
        }
    };
    MbIo<H> io0, io1;
    load(io0, t0);
    no_emit();
    load(io1, t0 + kMbT);
    no_emit();
    for (int r = 0; r < nr; r += 2) {
        round(io0, r, 0);
        round(io1, r + 1, 1);
    }
    // the token group's dL/dW partial sums: lane (row, grp) holds mixes
    // 16 mt + 4 grp + i of feature 16 ct + row
    float* P = a.part + (int64_t)tg * kMix * K;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 16 * mt + 4 * grp + i;
                if (m < kMix) P[m * K + (int64_t)j * d + col0 + mc + 16 * ct + row] = gw[mt][ct][i];
            }
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
    MixBwdArgs ma{(const uint16_t*)R, (const uint16_t*)gh, (const uint16_t*)gRo, W, coef, (uint16_t*)gR, part, n, d,
                  ntg};
    constexpr int kH = 2;                        // d % 128 == 0 (bwd_supported)
    k_mix_bwd<kH><<<(unsigned)((d / MbGeo<kH>::F) * ntg), MbGeo<kH>::kThreads, 0, s>>>(ma);
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
