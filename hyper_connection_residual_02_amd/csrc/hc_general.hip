// hc_general.hip -- the hyper-connection mixing for stream counts other than
// four (hc = 1..8, hc != 4).  The "Reading weights" page writes its split +
// Sinkhorn kernel for any hc_mult, and the mix formula of the "Mix
// projection" page projects the flattened hc*d stream to (2 + hc) * hc
// numbers for any hc; four streams take the tuned kernels of the other
// files.  Here every step is a plain kernel, one template instance per hc:
//
//  * k_gmix  -- projection and RMS: a 32-token tile per workgroup, the
//               reduction axis staged 64 elements at a time through LDS
//               (tokens as float, weights as float), each thread holding a
//               4 x 4 block of (token, output) sums in double, accumulated
//               in feature order (k_gmix_pairs: one pair per thread, for
//               fewer than 48 outputs and many tokens; k_gmix_wave: one
//               wave per 2-4 tokens, lanes splitting the features, for few
//               outputs or few tokens).
//               Products of a bf16 and an fp32 value are exact in double;
//               k_gmix_pairs sums in feature order, k_gmix as (even staged
//               steps) + (odd staged steps), and the wave kernel adds 64
//               per-lane partial sums in a fixed butterfly.  Each stream
//               count takes one summation order whatever the call's size,
//               so a token's mixes never depend on the rest of its call.
//  * k_gsplit -- split + epsilon-Sinkhorn, one token per thread, with the
//               gate, softmax and normalisation arithmetic of the four-stream
//               kernel (same functions, same order).
//  * k_gpre, k_gpost -- hc_pre and hc_post over 16-byte chunks (8 features
//               of one token), summed in double in the order of the formula
//               and rounded once to bf16 (nearest even).
#include "hc_device.hpp"
#include "hc_launch.hpp"

namespace hc {

bool gen_hc(int hc_) { return hc_ >= 1 && hc_ <= kGenMaxHC && hc_ != kHC; }

static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t gen_ws_bytes(int64_t n, int hc_) {
    const size_t M = (size_t)(2 + hc_) * hc_;
    return align256((size_t)n * M * 4) + align256((size_t)n * hc_ * 4);
}

namespace {

constexpr int kGThreads = 256;
constexpr int kGT = 32;      // tokens per projection tile (kGT * 8 == kGThreads)
constexpr int kGKC = 64;     // reduction elements per staged step
static_assert(kGT * 8 == kGThreads, "one 16-byte chunk of the token tile per thread");
// Output count from which the projection uses 4 x 4 micro-tiles: below it too
// few threads would own a tile (measured: at 8 outputs the per-pair mapping
// is 2x faster, at 80 outputs the micro-tiles are 3x faster).
constexpr int kGTileMinM = 48;
// Below that, one wave per 2-4 tokens (k_gmix_wave) for at most 15 outputs
// (hc = 1, 2, 3), else one pair per thread (k_gmix_pairs, hc = 5), at every
// n: the two add in different orders, so a size threshold between them
// would let a token's last mix bit depend on its call's size.  The wave
// kernel fills the chip at small n but reads the weights once per 2-4
// tokens; measured (fused call, d = 5120): hc = 2, 4,096 tokens 69 us
// against 311, 65,536 tokens 933 against 1,512; hc = 3, 4,096 tokens 225
// against 478, 65,536 tokens 3,480 against 3,050; hc = 5, 4,096 tokens
// 1,445 against 2,896, 65,536 tokens 18,813 against 10,827.
constexpr int kGWaveMaxM = 15;

// Mix formula of the "Mix projection" page: m_j = r * sum_i x_i W[j, i] with
// r = 1 / sqrt(sum_i x_i^2 / K + norm_eps), K = hc * d.
//
// H groups ("halves") of 256 threads take interleaved staged steps (group h
// the steps H s + h), each with its own LDS tiles, so that with H = 2 a
// thread walks half the reduction axis: that pays while the tiles alone
// leave compute units idle, and costs LDS and occupancy otherwise.  In a
// group, threads 0..NW-1 each own a 4-token x 4-output
// micro-tile (tokens tg + 8i, outputs 4 jg + u), so each step costs 8 LDS
// reads per 16 products; threads NW..NW+31 form one token's sum of squares.
// The loads of a half's next step are issued before the products of its
// current one.  Every sum is formed as (even steps) + (odd steps), each part
// in feature order: with H = 2 the two groups hold the two parts, with H = 1
// one thread keeps both, so the two variants give the same bits and a
// token's mixes do not depend on which one its call takes.
template <int HC, int H>
__global__ __launch_bounds__(H * kGThreads) void k_gmix(const uint16_t* __restrict__ R, const float* __restrict__ W,
                                                        float* __restrict__ mixes, int64_t n, int d, float norm_eps) {
    constexpr int M = (2 + HC) * HC;
    constexpr int TT = 4, JJ = 4;
    constexpr int NT = kGT / TT;                 // token groups
    constexpr int NJ = (M + JJ - 1) / JJ;        // output groups (the last may be padded)
    constexpr int NW = NT * NJ;                  // threads of a half with a micro-tile
    static_assert(NW + kGT <= kGThreads, "micro-tiles plus one sum-of-squares thread per token");
    constexpr int WCH = M * (kGKC / 4);          // 16-byte weight chunks per step
    constexpr int WPT = (WCH + kGThreads - 1) / kGThreads;
    static_assert(H == 1 || H == 2, "one or two groups");
    __shared__ float xs[H][kGT][kGKC + 1];       // odd row stride: a wave's rows fall in distinct banks
    __shared__ float ws[H][M][kGKC + 1];
    __shared__ double red[H == 2 ? NW : 1][TT * JJ];   // odd-step sums of group 1, added by group 0
    __shared__ double sred[H == 2 ? kGT : 1];
    __shared__ double ssq[kGT];
    const int64_t K = (int64_t)HC * d;
    const int64_t ntiles = (n + kGT - 1) / kGT;
    const int h = threadIdx.x / kGThreads;       // group
    const int tid = threadIdx.x - h * kGThreads;
    const int tg = tid % NT, jg = tid / NT;
    const int st = tid - NW;
    const int xt = tid >> 3, xq = tid & 7;       // staged x chunk of this thread

    // K is a multiple of 8: a chunk lies wholly inside its row or past its
    // end; past K every staged value is zero
    auto load = [&](int64_t t0, int64_t k0, uint4& xv, float4 (&wv)[WPT]) {
        const int64_t k = k0 + xq * 8;
        xv = make_uint4(0u, 0u, 0u, 0u);
        if (t0 + xt < n && k < K) xv = *reinterpret_cast<const uint4*>(R + (t0 + xt) * K + k);
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            const int c = tid + i * kGThreads;
            const int j = c / (kGKC / 4), q = c - j * (kGKC / 4);
            const int64_t kk = k0 + q * 4;
            wv[i] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (c < WCH && kk < K) wv[i] = *reinterpret_cast<const float4*>(W + (int64_t)j * K + kk);
        }
    };
    auto stage = [&](const uint4& xv, const float4 (&wv)[WPT]) {
        float* xr = &xs[h][xt][xq * 8];
        xr[0] = bf_lo(xv.x); xr[1] = bf_hi(xv.x);
        xr[2] = bf_lo(xv.y); xr[3] = bf_hi(xv.y);
        xr[4] = bf_lo(xv.z); xr[5] = bf_hi(xv.z);
        xr[6] = bf_lo(xv.w); xr[7] = bf_hi(xv.w);
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            const int c = tid + i * kGThreads;
            if (c < WCH) {
                const int j = c / (kGKC / 4), q = c - j * (kGKC / 4);
                float* wr = &ws[h][j][q * 4];
                wr[0] = wv[i].x; wr[1] = wv[i].y; wr[2] = wv[i].z; wr[3] = wv[i].w;
            }
        }
    };

    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int64_t t0 = tile * kGT;
        // acc / sacc: the even steps (H = 2: this group's steps); acc1 /
        // sacc1: the odd steps (H = 1 only)
        double acc[TT][JJ], acc1[TT][JJ];
#pragma unroll
        for (int i = 0; i < TT; ++i)
#pragma unroll
            for (int u = 0; u < JJ; ++u) acc[i][u] = acc1[i][u] = 0.0;
        double sacc = 0.0, sacc1 = 0.0;
        // one staged step into the accumulators a / sa
        auto step = [&](double (&a)[TT][JJ], double& sa) {
            if (tid < NW) {
                const float* xr[TT];
                const float* wr[JJ];
#pragma unroll
                for (int i = 0; i < TT; ++i) xr[i] = xs[h][tg + NT * i];
#pragma unroll
                for (int u = 0; u < JJ; ++u) wr[u] = ws[h][jg * JJ + u < M ? jg * JJ + u : M - 1];
#pragma unroll 8
                for (int k = 0; k < kGKC; ++k) {
                    double xk[TT], wk[JJ];
#pragma unroll
                    for (int i = 0; i < TT; ++i) xk[i] = xr[i][k];
#pragma unroll
                    for (int u = 0; u < JJ; ++u) wk[u] = wr[u][k];
#pragma unroll
                    for (int i = 0; i < TT; ++i)
#pragma unroll
                        for (int u = 0; u < JJ; ++u) a[i][u] = __builtin_fma(xk[i], wk[u], a[i][u]);
                }
            } else if (st < kGT) {
#pragma unroll 16
                for (int k = 0; k < kGKC; ++k) {
                    const double v = xs[h][st][k];
                    sa = __builtin_fma(v, v, sa);
                }
            }
        };
        uint4 xv;
        float4 wv[WPT];
        load(t0, h * kGKC, xv, wv);
        bool odd = false;
        for (int64_t k0 = 0; k0 < K; k0 += H * kGKC) {
            const int64_t kh = k0 + h * kGKC;    // this group's step
            stage(xv, wv);
            __syncthreads();
            // always: past K it stages zeros (with an odd step count group 1
            // runs one step more than it has data for)
            load(t0, kh + H * kGKC, xv, wv);
            if (H == 1 && odd)
                step(acc1, sacc1);
            else
                step(acc, sacc);
            odd = !odd;
            __syncthreads();
        }
        if (H == 1) {
            // the odd steps' sums in the place of group 1's (red / sred)
#pragma unroll
            for (int i = 0; i < TT; ++i)
#pragma unroll
                for (int u = 0; u < JJ; ++u) acc[i][u] = acc[i][u] + acc1[i][u];
            sacc = sacc + sacc1;
        }
        if (H == 2 && h == 1) {
            if (tid < NW) {
#pragma unroll
                for (int i = 0; i < TT; ++i)
#pragma unroll
                    for (int u = 0; u < JJ; ++u) red[tid][i * JJ + u] = acc[i][u];
            } else if (st < kGT) {
                sred[st] = sacc;
            }
        }
        __syncthreads();
        if (h == 0 && st >= 0 && st < kGT) ssq[st] = H == 2 ? sacc + sred[st] : sacc;
        __syncthreads();
        if (h == 0 && tid < NW) {
#pragma unroll
            for (int i = 0; i < TT; ++i) {
                const int t = tg + NT * i;
                if (t0 + t >= n) continue;
                const double r = 1.0 / __builtin_sqrt(ssq[t] / (double)K + (double)norm_eps);
#pragma unroll
                for (int u = 0; u < JJ; ++u) {
                    const int j = jg * JJ + u;
                    const double sum = H == 2 ? acc[i][u] + red[tid][i * JJ + u] : acc[i][u];
                    if (j < M) mixes[(t0 + t) * M + j] = (float)(sum * r);
                }
            }
        }
        __syncthreads();        // the staged tiles, red and ssq are rewritten by the next tile
    }
}

// The same projection for few outputs ((2 + hc) * hc < 48): every
// (token, output) pair, the sum of squares counted as output M, belongs to
// one thread, so that all 256 threads share the products; the staging and
// its prefetch are those of k_gmix.
template <int HC>
__global__ __launch_bounds__(kGThreads) void k_gmix_pairs(const uint16_t* __restrict__ R,
                                                          const float* __restrict__ W, float* __restrict__ mixes,
                                                          int64_t n, int d, float norm_eps) {
    constexpr int M = (2 + HC) * HC;
    constexpr int NP = kGT * (M + 1);
    constexpr int PPT = (NP + kGThreads - 1) / kGThreads;
    constexpr int WCH = M * (kGKC / 4);
    constexpr int WPT = (WCH + kGThreads - 1) / kGThreads;
    __shared__ float xs[kGT][kGKC + 1];
    __shared__ float ws[M][kGKC + 1];
    __shared__ double ssq[kGT];
    const int64_t K = (int64_t)HC * d;
    const int64_t ntiles = (n + kGT - 1) / kGT;
    const int tid = threadIdx.x;
    const int xt = tid >> 3, xq = tid & 7;

    auto load = [&](int64_t t0, int64_t k0, uint4& xv, float4 (&wv)[WPT]) {
        const int64_t k = k0 + xq * 8;
        xv = make_uint4(0u, 0u, 0u, 0u);
        if (t0 + xt < n && k < K) xv = *reinterpret_cast<const uint4*>(R + (t0 + xt) * K + k);
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            const int c = tid + i * kGThreads;
            const int j = c / (kGKC / 4), q = c - j * (kGKC / 4);
            const int64_t kk = k0 + q * 4;
            wv[i] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (c < WCH && kk < K) wv[i] = *reinterpret_cast<const float4*>(W + (int64_t)j * K + kk);
        }
    };
    auto stage = [&](const uint4& xv, const float4 (&wv)[WPT]) {
        float* xr = &xs[xt][xq * 8];
        xr[0] = bf_lo(xv.x); xr[1] = bf_hi(xv.x);
        xr[2] = bf_lo(xv.y); xr[3] = bf_hi(xv.y);
        xr[4] = bf_lo(xv.z); xr[5] = bf_hi(xv.z);
        xr[6] = bf_lo(xv.w); xr[7] = bf_hi(xv.w);
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            const int c = tid + i * kGThreads;
            if (c < WCH) {
                const int j = c / (kGKC / 4), q = c - j * (kGKC / 4);
                float* wr = &ws[j][q * 4];
                wr[0] = wv[i].x; wr[1] = wv[i].y; wr[2] = wv[i].z; wr[3] = wv[i].w;
            }
        }
    };

    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int64_t t0 = tile * kGT;
        double acc[PPT];
#pragma unroll
        for (int p = 0; p < PPT; ++p) acc[p] = 0.0;
        uint4 xv;
        float4 wv[WPT];
        load(t0, 0, xv, wv);
        for (int64_t k0 = 0; k0 < K; k0 += kGKC) {
            stage(xv, wv);
            __syncthreads();
            if (k0 + kGKC < K) load(t0, k0 + kGKC, xv, wv);
#pragma unroll
            for (int p = 0; p < PPT; ++p) {
                const int pair = tid + p * kGThreads;
                if (pair < NP) {
                    const int t = pair / (M + 1), j = pair - t * (M + 1);
                    const float* xr = xs[t];
                    const float* wr = j < M ? ws[j] : xs[t];
                    double a = acc[p];
#pragma unroll 16
                    for (int k = 0; k < kGKC; ++k) a = __builtin_fma((double)xr[k], (double)wr[k], a);
                    acc[p] = a;
                }
            }
            __syncthreads();
        }
#pragma unroll
        for (int p = 0; p < PPT; ++p) {
            const int pair = tid + p * kGThreads;
            const int t = pair / (M + 1), j = pair - t * (M + 1);
            if (pair < NP && j == M) ssq[t] = acc[p];
        }
        __syncthreads();
#pragma unroll
        for (int p = 0; p < PPT; ++p) {
            const int pair = tid + p * kGThreads;
            const int t = pair / (M + 1), j = pair - t * (M + 1);
            if (pair < NP && j < M && t0 + t < n) {
                const double r = 1.0 / __builtin_sqrt(ssq[t] / (double)K + (double)norm_eps);
                mixes[(t0 + t) * M + j] = (float)(acc[p] * r);
            }
        }
        __syncthreads();        // ssq and the staged tiles are rewritten by the next tile
    }
}

// Split + epsilon-Sinkhorn of the "Reading weights" page for hc streams:
// pre_j = sigmoid(s0 m_j + b_j) + eps, post_j = 2 sigmoid(s1 m_{hc+j} +
// b_{hc+j}), logits s2 m_{2hc + j hc + k} + b_{2hc + j hc + k}; a row softmax
// plus eps, a column normalisation, then (iters - 1) row and column
// normalisations, each dividing by (sum + eps).
template <int HC>
__global__ __launch_bounds__(kGThreads) void k_gsplit(const float* __restrict__ mixes, const float* __restrict__ scale,
                                                      const float* __restrict__ base, float* __restrict__ pre,
                                                      float* __restrict__ post, float* __restrict__ comb, int64_t n,
                                                      int iters, float eps) {
    constexpr int M = (2 + HC) * HC;
    const float s0 = scale[0], s1 = scale[1], s2 = scale[2];
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n; t += stride) {
        const float* m = mixes + t * M;
#pragma unroll
        for (int j = 0; j < HC; ++j) {
            if (pre) pre[t * HC + j] = pre_gate(m[j], s0, base[j], eps);
            post[t * HC + j] = post_gate(m[HC + j], s1, base[HC + j]);
        }
        float c[HC][HC];
#pragma unroll
        for (int j = 0; j < HC; ++j)
#pragma unroll
            for (int k = 0; k < HC; ++k) c[j][k] = m[2 * HC + j * HC + k] * s2 + base[2 * HC + j * HC + k];
        // row softmax (the maximum is subtracted for range only), then + eps
#pragma unroll
        for (int j = 0; j < HC; ++j) {
            float mx = c[j][0];
#pragma unroll
            for (int k = 1; k < HC; ++k) mx = fmaxf(mx, c[j][k]);
            float s = 0.0f;
#pragma unroll
            for (int k = 0; k < HC; ++k) {
                c[j][k] = expf(c[j][k] - mx);
                s += c[j][k];
            }
#pragma unroll
            for (int k = 0; k < HC; ++k) c[j][k] = c[j][k] / s + eps;
        }
        auto col = [&]() {
#pragma unroll
            for (int k = 0; k < HC; ++k) {
                float s = 0.0f;
#pragma unroll
                for (int j = 0; j < HC; ++j) s += c[j][k];
                const float r = __builtin_amdgcn_rcpf(s + eps);
#pragma unroll
                for (int j = 0; j < HC; ++j) c[j][k] *= r;
            }
        };
        col();
        for (int it = 1; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < HC; ++j) {
                float s = 0.0f;
#pragma unroll
                for (int k = 0; k < HC; ++k) s += c[j][k];
                const float r = __builtin_amdgcn_rcpf(s + eps);
#pragma unroll
                for (int k = 0; k < HC; ++k) c[j][k] *= r;
            }
            col();
        }
#pragma unroll
        for (int j = 0; j < HC; ++j)
#pragma unroll
            for (int k = 0; k < HC; ++k) comb[(t * HC + j) * HC + k] = c[j][k];
    }
}

// 8 features of one stream chunk as doubles (element e of the 16 bytes).
__device__ __forceinline__ double bf_at(const uint4& v, int e) {
    const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
    return (double)((e & 1) ? bf_hi(w) : bf_lo(w));
}

__device__ __forceinline__ uint4 pack8(const uint32_t (&o)[8]) {
    return make_uint4(pack2(o[0], o[1]), pack2(o[2], o[3]), pack2(o[4], o[5]), pack2(o[6], o[7]));
}

// hc_pre of the "Mix projection" page: h_c = bf16(sum_k pre_k R_{k,c}).
template <int HC>
__global__ __launch_bounds__(kGThreads) void k_gpre(const uint16_t* __restrict__ R, const float* __restrict__ pre,
                                                    uint16_t* __restrict__ h, int64_t n, int d) {
    const int cpt = d / 8;
    const int64_t items = n * cpt;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t it = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; it < items; it += stride) {
        const int64_t t = it / cpt;
        const int c0 = (int)(it - t * cpt) * 8;
        uint4 r[HC];
        double p[HC];
#pragma unroll
        for (int k = 0; k < HC; ++k) {
            r[k] = *reinterpret_cast<const uint4*>(R + (t * HC + k) * d + c0);
            p[k] = pre[t * HC + k];
        }
        uint32_t o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            double y = p[0] * bf_at(r[0], e);
#pragma unroll
            for (int k = 1; k < HC; ++k) y = __builtin_fma(p[k], bf_at(r[k], e), y);
            o[e] = bf16_rn_f64(y);
        }
        *reinterpret_cast<uint4*>(h + t * d + c0) = pack8(o);
    }
}

// hc_post of the "Mix projection" page: output stream k is
// bf16(post_k x_c + sum_j comb[j][k] R_{j,c}).  An item reads every stream
// of its chunk before writing any, so R_out may be R.
template <int HC>
__global__ __launch_bounds__(kGThreads) void k_gpost(const uint16_t* __restrict__ x, const uint16_t* R,
                                                     const float* __restrict__ post, const float* __restrict__ comb,
                                                     uint16_t* Rout, int64_t n, int d) {
    const int cpt = d / 8;
    const int64_t items = n * cpt;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t it = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; it < items; it += stride) {
        const int64_t t = it / cpt;
        const int c0 = (int)(it - t * cpt) * 8;
        const uint4 xv = *reinterpret_cast<const uint4*>(x + t * d + c0);
        uint4 r[HC];
#pragma unroll
        for (int j = 0; j < HC; ++j) r[j] = *reinterpret_cast<const uint4*>(R + (t * HC + j) * d + c0);
#pragma unroll
        for (int k = 0; k < HC; ++k) {
            const double pk = post[t * HC + k];
            double cj[HC];
#pragma unroll
            for (int j = 0; j < HC; ++j) cj[j] = comb[(t * HC + j) * HC + k];
            uint32_t o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                double y = pk * bf_at(xv, e);
#pragma unroll
                for (int j = 0; j < HC; ++j) y = __builtin_fma(cj[j], bf_at(r[j], e), y);
                o[e] = bf16_rn_f64(y);
            }
            *reinterpret_cast<uint4*>(Rout + (t * HC + k) * d + c0) = pack8(o);
        }
    }
}

// The projection for few outputs ((2 + hc) * hc < 48): one wave per TW
// tokens.  Lane l takes the 8-feature chunks l, l + 64, ... of the
// flattened stream and keeps, for each of its tokens, every output's
// partial sum (and the sum of squares) in double, in chunk order; a
// butterfly over the wave then adds the 64 partials in one fixed order, so
// that every lane holds the same total and results do not depend on n.
// The weights are read from memory (L2) once per TW tokens.
template <int HC>
__global__ __launch_bounds__(kGThreads) void k_gmix_wave(const uint16_t* __restrict__ R,
                                                         const float* __restrict__ W, float* __restrict__ mixes,
                                                         int64_t n, int d, float norm_eps) {
    constexpr int M = (2 + HC) * HC;
    constexpr int TW = M <= 15 ? 4 : 2;          // tokens per wave (register budget of the sums)
    constexpr int WAVES = kGThreads / 64;
    const int64_t K = (int64_t)HC * d;
    const int64_t nch = K / 8;
    const int lane = threadIdx.x & 63;
    const int64_t groups = (n + TW - 1) / TW;
    const int64_t stride = (int64_t)gridDim.x * WAVES;
    for (int64_t g = (int64_t)blockIdx.x * WAVES + (threadIdx.x >> 6); g < groups; g += stride) {
        const int64_t t0 = g * TW;
        double acc[TW][M + 1];
#pragma unroll
        for (int i = 0; i < TW; ++i)
#pragma unroll
            for (int j = 0; j <= M; ++j) acc[i][j] = 0.0;
        for (int64_t c = lane; c < nch; c += 64) {
            double x[TW][8];
#pragma unroll
            for (int i = 0; i < TW; ++i) {
                uint4 v = make_uint4(0u, 0u, 0u, 0u);
                if (t0 + i < n) v = *reinterpret_cast<const uint4*>(R + (t0 + i) * K + c * 8);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    x[i][e] = bf_at(v, e);
                    acc[i][M] = __builtin_fma(x[i][e], x[i][e], acc[i][M]);
                }
            }
#pragma unroll
            for (int j = 0; j < M; ++j) {
                const float4 w0 = *reinterpret_cast<const float4*>(W + (int64_t)j * K + c * 8);
                const float4 w1 = *reinterpret_cast<const float4*>(W + (int64_t)j * K + c * 8 + 4);
                const double wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
                for (int i = 0; i < TW; ++i)
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[i][j] = __builtin_fma(x[i][e], wv[e], acc[i][j]);
            }
        }
        // lane l and lane l ^ o add the same two values, so every lane ends
        // with the same bits
#pragma unroll
        for (int i = 0; i < TW; ++i)
#pragma unroll
            for (int j = 0; j <= M; ++j)
#pragma unroll
                for (int o = 32; o >= 1; o >>= 1) acc[i][j] += __shfl_xor(acc[i][j], o);
#pragma unroll
        for (int i = 0; i < TW; ++i) {
            if (t0 + i >= n) break;
            const double r = 1.0 / __builtin_sqrt(acc[i][M] / (double)K + (double)norm_eps);
            double v = 0.0;
#pragma unroll
            for (int j = 0; j < M; ++j) v = lane == j ? acc[i][j] : v;
            if (lane < M) mixes[(t0 + i) * M + lane] = (float)(v * r);
        }
    }
}

int grid_for(int64_t items) {
    const int64_t cap = (int64_t)num_cus() * 8;
    const int64_t need = (items + kGThreads - 1) / kGThreads;
    return (int)(need < cap ? (need > 0 ? need : 1) : cap);
}

template <template <int> class Op, typename... A>
int dispatch_hc(int hc_, A... args) {
    switch (hc_) {
        case 1: return Op<1>::run(args...);
        case 2: return Op<2>::run(args...);
        case 3: return Op<3>::run(args...);
        case 5: return Op<5>::run(args...);
        case 6: return Op<6>::run(args...);
        case 7: return Op<7>::run(args...);
        case 8: return Op<8>::run(args...);
        default: return -1;
    }
}

template <int HC>
int wave_grid(int64_t n) {
    constexpr int M = (2 + HC) * HC;
    constexpr int TW = M <= 15 ? 4 : 2;
    const int64_t groups = (n + TW - 1) / TW, per = kGThreads / 64;
    const int64_t need = (groups + per - 1) / per, cap = (int64_t)num_cus() * 16;
    return (int)(need < cap ? need : cap);
}

template <int HC>
struct MixOp {
    static int run(const void* R, const float* W, float* mixes, int64_t n, int d, float norm_eps, hipStream_t s) {
        const int64_t tiles = (n + kGT - 1) / kGT, cap = (int64_t)num_cus() * 16;
        constexpr int M = (2 + HC) * HC;
        const dim3 grid((unsigned)(tiles < cap ? tiles : cap));
        if constexpr (M >= kGTileMinM) {
            // two groups per tile while fewer than two tiles per compute unit
            // (measured at d = 5120, 4,096 tokens: hc = 6 2,064 against
            // 2,840 us, hc = 8 2,840 against 3,799; at 65,536 tokens one group
            // is faster: 12,020 against 17,198 and 19,477 against 23,707)
            const auto two = k_gmix<HC, 2>;
            const auto one = k_gmix<HC, 1>;
            if (tiles < 2 * (int64_t)num_cus())
                hipLaunchKernelGGL(two, grid, dim3(2 * kGThreads), 0, s, static_cast<const uint16_t*>(R), W, mixes,
                                   n, d, norm_eps);
            else
                hipLaunchKernelGGL(one, grid, dim3(kGThreads), 0, s, static_cast<const uint16_t*>(R), W, mixes, n,
                                   d, norm_eps);
        }
        else if (M <= kGWaveMaxM)
            hipLaunchKernelGGL(k_gmix_wave<HC>, dim3(wave_grid<HC>(n)), dim3(kGThreads), 0, s,
                               static_cast<const uint16_t*>(R), W, mixes, n, d, norm_eps);
        else
            hipLaunchKernelGGL(k_gmix_pairs<HC>, grid, dim3(kGThreads), 0, s, static_cast<const uint16_t*>(R), W,
                               mixes, n, d, norm_eps);
        return hipGetLastError() == hipSuccess ? 0 : -1;
    }
};

template <int HC>
struct SplitOp {
    static int run(const float* mixes, const float* scale, const float* base, float* pre, float* post, float* comb,
                   int64_t n, int iters, float eps, hipStream_t s) {
        hipLaunchKernelGGL(k_gsplit<HC>, dim3(grid_for(n)), dim3(kGThreads), 0, s, mixes, scale, base, pre, post,
                           comb, n, iters, eps);
        return hipGetLastError() == hipSuccess ? 0 : -1;
    }
};

template <int HC>
struct PreOp {
    static int run(const void* R, const float* pre, void* h, int64_t n, int d, hipStream_t s) {
        hipLaunchKernelGGL(k_gpre<HC>, dim3(grid_for(n * (d / 8))), dim3(kGThreads), 0, s,
                           static_cast<const uint16_t*>(R), pre, static_cast<uint16_t*>(h), n, d);
        return hipGetLastError() == hipSuccess ? 0 : -1;
    }
};

template <int HC>
struct PostOp {
    static int run(const void* x, const void* R, const float* post, const float* comb, void* Rout, int64_t n, int d,
                   hipStream_t s) {
        hipLaunchKernelGGL(k_gpost<HC>, dim3(grid_for(n * (d / 8))), dim3(kGThreads), 0, s,
                           static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(R), post, comb,
                           static_cast<uint16_t*>(Rout), n, d);
        return hipGetLastError() == hipSuccess ? 0 : -1;
    }
};

}  // namespace

int launch_gen_mixes(const void* R, const float* W, float* mixes, int64_t n, int hc_, int d, float norm_eps,
                     hipStream_t s) {
    return dispatch_hc<MixOp>(hc_, R, W, mixes, n, d, norm_eps, s);
}

int launch_gen_split(const float* mixes, const float* scale, const float* base, float* pre, float* post,
                     float* comb, int64_t n, int hc_, int iters, float eps, hipStream_t s) {
    return dispatch_hc<SplitOp>(hc_, mixes, scale, base, pre, post, comb, n, iters, eps, s);
}

int launch_gen_pre(const void* R, const float* pre, void* h, int64_t n, int hc_, int d, hipStream_t s) {
    return dispatch_hc<PreOp>(hc_, R, pre, h, n, d, s);
}

int launch_gen_post(const void* x, const void* R, const float* post, const float* comb, void* Rout, int64_t n,
                    int hc_, int d, hipStream_t s) {
    return dispatch_hc<PostOp>(hc_, x, R, post, comb, Rout, n, d, s);
}

int launch_gen_fused(const void* R, const float* W, const float* scale, const float* base, void* h, float* pre,
                     float* post, float* comb, float* mixes, void* ws, int64_t n, int hc_, int d, int iters,
                     float eps, float norm_eps, hipStream_t s) {
    // what this call keeps in the workspace starts at offset 0, so that the
    // four-stream kernels' header (its first 256 bytes) is overwritten and a
    // later four-stream call on the same workspace takes it as fresh
    // (clearing its record area) rather than trusting stale contents
    const size_t M = (size_t)(2 + hc_) * hc_;
    char* w = static_cast<char*>(ws);
    float* mx = mixes ? mixes : reinterpret_cast<float*>(w);
    float* pr = pre ? pre : reinterpret_cast<float*>(w + (mixes ? 0 : align256((size_t)n * M * 4)));
    if (launch_gen_mixes(R, W, mx, n, hc_, d, norm_eps, s)) return -1;
    if (launch_gen_split(mx, scale, base, pr, post, comb, n, hc_, iters, eps, s)) return -1;
    return launch_gen_pre(R, pr, h, n, hc_, d, s);
}

}  // namespace hc
