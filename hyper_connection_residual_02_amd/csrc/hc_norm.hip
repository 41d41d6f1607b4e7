// hc_norm.hip -- the pre-sublayer RMSNorm on hc_pre's output, alone
// (hc_rmsnorm) and fused with hc_pre (hc_pre_norm).
//
// "Mix projection" page, Block.__init__: every block holds two RMSNorms of
// width dim with norm_eps, and a sublayer's input is hc_pre's output.  The
// norm's formula is not printed; it is read as the page's mix-formula
// normalisation applied to the d features of h, times an fp32 per-feature
// weight g:
//
//   y_c = bf16( h_c * r * g_c ),   r = 1 / sqrt( sum_c h_c^2 / d + norm_eps ),
//
// where h is the bf16 output of hc_pre (the value a separate hc_pre call
// would store).  Arithmetic: h is formed exactly (hc_pre's double sum and
// one rounding); the sum of squares, r, (h * r) * g are taken in double,
// and y is rounded once, nearest-even.  Only the order of the sum of
// squares differs from a sequential evaluation, which changes r by at most
// an ulp of double.
//
// One kernel serves both calls.  HC = 0 reads h itself; HC >= 1 reads the
// HC streams of R and forms h on the way (writing it only if asked).  Each
// token is handled by W waves (W = 1, 2, 4, 8 or 16, the fewest that hold
// its d / 8 chunks at four per lane), every lane keeps its chunks of h in
// registers, the token's sum of squares is reduced within each wave and
// across its W waves through LDS in a fixed order, and y is written from
// the registers: R (or h) is read from HBM once and y written once.

#include "hc_device.hpp"
#include "hc_launch.hpp"

namespace hc {

namespace {

constexpr int kNIt = 4;                 // chunks of 8 features per lane (R in)
constexpr int kNItH = 8;                // chunks per lane (h in: fewer bytes per chunk)
constexpr int kNormMaxW = 16;           // waves per token at most (d <= 32,768)

__device__ __forceinline__ double shfl_xor_f64(double v, int m) {
    const int lo = __shfl_xor((int)(uint32_t)__double_as_longlong(v), m, 64);
    const int hi = __shfl_xor((int)(uint32_t)((uint64_t)__double_as_longlong(v) >> 32), m, 64);
    return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}

// h of one 8-feature chunk from HC streams: bf16(sum_k p_k R_k), the double
// sum in stream order rounded once (hc_pre's arithmetic).
template <int HC>
__device__ __forceinline__ u32x4 h_chunk(const double (&p)[HC], const u32x4 (&r)[HC]) {
    auto sum = [&](int w, int e) {
        double v = p[0] * (double)(e ? bf_hi(r[0][w]) : bf_lo(r[0][w]));
#pragma unroll
        for (int k = 1; k < HC; ++k) v = __builtin_fma(p[k], (double)(e ? bf_hi(r[k][w]) : bf_lo(r[k][w])), v);
        return v;
    };
    float f[4][2];
    bool mid = false;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        f[w][0] = f32_mid(sum(w, 0), mid);
        f[w][1] = f32_mid(sum(w, 1), mid);
    }
    u32x4 out;
    if (__builtin_amdgcn_ballot_w64(mid)) {
#pragma unroll
        for (int w = 0; w < 4; ++w) out[w] = pack2(bf16_rn_f64(sum(w, 0)), bf16_rn_f64(sum(w, 1)));
    } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) out[w] = bf16x2_rn(f[w][0], f[w][1]);
    }
    return out;
}

// y of one chunk: bf16((h * r) * g) for its 8 features.
__device__ __forceinline__ u32x4 y_chunk(const u32x4 hv, double r, const f32x4 g0, const f32x4 g1) {
    auto val = [&](int w, int e) {
        const double hv_ = (double)(e ? bf_hi(hv[w]) : bf_lo(hv[w]));
        const float g = w < 2 ? g0[2 * w + e] : g1[2 * (w - 2) + e];
        return (hv_ * r) * (double)g;
    };
    float f[4][2];
    bool mid = false;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        f[w][0] = f32_mid(val(w, 0), mid);
        f[w][1] = f32_mid(val(w, 1), mid);
    }
    u32x4 out;
    if (__builtin_amdgcn_ballot_w64(mid)) {
#pragma unroll
        for (int w = 0; w < 4; ++w) out[w] = pack2(bf16_rn_f64(val(w, 0)), bf16_rn_f64(val(w, 1)));
    } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) out[w] = bf16x2_rn(f[w][0], f[w][1]);
    }
    return out;
}

// Block: max(4, W) waves; token t = t0 + blockIdx.x * (waves / W) + wave / W.
// With HC = 0, y may be X itself (normalised in place): a token's chunks
// are all loaded before the reduction that every store depends on (and the
// barrier, when W > 1).
template <int HC, int NIT>
__global__ __launch_bounds__(64 * kNormMaxW) void k_pre_norm(const uint16_t* X, const float* __restrict__ pre,
                                                               const float* __restrict__ gamma, uint16_t* h,
                                                               uint16_t* y,
                                                               int64_t t0, int64_t n, int d, int W, float norm_eps) {
    __shared__ double red[kNormMaxW];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int tpb = (blockDim.x >> 6) / W;                 // tokens per block
    const int64_t t = t0 + (int64_t)blockIdx.x * tpb + wave / W;
    const bool live = t < n;
    const int tw = wave % W;                               // wave of the token
    const int cpt = d / 8;
    const int st = tw * 64 + lane;                         // lane of the token
    const int tpt = 64 * W;
    const int64_t tt = live ? t : 0;

    double p[HC > 0 ? HC : 1];
#pragma unroll
    for (int k = 0; k < HC; ++k) p[k] = pre[tt * HC + k];

    u32x4 hv[NIT];
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < NIT; ++i) {
        const int c8 = st + i * tpt;
        if (live && c8 < cpt) {
            if constexpr (HC == 0) {
                hv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(X + tt * d + 8 * c8));
            } else {
                u32x4 r[HC];
#pragma unroll
                for (int k = 0; k < HC; ++k)
                    r[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(X + (tt * HC + k) * d + 8 * c8));
                hv[i] = h_chunk<HC>(p, r);
            }
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const double a = bf_lo(hv[i][w]), b = bf_hi(hv[i][w]);
                ss = __builtin_fma(a, a, ss);
                ss = __builtin_fma(b, b, ss);
            }
        } else {
            hv[i] = u32x4{0u, 0u, 0u, 0u};
        }
    }
    // h after every load of the lane has been issued
    if (HC > 0 && h) {
#pragma unroll
        for (int i = 0; i < NIT; ++i) {
            const int c8 = st + i * tpt;
            if (live && c8 < cpt) __builtin_nontemporal_store(hv[i], reinterpret_cast<u32x4*>(h + tt * d + 8 * c8));
        }
    }
    if (y == nullptr) return;           // hc_pre alone (y is uniform: the whole block leaves)
    // the token's sum of squares: within the wave, then over its W waves in
    // wave order
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += shfl_xor_f64(ss, m);
    if (W > 1) {
        if (lane == 0) red[wave] = ss;
        __syncthreads();
        const int w0 = wave - tw;
        ss = red[w0];
        for (int k = 1; k < W; ++k) ss += red[w0 + k];
    }
    if (!live) return;
    const double r = 1.0 / __builtin_sqrt(ss / (double)d + (double)norm_eps);
#pragma unroll
    for (int i = 0; i < NIT; ++i) {
        const int c8 = st + i * tpt;
        if (c8 < cpt) {
            const f32x4 g0 = *reinterpret_cast<const f32x4*>(gamma + 8 * c8);
            const f32x4 g1 = *reinterpret_cast<const f32x4*>(gamma + 8 * c8 + 4);
            __builtin_nontemporal_store(y_chunk(hv[i], r, g0, g1), reinterpret_cast<u32x4*>(y + tt * d + 8 * c8));
        }
    }
}

}  // namespace

// Waves per token for width d: the fewest of 1, 2, 4, 8, 16 whose lanes hold
// every chunk at nit per lane; 0 if d is too wide.
static int waves_for(int d, int nit) {
    const int cpt = d / 8;
    for (int W = 1; W <= kNormMaxW; W *= 2)
        if (cpt <= 64 * W * nit) return W;
    return 0;
}

int norm_waves(int d) { return waves_for(d, kNIt); }

int launch_pre_norm(const void* R, const float* pre, const float* gamma, void* h, void* y, int64_t n, int hc,
                    int d, float norm_eps, hipStream_t s) {
    const int W = waves_for(d, hc == 0 ? kNItH : kNIt);
    if (W == 0 || hc < 0 || hc > kGenMaxHC) return -1;
    const int waves = W < 4 ? 4 : W;
    const int tpb = waves / W;
    auto X = static_cast<const uint16_t*>(R);
    auto H = static_cast<uint16_t*>(h);
    auto Y = static_cast<uint16_t*>(y);
    // at most 2^30 workgroups per launch; later launches start at token t0
    const int64_t per = (int64_t)tpb << 30;
    for (int64_t t0 = 0; t0 < n; t0 += per) {
        const int64_t m = n - t0 < per ? n - t0 : per;
        const dim3 g((unsigned)((m + tpb - 1) / tpb)), b((unsigned)(64 * waves));
        switch (hc) {
            case 0: k_pre_norm<0, kNItH><<<g, b, 0, s>>>(X, pre, gamma, nullptr, Y, t0, n, d, W, norm_eps); break;
            case 1: k_pre_norm<1, kNIt><<<g, b, 0, s>>>(X, pre, gamma, H, Y, t0, n, d, W, norm_eps); break;
            case 2: k_pre_norm<2, kNIt><<<g, b, 0, s>>>(X, pre, gamma, H, Y, t0, n, d, W, norm_eps); break;
            case 3: k_pre_norm<3, kNIt><<<g, b, 0, s>>>(X, pre, gamma, H, Y, t0, n, d, W, norm_eps); break;
            case 4: k_pre_norm<4, kNIt><<<g, b, 0, s>>>(X, pre, gamma, H, Y, t0, n, d, W, norm_eps); break;
            case 5: k_pre_norm<5, kNIt><<<g, b, 0, s>>>(X, pre, gamma, H, Y, t0, n, d, W, norm_eps); break;
            case 6: k_pre_norm<6, kNIt><<<g, b, 0, s>>>(X, pre, gamma, H, Y, t0, n, d, W, norm_eps); break;
            case 7: k_pre_norm<7, kNIt><<<g, b, 0, s>>>(X, pre, gamma, H, Y, t0, n, d, W, norm_eps); break;
            case 8: k_pre_norm<8, kNIt><<<g, b, 0, s>>>(X, pre, gamma, H, Y, t0, n, d, W, norm_eps); break;
        }
        if (hipGetLastError() != hipSuccess) return -1;
    }
    return 0;
}

}  // namespace hc
