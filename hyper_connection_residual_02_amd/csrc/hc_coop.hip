// hc_coop.hip -- the mix projection ("Mix projection" page, mix formula)
// and the fused projection + split/Sinkhorn + hc_pre, as one persistent,
// cooperatively launched kernel.
//
// Why this shape.  Every token needs all 24 x 4d projection weights
// (1.97 MB in fp32), and hc_pre needs the token's residual a second time
// after the full 4d-long reduction is known.  A tile of tokens large enough
// to amortise the weights does not fit on one CU, so instead the 4d
// reduction is split across the CUs of a group:
//
//  * G workgroups (one per CU, four waves each) form a group; member q owns
//    a 32*KS-feature slice of every stream (d = 5120: G = 32, 160 features,
//    KS = 5), keeps its slice of the weights resident in registers for the
//    whole kernel as MFMA B operands, and for each round of T tokens loads
//    only its slice of those tokens (one HBM pass over the residual).
//  * The projection of the slice runs on MFMA (v_mfma_f32_16x16x32_bf16).
//    The bf16 residual is exact; the fp32 weights are split exactly into
//    three bf16 pieces (w = hi + mid + lo), laid out as 80 MFMA columns
//    (3 x 24 used), so the products are exact and the sums are fp32.
//  * Members publish per-round partial sums (24 dots + sum of squares) to a
//    workspace, then meet at a counter; the owner of each token adds the G
//    partials in a fixed order, forms the mixes, runs the split and the
//    Sinkhorn on one 16-lane row, writes the coefficients, and publishes pre;
//    after a second counter every member forms h for its slice from the
//    residual still held in registers.
//  * Workgroup b belongs to group b % NG; with NG = 8 this puts a group on
//    one XCD (workgroups are dispatched round-robin over the XCDs).
//
// Cross-workgroup exchange uses device-scope (sc1) loads and stores and
// device-scope atomic counters, with an explicit wait for outstanding
// stores before each arrival, so no L2 writeback/invalidate is needed.
// Every wait is bounded in time; a timed-out wait raises a flag in the
// workspace and the kernel drains.

#include "hc_device.hpp"
#include "hc_launch.hpp"

namespace hc {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTiles = 5;          // 5 x 16 = 80 MFMA columns (72 used)
constexpr int kPStride = 32;       // floats per token in a partial record
constexpr int kCntStride = 64;     // uint32 per group of counters (2 x 128 B)

struct CoopArgs {
    const uint16_t* R;
    const float* W;
    const float* scale;
    const float* base;
    uint16_t* h;
    float* pre;
    float* post;
    float* comb;
    float* mixes;
    float* ws_part;     // [NG][2][G][T][kPStride]
    float* ws_pre;      // [NG][2][T][4]
    uint32_t* ws_cnt;   // [NG][kCntStride]: arrivals of partials at 0, of pre at 32; error flag after
    int64_t n;
    int64_t ntiles;
    int d;
    int G;
    int NG;
    int iters;
    float eps;
    float norm_eps;
    float K;
};

__device__ __forceinline__ void st_dev(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev_u(uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// All of this thread's outstanding memory operations have completed.
__device__ __forceinline__ void wait_all_mem() { __builtin_amdgcn_s_waitcnt(0); }

// Thread 0 waits until *cnt >= target (bounded: ~2 s of the 100 MHz
// real-time clock); the result is shared through LDS.  Returns false when
// this workgroup must stop (timeout here or a flag raised elsewhere).
__device__ bool group_wait(uint32_t* cnt, uint32_t target, uint32_t* err, int* lds_flag) {
    if (threadIdx.x == 0) {
        int ok = 1;
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        while (ld_dev_u(cnt) < target) {
            if (ld_dev_u(err) != 0u) { ok = 0; break; }
            if (__builtin_amdgcn_s_memrealtime() - t0 > 200000000ull) {
                __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                ok = 0;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        *lds_flag = ok;
    }
    __syncthreads();
    return *lds_flag != 0;
}

// Piece and mix index of MFMA column (tile ct, lane column i):
//   tiles 0..2: piece ct, j = i;   tile 3: i < 8 -> (0, 16+i), else (1, 8+i);
//   tile 4: i < 8 -> (2, 16+i), else unused.
__device__ __forceinline__ void col_map(int ct, int i, int& piece, int& j) {
    if (ct < 3) { piece = ct; j = i; }
    else if (ct == 3) { piece = i < 8 ? 0 : 1; j = 16 + (i & 7); }
    else { piece = i < 8 ? 2 : -1; j = 16 + i; }
}

template <int KS, int TM>
struct Frags {
    u32x4 r[TM][KS];
};

template <int KS, int TM>
__device__ __forceinline__ void load_round(Frags<KS, TM>& f, const CoopArgs& a, int64_t tile, int cw) {
    const int l = threadIdx.x & 63, row = l & 15, grp = l >> 4;
    constexpr int T = 16 * TM;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
        const int64_t tok = tile * T + 16 * tm + row;
        const bool ok = tok < a.n;
        const u32x4* src = reinterpret_cast<const u32x4*>(a.R + ((ok ? tok : 0) * kHC + grp) * (int64_t)a.d + cw);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (ok) v = __builtin_nontemporal_load(src + s);
            f.r[tm][s] = v;
        }
    }
}

template <int KS, int TM>
struct Lds {
    float red[kWaves][16 * TM][kPStride];   // per-wave partials of the round
    float mix[16][kPStride];                // owned tokens: summed partials
    float mixv[16][kMix];                   // owned tokens: mixes
    float preL[16 * TM][4];                 // pre of every token of the round
    int flag;
};

// One round: projection of this member's slice for T tokens, exchange,
// owners' split + Sinkhorn, and (fused) h for the slice.
template <int KS, int TM, bool FUSED>
__device__ __forceinline__ bool do_round(const Frags<KS, TM>& f, const bf16x8 (&wf)[KS][kTiles],
                                         const CoopArgs& a, Lds<KS, TM>& L, int64_t tile, uint32_t r,
                                         int g, int q, int cw) {
    constexpr int T = 16 * TM;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, row = l & 15, grp = l >> 4;
    const int slot = r & 1;
    uint32_t* cnt_part = a.ws_cnt + g * kCntStride;
    uint32_t* cnt_pre = cnt_part + 32;
    uint32_t* err = a.ws_cnt + a.NG * kCntStride;

    // ---- projection of the slice (MFMA) and sum of squares (fp32 FMA)
    f32x4 acc[TM][kTiles];
    float ss[TM];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
        ss[tm] = 0.0f;
#pragma unroll
        for (int ct = 0; ct < kTiles; ++ct) acc[tm][ct] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
            const bf16x8 av = __builtin_bit_cast(bf16x8, f.r[tm][s]);
#pragma unroll
            for (int ct = 0; ct < kTiles; ++ct)
                acc[tm][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, wf[s][ct], acc[tm][ct], 0, 0, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float lo = bf_lo(f.r[tm][s][e]), hi = bf_hi(f.r[tm][s][e]);
                ss[tm] = __builtin_fmaf(lo, lo, ss[tm]);
                ss[tm] = __builtin_fmaf(hi, hi, ss[tm]);
            }
        }
    }
    // ---- combine the three weight pieces; per-wave partials to LDS
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
        float sv = ss[tm];
        sv += __shfl_xor(sv, 16);
        sv += __shfl_xor(sv, 32);
        if (grp == 0) L.red[w][16 * tm + row][kMix] = sv;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int tk = 16 * tm + 4 * grp + rr;
            const float v0 = (acc[tm][2][rr] + acc[tm][1][rr]) + acc[tm][0][rr];
            const float t3 = acc[tm][3][rr];
            const float t3x = __shfl_xor(t3, 8);
            const float v1 = (acc[tm][4][rr] + t3x) + t3;
            L.red[w][tk][row] = v0;
            if (row < 8) L.red[w][tk][16 + row] = v1;
        }
    }
    __syncthreads();
    // ---- this member's partial for the round -> workspace
    {
        float* part = a.ws_part + ((((int64_t)g * 2 + slot) * a.G + q) * T) * kPStride;
        for (int i = tid; i < T * (kMix + 1); i += kThreads) {
            const int tk = i / (kMix + 1), e = i - tk * (kMix + 1);
            const float v = ((L.red[0][tk][e] + L.red[1][tk][e]) + L.red[2][tk][e]) + L.red[3][tk][e];
            st_dev(part + tk * kPStride + e, v);
        }
        wait_all_mem();
        __syncthreads();
        if (tid == 0) __hip_atomic_fetch_add(cnt_part, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (!group_wait(cnt_part, (uint32_t)a.G * (r + 1), err, &L.flag)) return false;

    // ---- owners: tokens tl = q + G*o of the round, 16 at a time
    const int nown = q < T ? (T - 1 - q) / a.G + 1 : 0;
    const float* part0 = a.ws_part + (((int64_t)g * 2 + slot) * a.G) * T * kPStride;
    for (int o0 = 0; o0 < nown; o0 += 16) {
        const int cnt = nown - o0 < 16 ? nown - o0 : 16;
        for (int i = tid; i < cnt * (kMix + 1); i += kThreads) {
            const int o = i / (kMix + 1), e = i - o * (kMix + 1);
            const int tl = q + a.G * (o0 + o);
            float s = 0.0f;
            for (int qq = 0; qq < a.G; ++qq) s += ld_dev(part0 + ((int64_t)qq * T + tl) * kPStride + e);
            L.mix[o][e] = s;
        }
        __syncthreads();
        for (int i = tid; i < cnt * kMix; i += kThreads) {
            const int o = i / kMix, j = i - o * kMix;
            const float rs = 1.0f / sqrtf(L.mix[o][kMix] / a.K + a.norm_eps);
            const float m = L.mix[o][j] * rs;
            L.mixv[o][j] = m;
            const int64_t t = tile * T + q + a.G * (o0 + o);
            if (a.mixes && t < a.n) a.mixes[t * kMix + j] = m;
        }
        __syncthreads();
        if (FUSED) {
            const int o = tid >> 4, e = tid & 15;
            const bool valid = o < cnt;
            float p, qv, c;
            split_sinkhorn16(L.mixv[valid ? o : 0], a.scale[0], a.scale[1], a.scale[2], a.base, a.iters, a.eps,
                             p, qv, c);
            if (valid) {
                const int tl = q + a.G * (o0 + o);
                const int64_t t = tile * T + tl;
                if (e < kHC) st_dev(a.ws_pre + (((int64_t)g * 2 + slot) * T + tl) * 4 + e, p);
                if (t < a.n) {
                    a.comb[t * (kHC * kHC) + e] = c;
                    if (e < kHC) {
                        if (a.pre) a.pre[t * kHC + e] = p;
                        a.post[t * kHC + e] = qv;
                    }
                }
            }
        }
        __syncthreads();
    }
    if (!FUSED) return true;
    wait_all_mem();
    __syncthreads();
    if (tid == 0) __hip_atomic_fetch_add(cnt_pre, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!group_wait(cnt_pre, (uint32_t)a.G * (r + 1), err, &L.flag)) return false;
    if (tid < T * 4) (&L.preL[0][0])[tid] = ld_dev(a.ws_pre + ((int64_t)g * 2 + slot) * T * 4 + tid);
    __syncthreads();

    // ---- h for this member's slice, from the residual still in registers
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
        const int tl = 16 * tm + row;
        const int64_t t = tile * T + tl;
        const double p0 = L.preL[tl][0], p1 = L.preL[tl][1], p2 = L.preL[tl][2], p3 = L.preL[tl][3];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            // 4x4 transpose across the lane groups: before, lane group g holds
            // stream g, feature pairs 0..3; after, it holds feature pair g of
            // streams 0..3.
            uint32_t v0 = f.r[tm][s][0], v1 = f.r[tm][s][1], v2 = f.r[tm][s][2], v3 = f.r[tm][s][3];
            auto x02 = __builtin_amdgcn_permlane32_swap(v0, v2, false, false);
            auto x13 = __builtin_amdgcn_permlane32_swap(v1, v3, false, false);
            v0 = x02[0]; v2 = x02[1]; v1 = x13[0]; v3 = x13[1];
            auto y01 = __builtin_amdgcn_permlane16_swap(v0, v1, false, false);
            auto y23 = __builtin_amdgcn_permlane16_swap(v2, v3, false, false);
            v0 = y01[0]; v1 = y01[1]; v2 = y23[0]; v3 = y23[1];
            double lo = p0 * (double)bf_lo(v0);
            lo = __builtin_fma(p1, (double)bf_lo(v1), lo);
            lo = __builtin_fma(p2, (double)bf_lo(v2), lo);
            lo = __builtin_fma(p3, (double)bf_lo(v3), lo);
            double hi = p0 * (double)bf_hi(v0);
            hi = __builtin_fma(p1, (double)bf_hi(v1), hi);
            hi = __builtin_fma(p2, (double)bf_hi(v2), hi);
            hi = __builtin_fma(p3, (double)bf_hi(v3), hi);
            if (t < a.n) {
                uint32_t* dst = reinterpret_cast<uint32_t*>(a.h + t * (int64_t)a.d + cw + 8 * s + 2 * grp);
                *dst = pack2(bf16_rn_f64(lo), bf16_rn_f64(hi));
            }
        }
    }
    return true;
}

template <int KS, int TM, bool FUSED>
__global__ __launch_bounds__(kThreads, 1) void k_coop(CoopArgs a) {
    constexpr int T = 16 * TM;
    __shared__ Lds<KS, TM> L;
    const int g = blockIdx.x % a.NG, q = blockIdx.x / a.NG;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63, row = l & 15, grp = l >> 4;
    const int cw = q * (32 * KS) + w * (8 * KS);
    int64_t tile = g;
    if (tile >= a.ntiles) return;

    // weights of this wave's slice, split exactly into bf16 pieces
    bf16x8 wf[KS][kTiles];
    const int64_t K = (int64_t)kHC * a.d;
#pragma unroll
    for (int ct = 0; ct < kTiles; ++ct) {
        int piece, j;
        col_map(ct, row, piece, j);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            bf16x8 v;
            if (piece < 0) {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = (__bf16)0.0f;
            } else {
                const f32x4* src = reinterpret_cast<const f32x4*>(a.W + j * K + (int64_t)grp * a.d + cw + 8 * s);
                const f32x4 w0 = src[0], w1 = src[1];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = e < 4 ? w0[e] : w1[e - 4];
                    const __bf16 hi = (__bf16)x;
                    const float r1 = x - (float)hi;
                    const __bf16 mid = (__bf16)r1;
                    const __bf16 lo = (__bf16)(r1 - (float)mid);
                    v[e] = piece == 0 ? hi : (piece == 1 ? mid : lo);
                }
            }
            wf[s][ct] = v;
        }
    }

    Frags<KS, TM> A, B;
    load_round<KS, TM>(A, a, tile, cw);
    uint32_t r = 0;
    for (;;) {
        int64_t nt = tile + a.NG;
        if (nt < a.ntiles) load_round<KS, TM>(B, a, nt, cw);
        if (!do_round<KS, TM, FUSED>(A, wf, a, L, tile, r, g, q, cw)) return;
        if (nt >= a.ntiles) break;
        tile = nt;
        ++r;
        __syncthreads();
        nt = tile + a.NG;
        if (nt < a.ntiles) load_round<KS, TM>(A, a, nt, cw);
        if (!do_round<KS, TM, FUSED>(B, wf, a, L, tile, r, g, q, cw)) return;
        if (nt >= a.ntiles) break;
        tile = nt;
        ++r;
        __syncthreads();
    }
    (void)T;
}

// Counters (and the error flag) start at zero on every call.
__global__ void k_zero(uint32_t* p, int n) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

// ------------------------------------------------------------------ host
int coop_ks(int d) {
    if (d <= 0 || d % 32 != 0) return 0;
    for (int k = 1; k <= 8; ++k)
        if (d % (32 * k) == 0 && d / (32 * k) <= 32) return k;
    return 0;
}

bool coop_plan(int64_t n, int d, CoopPlan& p) {
    const int KS = coop_ks(d);
    if (!KS) return false;
    p.KS = KS;
    p.G = d / (32 * KS);
    p.TM = n >= 4096 ? 2 : 1;
    const int T = 16 * p.TM;
    p.ntiles = (n + T - 1) / T;
    int ng = num_cus() / p.G;
    if (ng < 1) ng = 1;
    if (ng > p.ntiles) ng = (int)(p.ntiles > 0 ? p.ntiles : 1);
    p.NG = ng;
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    p.ws_part = 0;
    p.ws_pre = up((size_t)p.NG * 2 * p.G * T * kPStride * sizeof(float));
    p.ws_cnt = p.ws_pre + up((size_t)p.NG * 2 * T * 4 * sizeof(float));
    p.ws_bytes = p.ws_cnt + up(((size_t)p.NG * kCntStride + 64) * sizeof(uint32_t));
    return true;
}

template <int KS, int TM, bool FUSED>
static int launch_t(const CoopPlan& p, CoopArgs& a, hipStream_t s) {
    void* args[] = {&a};
    hipError_t e = hipLaunchCooperativeKernel((const void*)k_coop<KS, TM, FUSED>, dim3(p.G * p.NG), dim3(kThreads),
                                              args, 0, s);
    return e == hipSuccess ? 0 : -1;
}

template <int KS>
static int launch_ks(const CoopPlan& p, CoopArgs& a, bool fused, hipStream_t s) {
    if (p.TM == 1) return fused ? launch_t<KS, 1, true>(p, a, s) : launch_t<KS, 1, false>(p, a, s);
    return fused ? launch_t<KS, 2, true>(p, a, s) : launch_t<KS, 2, false>(p, a, s);
}

int launch_coop(const CoopPlan& p, const void* R, const float* W, const float* scale, const float* base,
                void* h, float* pre, float* post, float* comb, float* mixes, void* ws, int64_t n, int d,
                int iters, float eps, float norm_eps, bool fused, hipStream_t s) {
    char* wsb = static_cast<char*>(ws);
    CoopArgs a;
    a.R = static_cast<const uint16_t*>(R);
    a.W = W;
    a.scale = scale;
    a.base = base;
    a.h = static_cast<uint16_t*>(h);
    a.pre = pre;
    a.post = post;
    a.comb = comb;
    a.mixes = mixes;
    a.ws_part = reinterpret_cast<float*>(wsb + p.ws_part);
    a.ws_pre = reinterpret_cast<float*>(wsb + p.ws_pre);
    a.ws_cnt = reinterpret_cast<uint32_t*>(wsb + p.ws_cnt);
    a.n = n;
    a.ntiles = p.ntiles;
    a.d = d;
    a.G = p.G;
    a.NG = p.NG;
    a.iters = iters;
    a.eps = eps;
    a.norm_eps = norm_eps;
    a.K = (float)(kHC * d);
    k_zero<<<1, 256, 0, s>>>(a.ws_cnt, p.NG * kCntStride + 64);
    if (hipGetLastError() != hipSuccess) return -1;
    switch (p.KS) {
        case 1: return launch_ks<1>(p, a, fused, s);
        case 2: return launch_ks<2>(p, a, fused, s);
        case 3: return launch_ks<3>(p, a, fused, s);
        case 4: return launch_ks<4>(p, a, fused, s);
        case 5: return launch_ks<5>(p, a, fused, s);
        case 6: return launch_ks<6>(p, a, fused, s);
        case 7: return launch_ks<7>(p, a, fused, s);
        case 8: return launch_ks<8>(p, a, fused, s);
    }
    return -1;
}

}  // namespace hc
