// hc_general.hip -- the hyper-connection mixing for stream counts other than
// four (hc = 1..8, hc != 4).  The "Reading weights" page writes its split +
// Sinkhorn kernel for any hc_mult, and the mix formula of the "Mix
// projection" page projects the flattened hc*d stream to (2 + hc) * hc
// numbers for any hc; four streams take the tuned kernels of the other
// files.  Here every step is a plain kernel, one template instance per hc:
//
//  * k_gmm   -- projection and RMS on the matrix cores: a tile of 32..256
//               tokens per workgroup (one wave per 32), the reduction axis
//               in 64-element chunks staged through LDS, the fp32 weights
//               split exactly into three bf16 pieces (w = hi + mid + lo)
//               as they are staged, so every product is that of fp32
//               arithmetic; the sums are fp32 (v_mfma_f32_16x16x32_bf16),
//               the sums of squares come from A A^T on the same operands
//               (plain and scaled by 2^-72, for streams whose squares
//               overflow fp32).  The axis is cut into kSeg fixed segments,
//               each summed on its own and the segments added in order:
//               one workgroup may take all of them (large calls, and
//               hc_mixes, which has no workspace) or each its own with the
//               partial sums going through the workspace to k_gred (short
//               calls, to fill the chip).  The two give the same bits, and
//               the tile size does not matter to a token's sums, so a
//               token's mixes never depend on the rest of its call.
//  * k_gmm_tall -- the same sums for long fused calls at 7 or 8 streams:
//               512-token tiles with the residual loaded straight into the
//               MFMA registers, one segment per workgroup (the same bits).
//  * k_gsplit -- split + epsilon-Sinkhorn, one token per thread, with the
//               gate, softmax and normalisation arithmetic of the four-stream
//               kernel (same functions, same order).
//  * k_gpre, k_gpost -- hc_pre and hc_post over 16-byte chunks (8 features
//               of one token), summed in double in the order of the formula
//               and rounded once to bf16 (nearest even).
#include <type_traits>

#include "hc_device.hpp"
#include "hc_launch.hpp"

namespace hc {

bool gen_hc(int hc_) { return hc_ >= 1 && hc_ <= kGenMaxHC && hc_ != kHC; }

static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// Bytes of the weights split into k_gmm's B fragments: per 64-element
// chunk of the reduction axis, 2 k-steps x 3 pieces x ceil(M / 16) column
// tiles x 64 lanes of 16 bytes.
static size_t packed_gen_bytes(int hc_, int d) {
    const size_t M = (size_t)(2 + hc_) * hc_, K = (size_t)hc_ * d;
    return (K + 63) / 64 * 2 * 3 * ((M + 15) / 16) * 64 * 16;
}

constexpr int64_t kPackMinN = 1024;   // fused calls from this many tokens split the weights once

// The fused call's workspace: k_gmm's partial sums (kSeg segments of
// (2 + hc) * hc + 2 floats per token), then the mixes and pre (the minimum,
// gen_ws_min_bytes), then, for calls that split the weights once, the
// split weights (gen_ws_bytes, the size the query reports).
size_t gen_ws_min_bytes(int64_t n, int hc_, int d) {
    (void)d;
    const size_t M = (size_t)(2 + hc_) * hc_;
    return align256((size_t)n * 8 * (M + 2) * 4) + align256((size_t)n * M * 4) + align256((size_t)n * hc_ * 4);
}

size_t gen_ws_bytes(int64_t n, int hc_, int d) {
    return gen_ws_min_bytes(n, hc_, d) + (n >= kPackMinN ? align256(packed_gen_bytes(hc_, d)) : 0);
}

namespace {

constexpr int kGThreads = 256;
constexpr int kBufDword3 = 0x00020000;      // raw buffer resource, dword 3
constexpr int kBufOOB = 0x7FFFFFF0;         // buffer offset past every resource: loads read 0

// Mix formula of the "Mix projection" page: m_j = r * sum_i x_i W[j, i] with
// r = 1 / sqrt(sum_i x_i^2 / K + norm_eps), K = hc * d, over the flattened
// stream (x = R[t] read as K contiguous values).
constexpr int kSeg = 8;      // segments of the reduction axis, added in order
constexpr int kKC = 64;      // reduction elements per staged chunk (two MFMA k-steps)

template <int HC>
struct Gmm {
    static constexpr int M = (2 + HC) * HC;          // mixes per token
    static constexpr int CT = (M + 15) / 16;         // 16-column MFMA tiles
    static constexpr int F = M + 2;                  // partial fields: the M dots, sum of squares, scaled sum
};

// LDS of a k_gmm workgroup of T tokens.  a: the chunk of each token row,
// padded to 72 elements (144 bytes) so the 16 rows of an MFMA operand read
// fall on distinct banks; b: the weight pieces as MFMA B fragments,
// [k-step][piece][column tile][lane] of 8 bf16 (columns past M stay zero).
template <int HC, int T>
struct GmmLds {
    bf16x8 b[2][2][3][Gmm<HC>::CT][64];
    uint16_t a[2][T][kKC + 8];
    float ssb[T][2];
};

// Chunk ch of the reduction axis for this workgroup's tokens t0..t0+T-1,
// loaded into registers (zeros past n and past K): residual pieces of 8
// elements (token, 16-byte piece) and weight pieces of 4 (row j, 4 floats).
// PK: the weights come split already (k_gpack), as the chunk's B fragments
// (kP 16-byte words per thread).
template <int HC, int T, bool PK = false>
struct GmmRegs {
    static constexpr int kA = (T * (kKC / 8) + 2 * T - 1) / (2 * T);      // residual pieces per thread
    static constexpr int kW = PK ? 1 : (Gmm<HC>::M * (kKC / 4) + 2 * T - 1) / (2 * T);   // weight pieces per thread
    static constexpr int kFr = 2 * 3 * Gmm<HC>::CT * 64;                  // B fragments of a chunk
    static constexpr int kP = PK ? (kFr + 2 * T - 1) / (2 * T) : 1;
    uint4 a[kA];
    float4 w[kW];
    u32x4 p[kP];
};

template <int HC, int T, bool PK = false>
__device__ __forceinline__ void gmm_load(GmmRegs<HC, T, PK>& g, const uint16_t* __restrict__ R,
                                         const float* __restrict__ W, const u32x4* __restrict__ Wp, int64_t t0,
                                         int64_t n, int64_t K, int64_t ch) {
    constexpr int M = Gmm<HC>::M;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < GmmRegs<HC, T, PK>::kA; ++i) {
        const int p = i * 2 * T + tid;                  // piece p: token p / 8, elements 8 (p % 8) of the chunk
        const int tk = p >> 3;
        const int64_t k = ch * kKC + 8 * (p & 7);
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (p < T * 8 && t0 + tk < n && k < K) v = *reinterpret_cast<const uint4*>(R + (t0 + tk) * K + k);
        g.a[i] = v;
    }
    if constexpr (PK) {
        constexpr int kFr = GmmRegs<HC, T, PK>::kFr;
        const u32x4* src = Wp + ch * kFr;
#pragma unroll
        for (int i = 0; i < GmmRegs<HC, T, PK>::kP; ++i) {
            const int f = i * 2 * T + tid;
            g.p[i] = f < kFr ? src[f] : u32x4{0u, 0u, 0u, 0u};
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < GmmRegs<HC, T, PK>::kW; ++i) {
        const int p = i * 2 * T + tid;                  // piece p: row p / 16, elements 4 (p % 16) of the chunk
        const int j = p >> 4;
        const int64_t k = ch * kKC + 4 * (p & 15);
        float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (j < M && k < K) v = *reinterpret_cast<const float4*>(W + (int64_t)j * K + k);
        g.w[i] = v;
    }
}

// The loaded chunk into LDS buffer q: residual rows as they are, weights
// split into their three exact bf16 pieces in B-fragment order.
template <int HC, int T, bool PK = false>
__device__ __forceinline__ void gmm_store(const GmmRegs<HC, T, PK>& g, GmmLds<HC, T>& L, int q) {
    constexpr int M = Gmm<HC>::M;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < GmmRegs<HC, T, PK>::kA; ++i) {
        const int p = i * 2 * T + tid;
        if (p < T * 8) *reinterpret_cast<uint4*>(&L.a[q][p >> 3][8 * (p & 7)]) = g.a[i];
    }
    if constexpr (PK) {
        // the fragments as they are: L.b[q] has the same [k-step][piece][column tile][lane] order
        constexpr int kFr = GmmRegs<HC, T, PK>::kFr;
        u32x4* dst = reinterpret_cast<u32x4*>(&L.b[q][0][0][0][0]);
#pragma unroll
        for (int i = 0; i < GmmRegs<HC, T, PK>::kP; ++i) {
            const int f = i * 2 * T + tid;
            if (f < kFr) dst[f] = g.p[i];
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < GmmRegs<HC, T, PK>::kW; ++i) {
        const int p = i * 2 * T + tid;
        const int j = p >> 4;
        if (j >= M) continue;
        const int kc = 4 * (p & 15);                   // element of the chunk
        const int st = kc >> 5, kk = kc & 31, grp = kk >> 3, e0 = kk & 7;
        const int ct = j >> 4, lane = (j & 15) + 16 * grp;
        const float x[4] = {g.w[i].x, g.w[i].y, g.w[i].z, g.w[i].w};
        uint32_t pc[3][2];
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
            uint32_t hw[3][2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const float v = x[e + u];
                const __bf16 hi = (__bf16)v;
                const float r1 = v - (float)hi;
                const __bf16 mid = (__bf16)r1;
                const __bf16 lo = (__bf16)(r1 - (float)mid);
                hw[0][u] = (uint32_t)__builtin_bit_cast(uint16_t, hi);
                hw[1][u] = (uint32_t)__builtin_bit_cast(uint16_t, mid);
                hw[2][u] = (uint32_t)__builtin_bit_cast(uint16_t, lo);
            }
#pragma unroll
            for (int pc_ = 0; pc_ < 3; ++pc_) pc[pc_][e >> 1] = pack2(hw[pc_][0], hw[pc_][1]);
        }
#pragma unroll
        for (int pc_ = 0; pc_ < 3; ++pc_)
            *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(&L.b[q][st][pc_][ct][lane]) + e0) =
                u32x2{pc[pc_][0], pc[pc_][1]};
    }
}

// The weights split once per call (k_gpack): chunk ch of the reduction
// axis as the B fragments gmm_store forms in LDS, [ch][k-step][piece]
// [column tile][lane] of 8 bf16, columns past M zero.  Thread = (chunk,
// row j of the column tiles, 4 elements), with gmm_store's arithmetic, so
// a packed call's fragments are bitwise an unpacked call's.
template <int HC>
__global__ __launch_bounds__(kGThreads) void k_gpack(const float* __restrict__ W, bf16x8* __restrict__ out,
                                                     int64_t K) {
    constexpr int M = Gmm<HC>::M, CT = Gmm<HC>::CT;
    const int64_t C = (K + kKC - 1) / kKC;
    const int64_t items = C * (16 * CT) * 16;
    for (int64_t it = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; it < items;
         it += (int64_t)gridDim.x * blockDim.x) {
        const int64_t ch = it / (16 * CT * 16);
        const int rem = (int)(it - ch * (16 * CT * 16));
        const int j = rem >> 4;                         // row of the column tiles (j >= M: padding)
        const int kc = 4 * (rem & 15);                  // element of the chunk
        const int st = kc >> 5, kk = kc & 31, grp = kk >> 3, e0 = kk & 7;
        const int ct = j >> 4, lane = (j & 15) + 16 * grp;
        const int64_t k = ch * kKC + kc;
        float x[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (j < M && k < K) {
            const float4 v = *reinterpret_cast<const float4*>(W + (int64_t)j * K + k);
            x[0] = v.x;
            x[1] = v.y;
            x[2] = v.z;
            x[3] = v.w;
        }
        uint32_t pc[3][2];
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
            uint32_t hw[3][2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const float v = x[e + u];
                const __bf16 hi = (__bf16)v;
                const float r1 = v - (float)hi;
                const __bf16 mid = (__bf16)r1;
                const __bf16 lo = (__bf16)(r1 - (float)mid);
                hw[0][u] = (uint32_t)__builtin_bit_cast(uint16_t, hi);
                hw[1][u] = (uint32_t)__builtin_bit_cast(uint16_t, mid);
                hw[2][u] = (uint32_t)__builtin_bit_cast(uint16_t, lo);
            }
#pragma unroll
            for (int pc_ = 0; pc_ < 3; ++pc_) pc[pc_][e >> 1] = pack2(hw[pc_][0], hw[pc_][1]);
        }
        bf16x8* base = out + ch * (2 * 3 * CT * 64);
#pragma unroll
        for (int pc_ = 0; pc_ < 3; ++pc_)
            *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(&base[((st * 3 + pc_) * CT + ct) * 64 + lane]) + e0) =
                u32x2{pc[pc_][0], pc[pc_][1]};
    }
}

// Per-wave sums of one 32-token slice: tt = 16-token MFMA tile.
template <int HC>
struct GmmAcc {
    f32x4 dot[2][Gmm<HC>::CT];
    f32x4 sq[2], sb[2];
};

template <int HC>
__device__ __forceinline__ void gmm_zero(GmmAcc<HC>& A) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
        for (int ct = 0; ct < Gmm<HC>::CT; ++ct) A.dot[tt][ct] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        A.sq[tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        A.sb[tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
}

// Products of LDS buffer q for this wave's 32 tokens: per k-step, each
// column tile takes the hi, mid and lo pieces into one accumulator, and
// the operand against itself gives the sums of squares on the diagonal.
template <int HC, int T>
__device__ __forceinline__ void gmm_mma(GmmAcc<HC>& A, const GmmLds<HC, T>& L, int q) {
    const int l = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int row = l & 15, grp = l >> 4;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        bf16x8 ab[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const u32x4 av = *reinterpret_cast<const u32x4*>(&L.a[q][32 * wv + 16 * tt + row][32 * st + 8 * grp]);
            ab[tt] = __builtin_bit_cast(bf16x8, av);
            A.sq[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ab[tt], ab[tt], A.sq[tt], 0, 0, 0);
            const u32x4 as = u32x4{scaled_x2(av[0]), scaled_x2(av[1]), scaled_x2(av[2]), scaled_x2(av[3])};
            const bf16x8 sbf = __builtin_bit_cast(bf16x8, as);
            A.sb[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sbf, sbf, A.sb[tt], 0, 0, 0);
        }
        // each weight fragment is read once for both 16-token tiles (LDS
        // bandwidth, not the matrix cores, bounds this loop at many outputs)
#pragma unroll
        for (int ct = 0; ct < Gmm<HC>::CT; ++ct)
#pragma unroll
            for (int pc = 0; pc < 3; ++pc) {
                const bf16x8 b = L.b[q][st][pc][ct][l];
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
                    A.dot[tt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ab[tt], b, A.dot[tt][ct], 0, 0, 0);
            }
        // one k-step's fragments at a time: loaded further ahead they
        // would take the registers of the sums
        asm volatile("" ::: "memory");
    }
}

// One workgroup: token tile blockIdx.x / G, segments sg * (kSeg / G) ..
// (sg + 1) * (kSeg / G) - 1 with sg = blockIdx.x % G (G = 1 or kSeg).
// Segment s covers chunks s*C/kSeg .. (s+1)*C/kSeg - 1 (C = chunks of K);
// its sums start from zero and are added to the previous segments' total in
// order.  G = 1: the totals give the mixes here.  G = kSeg: each segment's
// sums go to part[t][s][F] (the dots, then the two sums of squares), and
// k_gred adds them in the same order.
template <int HC, int T, bool PK = false>
__global__ __launch_bounds__(2 * T) void k_gmm(const uint16_t* __restrict__ R, const float* __restrict__ W,
                                               const u32x4* __restrict__ Wp, float* __restrict__ mixes,
                                               float* __restrict__ part, int64_t n, int d, int G, float norm_eps) {
    constexpr int M = Gmm<HC>::M, CT = Gmm<HC>::CT, F = Gmm<HC>::F;
    __shared__ __attribute__((aligned(16))) GmmLds<HC, T> L;
    const int64_t K = (int64_t)HC * d;
    const int64_t C = (K + kKC - 1) / kKC;
    const int64_t tile = blockIdx.x / G;
    const int sg = (int)(blockIdx.x - tile * G);
    const int per = kSeg / G;
    const int64_t t0 = tile * T;
    const int l = threadIdx.x & 63, wv = threadIdx.x >> 6;
    // the padding columns of the weight fragments stay zero
    for (int i = threadIdx.x; i < (int)(sizeof(L.b) / 16); i += 2 * T)
        reinterpret_cast<uint4*>(&L.b[0][0][0][0][0])[i] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();

    GmmAcc<HC> tot, seg;
    gmm_zero<HC>(tot);
    gmm_zero<HC>(seg);
    const int s0 = sg * per, s1 = s0 + per;
    const int64_t c0 = s0 * C / kSeg, c1 = s1 * C / kSeg;
    // chunks in flight: kPD register sets, chunk c in set (c - c0) % kPD,
    // each loaded kPD - 1 chunks ahead of its turn in LDS
    constexpr int kPD = Gmm<HC>::M > 48 ? 2 : 3;
    GmmRegs<HC, T, PK> g[kPD];
    int s = s0;
    int64_t send = (int64_t)(s + 1) * C / kSeg;        // first chunk past segment s
#pragma unroll
    for (int i = 0; i < kPD; ++i)
        if (c0 + i < c1) gmm_load<HC, T, PK>(g[i], R, W, Wp, t0, n, K, c0 + i);
    if (c0 < c1) gmm_store<HC, T, PK>(g[0], L, 0);
    __syncthreads();
    auto close = [&]() {
        // segment s complete: into the total (or the partial sums)
        if (G == 1) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) tot.dot[tt][ct] = s == 0 ? seg.dot[tt][ct] : tot.dot[tt][ct] + seg.dot[tt][ct];
                tot.sq[tt] = s == 0 ? seg.sq[tt] : tot.sq[tt] + seg.sq[tt];
                tot.sb[tt] = s == 0 ? seg.sb[tt] : tot.sb[tt] + seg.sb[tt];
            }
        } else {
            const int row = l & 15, grp = l >> 4;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t t = t0 + 32 * wv + 16 * tt + 4 * grp + r;
                    float* pt = part + (t * kSeg + s) * F;
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct)
                        if (t < n && 16 * ct + row < M) pt[16 * ct + row] = seg.dot[tt][ct][r];
                    // the diagonal of A A^T: token 4 grp + r of the tile is row == 4 grp + r
                    if (t < n && row == 4 * grp + r) {
                        pt[M] = seg.sq[tt][r];
                        pt[M + 1] = seg.sb[tt][r];
                    }
                }
        }
        gmm_zero<HC>(seg);
    };
    // empty segments before the first chunk (short axes)
    while (s < s1 && send <= c0) {
        close();
        ++s;
        send = (int64_t)(s + 1) * C / kSeg;
    }
    // chunk ch (in set I): its products from LDS buffer (ch - c0) & 1,
    // then chunk ch + 1 (set I + 1) into the other buffer, and set I
    // refilled with chunk ch + kPD
    auto step = [&](int64_t ch, auto I) {
        constexpr int i = decltype(I)::value;
        const int q = (int)((ch - c0) & 1);
        gmm_mma<HC, T>(seg, L, q);
        // segments that end here (and empty ones after them)
        while (s < s1 && send <= ch + 1) {
            close();
            ++s;
            send = (int64_t)(s + 1) * C / kSeg;
        }
        if (ch + 1 < c1) gmm_store<HC, T, PK>(g[(i + 1) % kPD], L, q ^ 1);
        if (ch + kPD < c1) gmm_load<HC, T, PK>(g[i], R, W, Wp, t0, n, K, ch + kPD);
        __syncthreads();
    };
    for (int64_t ch = c0; ch < c1; ch += kPD) {
        step(ch, std::integral_constant<int, 0>{});
        if (ch + 1 < c1) step(ch + 1, std::integral_constant<int, 1>{});
        if constexpr (kPD > 2)
            if (ch + 2 < c1) step(ch + 2, std::integral_constant<int, 2>{});
    }
    while (s < s1) {            // empty segments at the end
        close();
        ++s;
    }
    if (G != 1) return;
    // the mixes of this wave's 32 tokens: sums of squares from the diagonal
    const int row = l & 15, grp = l >> 4;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (row == 4 * grp + r) {
                L.ssb[32 * wv + 16 * tt + row][0] = tot.sq[tt][r];
                L.ssb[32 * wv + 16 * tt + row][1] = tot.sb[tt][r];
            }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");     // the wave reads back its own LDS writes
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int tl = 32 * wv + 16 * tt + 4 * grp + r;
            const int64_t t = t0 + tl;
            const MixScale ms = mix_scale(L.ssb[tl][0], L.ssb[tl][1], (float)K, norm_eps);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
                if (t < n && 16 * ct + row < M) mixes[t * M + 16 * ct + row] = mix_value(tot.dot[tt][ct][r], ms);
        }
}

// Tall tiles for long fused calls (weights split once, a workspace for the
// partial sums): a workgroup takes 512 tokens (8 waves of 64) and one of
// the kSeg segments, loads the residual straight from HBM into the MFMA A
// registers (two chunks ahead, no LDS), and stages only the split weights
// through LDS.  A segment's weight pieces are then read once per 512 tokens
// (k_gmm: per tile of at most 256, with the tile's residual rows in LDS
// beside them), and each weight fragment read from LDS serves four 16-token
// MFMA tiles.  Every accumulator sees k_gmm's sequence of MFMAs (per k-step
// the hi, mid and lo pieces; the sums of squares from A A^T), the segment's
// sums go to the workspace as in k_gmm's segment mode and k_gred adds them
// in order: the bits are k_gmm's.  Every chunk step issues the same memory
// instructions (chunks past the segment lie outside their buffer
// resources: zeros in), so the loop body is straight-line and the loads of
// the next chunks stay in flight across its waits.
constexpr int kTallT = 512;                 // tokens per workgroup
constexpr int64_t kTallMinN = 16384;        // from here the tall tiles fill the chip on their own
// Stream counts whose weights the tall tiles pay for: more than 48 mixes
// (hc = 7, 8).  At hc = 8 the fused call took 2,598 against 2,960 us at
// 65,536 tokens, d = 5120, at hc = 7 2,175 against 2,339 us; at hc = 5 and 6
// (35 and 48 mixes, the residual's bytes dominating) k_gmm was 1-2 % faster.
constexpr int kTallMinM = 48;

template <int HC>
struct TallLds {
    bf16x8 b[2][2][3][Gmm<HC>::CT][64];     // the chunk's B fragments, by chunk parity
};

template <int HC>
__global__ __launch_bounds__(512, 1) void k_gmm_tall(const uint16_t* __restrict__ R, const u32x4* __restrict__ Wp,
                                                     float* __restrict__ part, int64_t n, int d) {
    constexpr int M = Gmm<HC>::M, CT = Gmm<HC>::CT, F = Gmm<HC>::F;
    constexpr int kFr = 2 * 3 * CT * 64;                   // 16-byte B fragments per chunk
    constexpr int kP = (kFr + 511) / 512;                  // per thread
    __shared__ __attribute__((aligned(16))) TallLds<HC> L;
    const int64_t K = (int64_t)HC * d;
    const int64_t C = (K + kKC - 1) / kKC;
    const int64_t tile = blockIdx.x / kSeg;
    const int sg = (int)(blockIdx.x % kSeg);
    const int tid = threadIdx.x, l = tid & 63, wv = tid >> 6;
    const int row = l & 15, grp = l >> 4;
    const int64_t c0 = sg * C / kSeg, c1 = (sg + 1) * C / kSeg;
    // the wave's 64 token rows as a buffer resource (rows past n outside it)
    const int64_t tw = tile * kTallT + 64 * wv;
    int64_t rows = n - tw;
    rows = rows < 0 ? 0 : (rows > 64 ? 64 : rows);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(R) + (rows > 0 ? tw : 0) * K, 0, (int)(rows * K * 2), kBufDword3);
    // the segment's split weights: chunks c0 .. c1 - 1
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<u32x4*>(Wp) + c0 * kFr, 0, (int)((c1 - c0) * kFr * 16), kBufDword3);
    // A pieces of chunk ch: [16-token tile][k-step]; k past K reads zeros
    auto load_a = [&](u32x4 (&a)[4][2], int64_t ch) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                const int64_t k = ch * kKC + 32 * st + 8 * grp;
                const int off = ch < c1 && k < K ? (int)(((int64_t)(16 * tt + row) * K + k) * 2) : kBufOOB;
                a[tt][st] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0));
            }
    };
    auto load_b = [&](u32x4 (&p)[kP], int64_t ch) {
#pragma unroll
        for (int i = 0; i < kP; ++i) {
            const int f = i * 512 + tid;
            const int off = ch < c1 && f < kFr ? (int)(((ch - c0) * kFr + f) * 16) : kBufOOB;
            p[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, 0));
        }
    };
    auto store_b = [&](const u32x4 (&p)[kP], int q) {
        u32x4* dst = reinterpret_cast<u32x4*>(&L.b[q][0][0][0][0]);
#pragma unroll
        for (int i = 0; i < kP; ++i) {
            const int f = i * 512 + tid;
            if (f < kFr) dst[f] = p[i];
        }
    };
    f32x4 dot[4][CT], sq[4], sb[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) dot[tt][ct] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        sq[tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        sb[tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    // products of one chunk from A registers a and LDS buffer q (k_gmm's
    // order for every accumulator)
    auto mma = [&](const u32x4 (&a)[4][2], int q) {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            bf16x8 ab[4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const u32x4 av = a[tt][st];
                ab[tt] = __builtin_bit_cast(bf16x8, av);
                sq[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ab[tt], ab[tt], sq[tt], 0, 0, 0);
                const u32x4 as = u32x4{scaled_x2(av[0]), scaled_x2(av[1]), scaled_x2(av[2]), scaled_x2(av[3])};
                const bf16x8 sbf = __builtin_bit_cast(bf16x8, as);
                sb[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sbf, sbf, sb[tt], 0, 0, 0);
            }
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int pc = 0; pc < 3; ++pc) {
                    const bf16x8 b = L.b[q][st][pc][ct][l];
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt)
                        dot[tt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ab[tt], b, dot[tt][ct], 0, 0, 0);
                }
            asm volatile("" ::: "memory");
        }
    };
    if (c0 < c1) {
        u32x4 a0[4][2], a1[4][2], pb[kP];
        load_b(pb, c0);
        store_b(pb, 0);
        load_b(pb, c0 + 1);
        load_a(a0, c0);
        load_a(a1, c0 + 1);
        __syncthreads();
        // chunk ch from a0 / buffer 0, chunk ch + 1 from a1 / buffer 1; the
        // weights of the next chunk go to the other buffer before the
        // barrier, and each register set is refilled two chunks ahead
        int64_t ch = c0;
        for (; ch + 1 < c1; ch += 2) {
            mma(a0, 0);
            store_b(pb, 1);                 // chunk ch + 1
            load_b(pb, ch + 2);
            load_a(a0, ch + 2);
            __syncthreads();
            mma(a1, 1);
            store_b(pb, 0);                 // chunk ch + 2
            load_b(pb, ch + 3);
            load_a(a1, ch + 3);
            __syncthreads();
        }
        if (ch < c1) mma(a0, 0);            // an odd last chunk
    }
    // the segment's sums: lane (row, grp) holds tokens 4 grp + r of each
    // 16-token tile for column row; the sums of squares are the diagonal
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t t = tw + 16 * tt + 4 * grp + r;
            if (t >= n) continue;
            float* pt = part + (t * kSeg + sg) * F;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
                if (16 * ct + row < M) pt[16 * ct + row] = dot[tt][ct][r];
            if (row == 4 * grp + r) {
                pt[M] = sq[tt][r];
                pt[M + 1] = sb[tt][r];
            }
        }
}

// The partial sums of k_gmm's segments, added in segment order (the order
// of a workgroup that takes them all), then the mixes.  One thread per token.
template <int HC>
__global__ __launch_bounds__(kGThreads) void k_gred(const float* __restrict__ part, float* __restrict__ mixes,
                                                    int64_t n, float K, float norm_eps) {
    constexpr int M = Gmm<HC>::M, F = Gmm<HC>::F;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n; t += stride) {
        const float* p = part + t * kSeg * F;
        float acc[F];
#pragma unroll
        for (int f = 0; f < F; ++f) acc[f] = p[f];
        for (int s = 1; s < kSeg; ++s)
#pragma unroll
            for (int f = 0; f < F; ++f) acc[f] = acc[f] + p[s * F + f];
        const MixScale ms = mix_scale(acc[M], acc[M + 1], K, norm_eps);
#pragma unroll
        for (int j = 0; j < M; ++j) mixes[t * M + j] = mix_value(acc[j], ms);
    }
}

// Split + epsilon-Sinkhorn of the "Reading weights" page for hc streams:
// pre_j = sigmoid(s0 m_j + b_j) + eps, post_j = 2 sigmoid(s1 m_{hc+j} +
// b_{hc+j}), logits s2 m_{2hc + j hc + k} + b_{2hc + j hc + k}; a row softmax
// plus eps, a column normalisation, then (iters - 1) row and column
// normalisations, each dividing by (sum + eps).
template <int HC>
// scrub (the fused call): the workspace's first 256 bytes, zeroed here so
// that a four-stream call on the same workspace later finds no valid header
// and clears its record area (they belong to the partial sums, which k_gmm
// and k_gred are done with by now).
__global__ __launch_bounds__(kGThreads) void k_gsplit(const float* __restrict__ mixes, const float* __restrict__ scale,
                                                      const float* __restrict__ base, float* __restrict__ pre,
                                                      float* __restrict__ post, float* __restrict__ comb, int64_t n,
                                                      int iters, float eps, uint32_t* __restrict__ scrub) {
    constexpr int M = (2 + HC) * HC;
    if (scrub && blockIdx.x == 0 && threadIdx.x < 64) scrub[threadIdx.x] = 0u;
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

// hc_pre of the "Mix projection" page: h_c = bf16(sum_k pre_k R_{k,c}),
// summed in double in stream order and rounded once (the float fast path
// of f32_mid, redone with bf16_rn_f64 by a wave in which any lane hit a
// float halfway point: the same bits either way).  Streaming accesses are
// non-temporal; a wave's 64 chunks share one token when 8 * 64 divides d,
// and its pre then comes through scalar loads.
template <int HC>
__global__ __launch_bounds__(kGThreads) void k_gpre(const uint16_t* __restrict__ R, const float* __restrict__ pre,
                                                    uint16_t* __restrict__ h, int64_t n, int d) {
    const int cpt = d / 8;
    const bool uniform = cpt % 64 == 0;
    const int64_t items = n * cpt;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t it = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; it < items; it += stride) {
        int64_t t = it / cpt;
        if (uniform)
            t = (int64_t)__builtin_amdgcn_readfirstlane((uint32_t)t) |
                ((int64_t)__builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)t >> 32)) << 32);
        const int c0 = (int)(it - t * cpt) * 8;
        u32x4 r[HC];
        double p[HC];
#pragma unroll
        for (int k = 0; k < HC; ++k) {
            r[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(R + (t * HC + k) * d + c0));
            p[k] = pre[t * HC + k];
        }
        auto sum = [&](int w, int e) {
            double y = p[0] * (double)(e ? bf_hi(r[0][w]) : bf_lo(r[0][w]));
#pragma unroll
            for (int k = 1; k < HC; ++k) y = __builtin_fma(p[k], (double)(e ? bf_hi(r[k][w]) : bf_lo(r[k][w])), y);
            return y;
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
        __builtin_nontemporal_store(out, reinterpret_cast<u32x4*>(h + t * d + c0));
    }
}

// hc_post of the "Mix projection" page: output stream k is
// bf16(post_k x_c + sum_j comb[j][k] R_{j,c}), the double sum rounded once.
// An item reads every stream of its chunk before writing any, and the next
// item's loads (issued early) touch only that item's chunk, so R_out may be
// R.  Up to 6 streams (k_gpost_lean beyond).
template <int HC>
__global__ __launch_bounds__(kGThreads) void k_gpost(const uint16_t* __restrict__ x, const uint16_t* R,
                                                     const float* __restrict__ post, const float* __restrict__ comb,
                                                     uint16_t* Rout, int64_t n, int d) {
    const int cpt = d / 8;
    const int64_t items = n * cpt;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t it = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (it >= items) return;
    struct Item {
        int64_t t;
        int c0;
        u32x4 xv, r[HC];
    };
    // the next item's loads are in flight while this item is computed; past
    // the end the last item is loaded again (no branch around the loads)
    auto fetch = [&](int64_t i, Item& I) {
        const int64_t ii = i < items ? i : items - 1;
        I.t = ii / cpt;
        I.c0 = (int)(ii - I.t * cpt) * 8;
        I.xv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + I.t * d + I.c0));
#pragma unroll
        for (int j = 0; j < HC; ++j)
            I.r[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(R + (I.t * HC + j) * d + I.c0));
    };
    auto bf = [](const u32x4& v, int e) { return (double)((e & 1) ? bf_hi(v[e >> 1]) : bf_lo(v[e >> 1])); };
    Item cur, nxt;
    fetch(it, cur);
    for (; it < items; it += stride) {
        fetch(it + stride, nxt);
        const int64_t t = cur.t;
#pragma unroll
        for (int k = 0; k < HC; ++k) {
            const double pk = post[t * HC + k];
            double cj[HC];
#pragma unroll
            for (int j = 0; j < HC; ++j) cj[j] = comb[(t * HC + j) * HC + k];
            auto sum = [&](int e) {
                double y = pk * bf(cur.xv, e);
#pragma unroll
                for (int j = 0; j < HC; ++j) y = __builtin_fma(cj[j], bf(cur.r[j], e), y);
                return y;
            };
            // each output is bf16_rn_f64 of its double sum: through the float
            // rounding unless a lane of the wave hit a float halfway point
            float f[8];
            bool mid = false;
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = f32_mid(sum(e), mid);
            uint32_t o[8];
            if (__builtin_amdgcn_ballot_w64(mid)) {
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = bf16_rn_f64(sum(e));
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = bf16_rn(f[e]);
            }
            const uint4 pk8 = pack8(o);
            __builtin_nontemporal_store(u32x4{pk8.x, pk8.y, pk8.z, pk8.w},
                                        reinterpret_cast<u32x4*>(Rout + (t * HC + k) * d + cur.c0));
        }
        cur = nxt;
    }
}

// hc_post for 7 and 8 streams: k_gpost's arithmetic without its prefetch
// and fast path, whose registers (a second item of up to 8 streams) cost
// more in resident waves than they gain there.  Each output is the same
// bf16_rn_f64 of the same double sum.
template <int HC>
__global__ __launch_bounds__(kGThreads) void k_gpost_lean(const uint16_t* __restrict__ x, const uint16_t* R,
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

// Bytes of k_gmm's per-segment partial sums for n tokens.
template <int HC>
size_t gmm_part_bytes(int64_t n) { return align256((size_t)n * kSeg * Gmm<HC>::F * 4); }

template <int HC, int T>
int gmm_launch(const void* R, const float* W, const u32x4* Wp, float* mixes, float* part, int64_t n, int d, int G,
               float norm_eps, hipStream_t s) {
    const int64_t tiles = (n + T - 1) / T;
    if (Wp)
        hipLaunchKernelGGL((k_gmm<HC, T, true>), dim3((unsigned)(tiles * G)), dim3(2 * T), 0, s,
                           static_cast<const uint16_t*>(R), W, Wp, mixes, part, n, d, G, norm_eps);
    else
        hipLaunchKernelGGL((k_gmm<HC, T, false>), dim3((unsigned)(tiles * G)), dim3(2 * T), 0, s,
                           static_cast<const uint16_t*>(R), W, Wp, mixes, part, n, d, G, norm_eps);
    if (hipGetLastError() != hipSuccess) return -1;
    if (G != 1) {
        hipLaunchKernelGGL(k_gred<HC>, dim3(grid_for(n)), dim3(kGThreads), 0, s, part, mixes, n,
                           (float)((int64_t)HC * d), norm_eps);
        if (hipGetLastError() != hipSuccess) return -1;
    }
    return 0;
}

// The projection.  With the weights split once and a workspace for the
// partial sums, long calls at 7 or 8 streams take k_gmm_tall.  Otherwise tiles of 256 tokens
// while they fill the compute units on their own; shorter calls take
// smaller tiles, and with a workspace for the partial sums (part) one
// workgroup per segment as well.  Every choice gives the same bits.
template <int HC>
struct MixOp {
    static int run(const void* R, const float* W, const u32x4* Wp, float* mixes, float* part, int64_t n, int d,
                   float norm_eps, hipStream_t s) {
        if (Gmm<HC>::M > kTallMinM && Wp && part && n >= kTallMinN &&
            (int64_t)HC * d * 2 * kTallT < ((int64_t)1 << 31)) {
            const int64_t tiles = (n + kTallT - 1) / kTallT;
            hipLaunchKernelGGL(k_gmm_tall<HC>, dim3((unsigned)(tiles * kSeg)), dim3(512), 0, s,
                               static_cast<const uint16_t*>(R), Wp, part, n, d);
            if (hipGetLastError() != hipSuccess) return -1;
            hipLaunchKernelGGL(k_gred<HC>, dim3(grid_for(n)), dim3(kGThreads), 0, s, part, mixes, n,
                               (float)((int64_t)HC * d), norm_eps);
            return hipGetLastError() == hipSuccess ? 0 : -1;
        }
        const int64_t cus = num_cus();
        const int G = (part && (n + 255) / 256 < cus) ? kSeg : 1;
        const int64_t want = G == 1 ? cus : (cus + kSeg - 1) / kSeg;      // tiles that fill the chip
        // smallest tile: the weight chunk (M x 64 floats) spread over its
        // threads stays within 8 loads each
        constexpr int M = Gmm<HC>::M;
        // at 8 mixes or fewer, 128-token tiles stream faster (two workgroups
        // per CU): 547 against 565 us at hc = 2, 65,536 tokens
        if (M > 8 && (n + 255) / 256 >= want) return gmm_launch<HC, 256>(R, W, Wp, mixes, part, n, d, G, norm_eps, s);
        if constexpr (M > 48) return gmm_launch<HC, 128>(R, W, Wp, mixes, part, n, d, G, norm_eps, s);
        if ((n + 127) / 128 >= want) return gmm_launch<HC, 128>(R, W, Wp, mixes, part, n, d, G, norm_eps, s);
        if constexpr (M > 16) return gmm_launch<HC, 64>(R, W, Wp, mixes, part, n, d, G, norm_eps, s);
        if ((n + 63) / 64 >= want) return gmm_launch<HC, 64>(R, W, Wp, mixes, part, n, d, G, norm_eps, s);
        return gmm_launch<HC, 32>(R, W, Wp, mixes, part, n, d, G, norm_eps, s);
    }
};

template <int HC>
struct PackOp {
    static int run(const float* W, void* out, int d, hipStream_t s) {
        const int64_t K = (int64_t)HC * d;
        const int64_t items = (K + kKC - 1) / kKC * (16 * Gmm<HC>::CT) * 16;
        int64_t blocks = (items + kGThreads - 1) / kGThreads;
        if (blocks > (int64_t)num_cus() * 8) blocks = (int64_t)num_cus() * 8;
        hipLaunchKernelGGL(k_gpack<HC>, dim3((unsigned)blocks), dim3(kGThreads), 0, s, W,
                           static_cast<bf16x8*>(out), K);
        return hipGetLastError() == hipSuccess ? 0 : -1;
    }
};

template <int HC>
struct PartOp {
    static int run(int64_t n, size_t* out) {
        *out = gmm_part_bytes<HC>(n);
        return 0;
    }
};

template <int HC>
struct SplitOp {
    static int run(const float* mixes, const float* scale, const float* base, float* pre, float* post, float* comb,
                   int64_t n, int iters, float eps, uint32_t* scrub, hipStream_t s) {
        hipLaunchKernelGGL(k_gsplit<HC>, dim3(grid_for(n)), dim3(kGThreads), 0, s, mixes, scale, base, pre, post,
                           comb, n, iters, eps, scrub);
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
        if constexpr (HC <= 6)
            hipLaunchKernelGGL(k_gpost<HC>, dim3(grid_for(n * (d / 8))), dim3(kGThreads), 0, s,
                               static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(R), post, comb,
                               static_cast<uint16_t*>(Rout), n, d);
        else
            hipLaunchKernelGGL(k_gpost_lean<HC>, dim3(grid_for(n * (d / 8))), dim3(kGThreads), 0, s,
                               static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(R), post, comb,
                               static_cast<uint16_t*>(Rout), n, d);
        return hipGetLastError() == hipSuccess ? 0 : -1;
    }
};

}  // namespace

int launch_gen_mixes(const void* R, const float* W, float* mixes, int64_t n, int hc_, int d, float norm_eps,
                     hipStream_t s) {
    return dispatch_hc<MixOp>(hc_, R, W, (const u32x4*)nullptr, mixes, (float*)nullptr, n, d, norm_eps, s);
}

int launch_gen_split(const float* mixes, const float* scale, const float* base, float* pre, float* post,
                     float* comb, int64_t n, int hc_, int iters, float eps, hipStream_t s) {
    return dispatch_hc<SplitOp>(hc_, mixes, scale, base, pre, post, comb, n, iters, eps, (uint32_t*)nullptr, s);
}

int launch_gen_pre(const void* R, const float* pre, void* h, int64_t n, int hc_, int d, hipStream_t s) {
    return dispatch_hc<PreOp>(hc_, R, pre, h, n, d, s);
}

int launch_gen_post(const void* x, const void* R, const float* post, const float* comb, void* Rout, int64_t n,
                    int hc_, int d, hipStream_t s) {
    return dispatch_hc<PostOp>(hc_, x, R, post, comb, Rout, n, d, s);
}

int launch_gen_fused(const void* R, const float* W, const float* scale, const float* base, void* h, float* pre,
                     float* post, float* comb, float* mixes, void* ws, size_t ws_bytes, int64_t n, int hc_, int d,
                     int iters, float eps, float norm_eps, hipStream_t s) {
    // the workspace holds the projection's partial sums, then the mixes and
    // pre when the caller does not keep them, then the weights split once
    // for this call; its first 256 bytes (a four-stream call's header) are
    // zeroed by the split kernel, so that a later four-stream call on the
    // same workspace takes it as fresh (clearing its record area) rather
    // than trusting stale contents
    const size_t M = (size_t)(2 + hc_) * hc_;
    char* w = static_cast<char*>(ws);
    size_t pb = 0;
    if (dispatch_hc<PartOp>(hc_, n, &pb)) return -1;
    float* part = reinterpret_cast<float*>(w);
    size_t off = pb;
    float* mx = mixes ? mixes : reinterpret_cast<float*>(w + off);
    if (!mixes) off += align256((size_t)n * M * 4);
    float* pr = pre ? pre : reinterpret_cast<float*>(w + off);
    // calls of many tiles split the weights once (every 256-token tile
    // would otherwise split all of them again), when the workspace holds
    // them; short calls split them as they are staged, which saves the extra
    // launch.  Both give the same fragments, so the same bits.
    const void* wp = nullptr;
    if (n >= kPackMinN && ws_bytes >= gen_ws_bytes(n, hc_, d)) {
        void* dst = w + gen_ws_min_bytes(n, hc_, d);
        if (dispatch_hc<PackOp>(hc_, W, dst, d, s)) return -1;
        wp = dst;
    }
    if (dispatch_hc<MixOp>(hc_, R, W, (const u32x4*)wp, mx, part, n, d, norm_eps, s)) return -1;
    if (dispatch_hc<SplitOp>(hc_, mx, scale, base, pr, post, comb, n, iters, eps, reinterpret_cast<uint32_t*>(w), s))
        return -1;
    // h with hc_pre's one-token-per-workgroup kernel where it applies (the
    // same exact double sums and one rounding as k_gpre)
    if (norm_waves(d)) return launch_pre_norm(R, pr, nullptr, h, nullptr, n, hc_, d, 0.0f, s);
    return launch_gen_pre(R, pr, h, n, hc_, d, s);
}

}  // namespace hc
