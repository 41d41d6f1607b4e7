// hc_coop.hip -- the mix projection ("Mix projection" page, mix formula)
// and the fused projection + split/Sinkhorn + hc_pre, as one persistent,
// cooperatively launched kernel.
//
// Why this shape.  Every token needs all 24 x 4d projection weights
// (1.97 MB in fp32), and hc_pre needs the token's residual a second time,
// after the whole 4d-long reduction is known.  A tile of tokens large
// enough to amortise the weights does not fit on one CU, so the 4d
// reduction is split across the CUs of a group instead:
//
//  * G workgroups (one per CU) form a group.  Member q owns a 32*KS-feature
//    slice of every stream (d = 5120: G = 32, 160 features, KS = 5) and
//    keeps that slice of the weights resident in LDS for the whole kernel,
//    split exactly into three bf16 pieces (w = hi + mid + lo) laid out as
//    80 MFMA columns (3 x 24 used): the products are exact, sums are fp32.
//  * A round is T = 32 tokens.  Each of the 8 waves takes one 16-token tile
//    and one of 4 k-groups of the slice and runs v_mfma_f32_16x16x32_bf16
//    on the bf16 residual straight from registers; it also forms the sum of
//    squares.  The member's 25 partial sums per token are published to the
//    workspace as tagged 16-byte records (3 floats + a round tag).
//  * Every member then reads the pre-relevant partials of all G members
//    (m_0..m_3 and the sum of squares), forms pre for all T tokens in one
//    fixed order, and writes h for its slice from the residual still in
//    registers: one HBM pass over the residual.  The owner of each token
//    (member t mod G) also reads all 25 partials, forms the mixes and runs
//    the split + Sinkhorn on one 16-lane row.
//  * Rounds are software-pipelined: in iteration i a wave issues its
//    exchange loads for round i, then the residual loads for round i+3, then
//    the projection and publication of round i+1, the owner's Sinkhorn of
//    round i-1, and finally pre and h of round i.  A wave's loads retire in
//    issue order, so exchange loads go out before residual prefetches, and
//    nothing waits for a store to complete: readers check tags instead.
//  * Workgroup b belongs to group b % NG; with NG = 8 a group sits on one
//    XCD (workgroups are dispatched round-robin over the XCDs), so the
//    first read of a record is served by that XCD's L2.  A record with a
//    stale tag is re-read at device scope, so placement only affects speed.
//  * Every wait is bounded in time; a timed-out wait raises a flag in the
//    workspace header and the workgroup stops.

#include "hc_device.hpp"
#include "hc_launch.hpp"

namespace hc {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kTT = 2;             // 16-token tiles per round
constexpr int kKG = 4;             // k-groups of a member's slice
constexpr int kT = 16 * kTT;       // tokens per round
constexpr int kTiles = 5;          // 5 x 16 = 80 MFMA columns (72 used)
constexpr int kChunks = 9;         // 16-byte chunks per partial record (25 fields + tag words)
constexpr int kSlots = 4;          // rounds of records kept per group
constexpr int kOwnMax = 7;         // owned tokens per batch (one batch when G >= 5)
constexpr int kRed = 28;           // floats per token in the per-k-group LDS partials
constexpr uint64_t kMagic = 0x6863776b73703031ull;   // marks an initialised workspace
constexpr uint32_t kEpochMask = 0xFFFFFu;            // 20-bit call epoch in each tag
constexpr int kBufDword3 = 0x00020000;               // raw buffer resource, dword 3

// Workspace header (first 256 bytes): magic, call epoch, error flag.
struct WsHeader {
    uint64_t magic;
    uint32_t epoch;
    uint32_t err;
};

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
    WsHeader* hdr;
    u32x4* part;        // [NG][kSlots][G][kT][kChunks] tagged records
    int64_t n;
    int64_t ntiles;
    int d;
    int G;
    int NG;
    int iters;
    float eps;
    float norm_eps;
    float K;
    int part_bytes;
};

// Field f of a partial record (0..23 = the 24 dot products, 24 = sum of
// squares) by chunk and slot.  The pre-relevant fields (0..3 and 24) are
// in chunks 0 and 1.
__device__ __forceinline__ int field_at(int chunk, int slot) {
    if (chunk == 0) return slot;                                    // m0 m1 m2
    if (chunk == 1) return slot == 0 ? 3 : (slot == 1 ? 24 : 4);    // m3 ss m4
    const int f = 5 + 3 * (chunk - 2) + slot;                       // m5 .. m23
    return f <= 23 ? f : -1;
}

struct RoundCtx {
    int g, q, w, l, row, grp, tt, kg;
    int nr;                 // rounds of this group
    int mpo;                // members per octet = ceil(G / 8)
    uint32_t epoch;
    __amdgpu_buffer_rsrc_t rsrc;   // the record area
};

__device__ __forceinline__ uint32_t tag_of(const RoundCtx& c, int r) {
    return (c.epoch << 12) | ((uint32_t)r & 0xFFFu);
}

// Byte offset of a record chunk within the record area.
__device__ __forceinline__ int rec_off(const CoopArgs& a, const RoundCtx& c, int r, int member, int t, int chunk) {
    const int slot = r % kSlots;
    return ((((c.g * kSlots + slot) * a.G + member) * kT + t) * kChunks + chunk) * 16;
}

__device__ __forceinline__ u32x4 ld_l2(const RoundCtx& c, int off) {   // first read: served by the L2
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(c.rsrc, off, 0, 1));
}
__device__ __forceinline__ u32x4 ld_dev(const RoundCtx& c, int off) {  // device scope
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(c.rsrc, off, 0, 16));
}
__device__ __forceinline__ void st_dev(const RoundCtx& c, int off, u32x4 v) {   // device scope
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((__vector_size__(16))) int, v), c.rsrc,
                                           off, 0, 16);
}

__device__ __forceinline__ int64_t tile_of(const RoundCtx& c, const CoopArgs& a, int r) {
    return (int64_t)c.g + (int64_t)r * a.NG;
}

template <int KS>
struct Frags {
    u32x4 r[KS];
};

template <int KS>
struct Lds {
    bf16x8 wf[kKG * KS][kTiles][64];       // weight slice as MFMA B fragments
    float red[kKG][kT][kRed];              // per-k-group partials of the round being published
    float xs[kT][2][8][4];                 // pre fields: per member-octet sums
    float os[kOwnMax + 1][kChunks][8][4];  // owned tokens: per member-octet sums of all chunks
    float osum[kOwnMax + 1][kRed];         // owned tokens: summed fields
    float omix[kOwnMax + 1][kMix];         // owned tokens: mixes (split in the next iteration)
    float preL[kT][4];                     // pre of every token of the round
    int flag;
};

// Residual fragments of round r for this wave: 16 tokens of tile tt, the
// KS k-steps of k-group kg; lane (row, grp) holds 8 features of stream grp.
template <int KS>
__device__ __forceinline__ void load_round(Frags<KS>& f, const CoopArgs& a, const RoundCtx& c, int r) {
    const int64_t tok = tile_of(c, a, r) * kT + 16 * c.tt + c.row;
    const bool ok = tok < a.n;
    const int c0 = c.q * (32 * KS) + 8 * (c.kg * KS);
    const u32x4* src = reinterpret_cast<const u32x4*>(a.R + ((ok ? tok : 0) * kHC + c.grp) * (int64_t)a.d + c0);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (ok) v = __builtin_nontemporal_load(src + s);
        f.r[s] = v;
    }
}

// Bounded wait for a record chunk carrying the expected tag (device-scope
// reads).  On a timeout (or a flag raised elsewhere) it raises the flag and
// returns a chunk whose tag does not match, which the caller treats as a stop.
__device__ __noinline__ u32x4 reread(__amdgpu_buffer_rsrc_t rsrc, int off, uint32_t tag, WsHeader* hdr) {
    u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 16));
    if (v[3] == tag) return v;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    for (;;) {
        __builtin_amdgcn_s_sleep(1);
        v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 16));
        if (v[3] == tag) return v;
        if (__builtin_amdgcn_s_memrealtime() - t0 > 200000000ull ||
            __hip_atomic_load(&hdr->err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
            __hip_atomic_store(&hdr->err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            v[3] = ~tag;
            return v;
        }
    }
}

// ---------------------------------------------------- stage A: publish r
template <int KS>
__device__ __forceinline__ void publish(const Frags<KS>& f, const CoopArgs& a, const RoundCtx& c, Lds<KS>& L,
                                        int r) {
    f32x4 acc[kTiles];
#pragma unroll
    for (int ct = 0; ct < kTiles; ++ct) acc[ct] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float ss = 0.0f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const bf16x8 av = __builtin_bit_cast(bf16x8, f.r[s]);
        const int kk = c.kg * KS + s;
#pragma unroll
        for (int ct = 0; ct < kTiles; ++ct)
            acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, L.wf[kk][ct][c.l], acc[ct], 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float lo = bf_lo(f.r[s][e]), hi = bf_hi(f.r[s][e]);
            ss = __builtin_fmaf(lo, lo, ss);
            ss = __builtin_fmaf(hi, hi, ss);
        }
    }
    // sum of squares over the 4 lane groups (rows of 16 lanes)
    {
        auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(ss), __float_as_uint(ss), false, false);
        ss = __uint_as_float(x[0]) + __uint_as_float(x[1]);
        auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(ss), __float_as_uint(ss), false, false);
        ss = __uint_as_float(y[0]) + __uint_as_float(y[1]);
    }
    if (c.grp == 0) L.red[c.kg][16 * c.tt + c.row][24] = ss;
    // combine the three weight pieces (lo + mid first, then hi)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
        const int t = 16 * c.tt + 4 * c.grp + rr;
        const float v0 = (acc[2][rr] + acc[1][rr]) + acc[0][rr];
        const float t3 = acc[3][rr];
        const float t3x = dpp<0x128>(t3);
        const float v1 = (acc[4][rr] + t3x) + t3;
        L.red[c.kg][t][c.row] = v0;
        if (c.row < 8) L.red[c.kg][t][16 + c.row] = v1;
    }
    __syncthreads();
    const int tid = threadIdx.x;
    if (tid < kT * kChunks) {
        const int t = tid / kChunks, ch = tid - t * kChunks;
        u32x4 v;
#pragma unroll
        for (int sl = 0; sl < 3; ++sl) {
            const int fi = field_at(ch, sl);
            float x = 0.0f;
            if (fi >= 0) x = ((L.red[0][t][fi] + L.red[1][t][fi]) + L.red[2][t][fi]) + L.red[3][t][fi];
            v[sl] = __float_as_uint(x);
        }
        v[3] = tag_of(c, r);
        st_dev(c, rec_off(a, c, r, c.q, t, ch), v);
    }
}

// Exchange loads of round r issued ahead of time (held in registers).
template <int MPO_MAX>
struct XLoads {
    u32x4 pre[MPO_MAX];    // pre-field chunk of members mq*mpo .. +mpo
    u32x4 own[MPO_MAX];    // owned-token chunk of the same members
};

// Thread roles for the exchange reads: pre fields -> (t, ch, mq) with
// t = tid / 16, ch = (tid / 8) & 1, mq = tid & 7; owned tokens ->
// (o, ch, mq) with o = tid / 72, ch = (tid % 72) / 8, mq = tid & 7.
template <int MPO_MAX, bool FUSED>
__device__ __forceinline__ void issue_x(XLoads<MPO_MAX>& X, const CoopArgs& a, const RoundCtx& c, int r, int nown) {
    const int tid = threadIdx.x;
    if (FUSED) {
        const int t = tid >> 4, ch = (tid >> 3) & 1, mq = tid & 7;
#pragma unroll
        for (int m = 0; m < MPO_MAX; ++m) {
            const int qq = mq * c.mpo + m;
            if (m < c.mpo && qq < a.G) X.pre[m] = ld_l2(c, rec_off(a, c, r, qq, t, ch));
        }
    }
    const int o = tid / 72, rem = tid - o * 72, ch = rem >> 3, mq = rem & 7;
    if (o < nown && o < kOwnMax) {
        const int tl = c.q + a.G * o;
#pragma unroll
        for (int m = 0; m < MPO_MAX; ++m) {
            const int qq = mq * c.mpo + m;
            if (m < c.mpo && qq < a.G) X.own[m] = ld_l2(c, rec_off(a, c, r, qq, tl, ch));
        }
    }
}

// Sum the 3 data floats of this thread's members (in member order) after
// checking tags; stale chunks are re-read at device scope.
template <int MPO_MAX>
__device__ __forceinline__ void member_sum(const u32x4 (&v)[MPO_MAX], const CoopArgs& a, const RoundCtx& c, int r,
                                           int t, int ch, int mq, float* out3, int* bad) {
    const uint32_t tag = tag_of(c, r);
    float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f;
#pragma unroll
    for (int m = 0; m < MPO_MAX; ++m) {
        const int qq = mq * c.mpo + m;
        if (m < c.mpo && qq < a.G) {
            u32x4 x = v[m];
            if (x[3] != tag) {
                x = reread(c.rsrc, rec_off(a, c, r, qq, t, ch), tag, a.hdr);
                if (x[3] != tag) *bad = 1;
            }
            s0 += __uint_as_float(x[0]);
            s1 += __uint_as_float(x[1]);
            s2 += __uint_as_float(x[2]);
        }
    }
    out3[0] = s0;
    out3[1] = s1;
    out3[2] = s2;
}

// Owner reduction of a batch of owned tokens (all 25 fields), then their
// mixes into L.omix and the mixes output.  With `pre_loaded` the chunks
// come from X (issued ahead), otherwise they are loaded here.
template <int MPO_MAX, int KS>
__device__ __forceinline__ void owner_reduce(const XLoads<MPO_MAX>& X, bool pre_loaded, const CoopArgs& a,
                                             const RoundCtx& c, Lds<KS>& L, int r, int o0, int cnt, int* bad) {
    const int tid = threadIdx.x;
    const int o = tid / 72, rem = tid - o * 72, ch = rem >> 3, mq = rem & 7;
    if (o < cnt) {
        const int tl = c.q + a.G * (o0 + o);
        u32x4 v[MPO_MAX];
#pragma unroll
        for (int m = 0; m < MPO_MAX; ++m) {
            const int qq = mq * c.mpo + m;
            if (m < c.mpo && qq < a.G) v[m] = pre_loaded ? X.own[m] : ld_l2(c, rec_off(a, c, r, qq, tl, ch));
        }
        member_sum<MPO_MAX>(v, a, c, r, tl, ch, mq, &L.os[o][ch][mq][0], bad);
    }
    __syncthreads();
    if (tid < cnt * 25) {
        const int oo = tid / 25, fi = tid - oo * 25;
        int chk = 0, sl = 0;
        for (int q2 = 0; q2 < kChunks; ++q2)
            for (int s2 = 0; s2 < 3; ++s2)
                if (field_at(q2, s2) == fi) { chk = q2; sl = s2; }
        float s = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) s += L.os[oo][chk][k][sl];
        L.osum[oo][fi] = s;
    }
    __syncthreads();
    if (tid < cnt * kMix) {
        const int oo = tid / kMix, j = tid - oo * kMix;
        const float rs = rms_scale(L.osum[oo][24], a.K, a.norm_eps);
        const float mval = L.osum[oo][j] * rs;
        L.omix[oo][j] = mval;
        const int64_t t = tile_of(c, a, r) * kT + c.q + (int64_t)a.G * (o0 + oo);
        if (a.mixes && t < a.n) a.mixes[t * kMix + j] = mval;
    }
    __syncthreads();
}

// Split + Sinkhorn of a batch of owned tokens of round r (mixes in
// L.omix), one 16-lane row per token, and the coefficient outputs.  Waves
// whose rows are all beyond the batch skip it.
template <int KS>
__device__ __forceinline__ void owner_split(const CoopArgs& a, const RoundCtx& c, Lds<KS>& L, int r, int o0,
                                            int cnt) {
    if (c.w * 4 >= cnt) return;
    const int o = threadIdx.x >> 4, e = threadIdx.x & 15;
    const bool valid = o < cnt;
    float p, qv, cv;
    split_sinkhorn16(L.omix[valid ? o : 0], a.scale[0], a.scale[1], a.scale[2], a.base, a.iters, a.eps, p, qv, cv);
    if (valid) {
        const int64_t t = tile_of(c, a, r) * kT + c.q + (int64_t)a.G * (o0 + o);
        if (t < a.n) {
            a.comb[t * (kHC * kHC) + e] = cv;
            if (e < kHC) {
                if (a.pre) a.pre[t * kHC + e] = p;
                a.post[t * kHC + e] = qv;
            }
        }
    }
}

// pre for all T tokens of round r from the exchange loads, into L.preL.
// The member sums follow the owners' order, so pre here is bitwise the
// owner's (and hc_split_sinkhorn's on the same mixes).
template <int MPO_MAX, int KS>
__device__ __forceinline__ void form_pre(const XLoads<MPO_MAX>& X, const CoopArgs& a, const RoundCtx& c, Lds<KS>& L,
                                         int r, int* bad) {
    const int tid = threadIdx.x;
    const int t = tid >> 4, ch = (tid >> 3) & 1, mq = tid & 7;
    member_sum<MPO_MAX>(X.pre, a, c, r, t, ch, mq, &L.xs[t][ch][mq][0], bad);
    __syncthreads();
    if (tid < kT * 4) {
        const int tk = tid >> 2, j = tid & 3;
        const int chj = j < 3 ? 0 : 1, slj = j < 3 ? j : 0;    // m_0..m_2: chunk 0; m_3: chunk 1 slot 0
        float sj = 0.0f, sq = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            sj += L.xs[tk][chj][k][slj];
            sq += L.xs[tk][1][k][1];                             // sum of squares: chunk 1 slot 1
        }
        const float rs = rms_scale(sq, a.K, a.norm_eps);
        L.preL[tk][j] = pre_gate(sj * rs, a.scale[0], a.base[j], a.eps);
    }
    __syncthreads();
}

// h for this wave's 16 tokens x KS k-steps of round r, from registers.
template <int KS>
__device__ __forceinline__ void write_h(const Frags<KS>& f, const CoopArgs& a, const RoundCtx& c, Lds<KS>& L, int r) {
    const int tl = 16 * c.tt + c.row;
    const int64_t t = tile_of(c, a, r) * kT + tl;
    const double p0 = L.preL[tl][0], p1 = L.preL[tl][1], p2 = L.preL[tl][2], p3 = L.preL[tl][3];
    uint32_t* dst = reinterpret_cast<uint32_t*>(a.h + (t < a.n ? t : 0) * (int64_t)a.d + c.q * (32 * KS) +
                                                8 * (c.kg * KS) + 2 * c.grp);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        // 4x4 transpose across the lane groups: before, lane group g holds
        // stream g, feature pairs 0..3; after, feature pair g of streams 0..3.
        uint32_t v0 = f.r[s][0], v1 = f.r[s][1], v2 = f.r[s][2], v3 = f.r[s][3];
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
        if (t < a.n) __builtin_nontemporal_store(pack2(bf16_rn_f64(lo), bf16_rn_f64(hi)), dst + 4 * s);
    }
}

// A workgroup stops as a whole once any of its threads hit a timeout.
template <int KS>
__device__ __forceinline__ bool stopped(Lds<KS>& L, int bad) {
    if (threadIdx.x == 0) L.flag = 0;
    __syncthreads();
    if (bad) L.flag = 1;
    __syncthreads();
    return L.flag != 0;
}

__device__ __forceinline__ int owned_per_round(const RoundCtx& c, int G) {
    return c.q < kT ? (kT - 1 - c.q) / G + 1 : 0;
}

// One pipeline iteration: exchange loads of round i, prefetch of round i+3,
// publication of round i+1, owner split of round i-1, pre and h of round i,
// owner reduction of round i.
template <int KS, int MPO_MAX, bool FUSED>
__device__ __forceinline__ bool iteration(const Frags<KS>& H, const Frags<KS>& M, Frags<KS>& P, const CoopArgs& a,
                                          const RoundCtx& c, Lds<KS>& L, int i) {
    const int nown = owned_per_round(c, a.G);
    XLoads<MPO_MAX> X;
    issue_x<MPO_MAX, FUSED>(X, a, c, i, nown);
    if (i + 3 < c.nr) load_round<KS>(P, a, c, i + 3);
    if (i + 1 < c.nr) publish<KS>(M, a, c, L, i + 1);
    if (FUSED && i >= 1 && nown > 0 && nown <= kOwnMax) owner_split<KS>(a, c, L, i - 1, 0, nown);
    int bad = 0;
    if (FUSED) {
        form_pre<MPO_MAX, KS>(X, a, c, L, i, &bad);
        write_h<KS>(H, a, c, L, i);
    }
    for (int o0 = 0; o0 < nown; o0 += kOwnMax) {
        const int cnt = nown - o0 < kOwnMax ? nown - o0 : kOwnMax;
        owner_reduce<MPO_MAX, KS>(X, o0 == 0, a, c, L, i, o0, cnt, &bad);
        if (FUSED && nown > kOwnMax) {
            // groups this small own several batches: split each one now
            owner_split<KS>(a, c, L, i, o0, cnt);
            __syncthreads();
        }
    }
    return !stopped<KS>(L, bad);
}

template <int KS, int MPO_MAX, bool FUSED>
__global__ __launch_bounds__(kThreads, 1) void k_coop(CoopArgs a) {
    __shared__ Lds<KS> L;
    RoundCtx c;
    c.g = blockIdx.x % a.NG;
    c.q = blockIdx.x / a.NG;
    c.w = threadIdx.x >> 6;
    c.l = threadIdx.x & 63;
    c.row = c.l & 15;
    c.grp = c.l >> 4;
    c.tt = c.w & 1;
    c.kg = c.w >> 1;
    c.mpo = (a.G + 7) / 8;
    c.epoch = a.hdr->epoch;
    c.rsrc = __builtin_amdgcn_make_buffer_rsrc(a.part, 0, a.part_bytes, kBufDword3);
    if (c.g >= a.ntiles) return;
    c.nr = (int)((a.ntiles - c.g + a.NG - 1) / a.NG);

    // weight slice -> LDS as MFMA B fragments, split exactly into bf16 pieces;
    // column (tile ct, lane column i): tiles 0..2 hold piece ct of mix i;
    // tile 3 holds hi of mixes 16..23 (i < 8) and mid of them (i >= 8);
    // tile 4 holds lo of mixes 16..23 (i < 8).
    const int64_t K = (int64_t)kHC * a.d;
    for (int fi = c.w; fi < kKG * KS * kTiles; fi += kWaves) {
        const int kk = fi / kTiles, ct = fi - kk * kTiles;
        int piece, j;
        if (ct < 3) { piece = ct; j = c.row; }
        else if (ct == 3) { piece = c.row < 8 ? 0 : 1; j = 16 + (c.row & 7); }
        else { piece = c.row < 8 ? 2 : -1; j = 16 + c.row; }
        bf16x8 v;
        if (piece < 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = (__bf16)0.0f;
        } else {
            const f32x4* src =
                reinterpret_cast<const f32x4*>(a.W + j * K + (int64_t)c.grp * a.d + c.q * (32 * KS) + 8 * kk);
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
        L.wf[kk][ct][c.l] = v;
    }
    __syncthreads();

    Frags<KS> B0, B1, B2, B3;
    load_round<KS>(B0, a, c, 0);
    if (1 < c.nr) load_round<KS>(B1, a, c, 1);
    if (2 < c.nr) load_round<KS>(B2, a, c, 2);
    publish<KS>(B0, a, c, L, 0);
    for (int i = 0; i < c.nr; i += 4) {
        if (!iteration<KS, MPO_MAX, FUSED>(B0, B1, B3, a, c, L, i)) return;
        if (i + 1 >= c.nr) break;
        if (!iteration<KS, MPO_MAX, FUSED>(B1, B2, B0, a, c, L, i + 1)) return;
        if (i + 2 >= c.nr) break;
        if (!iteration<KS, MPO_MAX, FUSED>(B2, B3, B1, a, c, L, i + 2)) return;
        if (i + 3 >= c.nr) break;
        if (!iteration<KS, MPO_MAX, FUSED>(B3, B0, B2, a, c, L, i + 3)) return;
    }
    const int nown = owned_per_round(c, a.G);
    if (FUSED && nown > 0 && nown <= kOwnMax) owner_split<KS>(a, c, L, c.nr - 1, 0, nown);
}

// Per-call header update.  Clears every record on the first use of a
// workspace and when the 20-bit call epoch wraps, so a stale record never
// carries a current tag.
__global__ __launch_bounds__(1024) void k_init(WsHeader* hdr, u32x4* part, int64_t nchunks) {
    __shared__ int clear;
    __shared__ uint32_t next;
    if (threadIdx.x == 0) {
        const uint32_t e = hdr->epoch;
        const bool fresh = hdr->magic != kMagic;
        uint32_t ne = fresh ? 1u : (e & kEpochMask) + 1u;
        clear = fresh || ne > kEpochMask;
        if (ne > kEpochMask) ne = 1u;
        next = ne;
    }
    __syncthreads();
    if (clear)
        for (int64_t i = threadIdx.x; i < nchunks; i += blockDim.x) part[i] = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
    if (threadIdx.x == 0) {
        hdr->magic = kMagic;
        hdr->epoch = next;
        hdr->err = 0u;
    }
}

// ------------------------------------------------------------------ host
int coop_ks(int d) {
    if (d <= 0 || d % 32 != 0) return 0;
    for (int k = 1; k <= 5; ++k)
        if (d % (32 * k) == 0 && d / (32 * k) <= 32) return k;
    for (int k = 1; k <= 5; ++k)
        if (d % (32 * k) == 0 && d / (32 * k) <= 64) return k;
    return 0;
}

bool coop_plan(int64_t n, int d, CoopPlan& p) {
    const int KS = coop_ks(d);
    if (!KS) return false;
    p.KS = KS;
    p.G = d / (32 * KS);
    p.TM = kTT;
    p.ntiles = (n + kT - 1) / kT;
    int ng = num_cus() / p.G;
    if (ng < 1) ng = 1;
    if (ng > p.ntiles) ng = (int)(p.ntiles > 0 ? p.ntiles : 1);
    p.NG = ng;
    p.ws_pre = 0;
    p.ws_cnt = 0;
    p.ws_part = 256;
    p.ws_bytes = p.ws_part + (size_t)p.NG * kSlots * p.G * kT * kChunks * 16;
    return true;
}

template <int KS, int MPO, bool FUSED>
static int launch_t(const CoopPlan& p, CoopArgs& a, hipStream_t s) {
    void* args[] = {&a};
    hipError_t e = hipLaunchCooperativeKernel((const void*)k_coop<KS, MPO, FUSED>, dim3(p.G * p.NG),
                                              dim3(kThreads), args, 0, s);
    return e == hipSuccess ? 0 : -1;
}

template <int KS>
static int launch_ks(const CoopPlan& p, CoopArgs& a, bool fused, hipStream_t s) {
    const int mpo = (p.G + 7) / 8;
    if (mpo <= 4) return fused ? launch_t<KS, 4, true>(p, a, s) : launch_t<KS, 4, false>(p, a, s);
    return fused ? launch_t<KS, 8, true>(p, a, s) : launch_t<KS, 8, false>(p, a, s);
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
    a.hdr = reinterpret_cast<WsHeader*>(wsb);
    a.part = reinterpret_cast<u32x4*>(wsb + p.ws_part);
    a.n = n;
    a.ntiles = p.ntiles;
    a.d = d;
    a.G = p.G;
    a.NG = p.NG;
    a.iters = iters;
    a.eps = eps;
    a.norm_eps = norm_eps;
    a.K = (float)(kHC * d);
    a.part_bytes = (int)(p.ws_bytes - p.ws_part);
    k_init<<<1, 1024, 0, s>>>(a.hdr, a.part, (int64_t)((p.ws_bytes - p.ws_part) / 16));
    if (hipGetLastError() != hipSuccess) return -1;
    switch (p.KS) {
        case 1: return launch_ks<1>(p, a, fused, s);
        case 2: return launch_ks<2>(p, a, fused, s);
        case 3: return launch_ks<3>(p, a, fused, s);
        case 4: return launch_ks<4>(p, a, fused, s);
        case 5: return launch_ks<5>(p, a, fused, s);
    }
    return -1;
}

}  // namespace hc
