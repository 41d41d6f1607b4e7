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
//  * A round is T = 32 tokens.  The residual of a round is read with
//    coalesced 16-byte loads (each instruction covers whole 64-byte-aligned
//    runs of the member's slice) and transposed through LDS into the MFMA
//    operand layout.  Each of the 8 waves then takes one 16-token tile and
//    one of 4 k-groups of the slice and runs v_mfma_f32_16x16x32_bf16 from
//    registers, and forms the sum of squares.
//  * The member's 25 partial sums per token are published to the workspace
//    as tagged 16-byte records (3 floats + a round tag), stored member-
//    fastest so that the G records of a (token, chunk) are contiguous.
//    Every member reads the pre-relevant records (m_0..m_3 and the sum of
//    squares) of all members with contiguous loads, adds them across lanes
//    in one fixed butterfly order, forms pre for all T tokens, and writes h
//    for its slice from the residual still in registers (staged through
//    LDS for coalesced stores): one HBM pass over the residual.  The owner
//    of each token (member t mod G) adds all 25 fields the same way and
//    writes the mixes (and pre); the split + Sinkhorn of post and comb then
//    runs over those mixes in the split kernel, which shares its per-token
//    code with hc_split_sinkhorn.
//  * Rounds are software-pipelined: in iteration i a wave issues its
//    exchange loads for round i, then the residual loads for round i+3, then
//    the projection and publication of round i+1, and finally the exchange
//    sums, pre, mixes and h of round i.  A wave's loads retire in
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
constexpr int kRed = 25;           // floats per token in the per-k-group LDS partials
constexpr int kPrePairs = 2 * kT;  // (chunk, token) pairs holding the pre-relevant fields
constexpr int kOwnPairs = kChunks * kT;   // (owned token, chunk) pairs at most (G = 1)
constexpr uint64_t kMagic = 0x6863776b73703031ull;   // marks an initialised workspace
constexpr uint32_t kEpochMask = 0xFFFFFu;            // 20-bit call epoch in each tag
constexpr int kBufDword3 = 0x00020000;               // raw buffer resource, dword 3

// Workspace header (first 256 bytes): magic, call epoch, error flag, and
// the length (16-byte records) of the record area known to hold only
// tagged records or zeros.
struct WsHeader {
    uint64_t magic;
    uint32_t epoch;
    uint32_t err;
    int64_t clean;
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
    float* mixes;       // mixes of every token (the caller's buffer or workspace)
    WsHeader* hdr;
    u32x4* part;        // [NG][kSlots][kChunks][kT][GP] tagged records, member fastest
    int64_t n;
    int64_t ntiles;
    int d;
    int G;
    int GP;             // G rounded up to a power of two (record stride)
    int gp_log2;
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
__device__ __forceinline__ void field_pos(int f, int& chunk, int& slot) {
    if (f < 3) { chunk = 0; slot = f; }
    else if (f == 3) { chunk = 1; slot = 0; }
    else if (f == 24) { chunk = 1; slot = 1; }
    else if (f == 4) { chunk = 1; slot = 2; }
    else { chunk = 2 + (f - 5) / 3; slot = (f - 5) % 3; }
}

// Staging geometry of one 16-token tile of a member slice: per token,
// 4 streams x 4*KS 16-byte chunks, plus one pad chunk (odd stride keeps
// the 16 rows of an MFMA operand read on distinct LDS banks).
template <int KS>
struct Geo {
    static constexpr int kRow = 4 * KS;            // chunks per (token, stream) in the slice
    static constexpr int kTok = 16 * KS + 1;       // staging stride per token, in chunks
    static constexpr int kHTok = 16 * KS + 1;      // h staging stride per token, in 32-bit words
};

template <int KS>
struct Lds {
    bf16x8 wf[kKG * KS][kTiles][64];       // weight slice as MFMA B fragments
    union {
        u32x4 stage[kTT][16 * Geo<KS>::kTok];          // residual transpose
        float red[kKG][kT][kRed];                      // per-k-group partials being published
        uint32_t hst[kTT][16 * Geo<KS>::kHTok];        // h transpose
    } u;
    float xsum[kPrePairs][4];              // pre-relevant member sums per (chunk, token)
    float xown[kOwnPairs][4];              // owned tokens: member sums per (owned token, chunk)
    float preL[kT][4];                     // pre of every token of the round
};

struct RoundCtx {
    int g, q, w, l, row, grp, tt, kg;
    int nr;                 // rounds of this group
    int nown;               // tokens of a round this member owns
    uint32_t epoch;
    __amdgpu_buffer_rsrc_t rsrc;   // the record area
};

__device__ __forceinline__ uint32_t tag_of(const RoundCtx& c, int r) {
    return (c.epoch << 12) | ((uint32_t)r & 0xFFFu);
}

// Byte offset of record chunk (member, token t, chunk) of round r.
__device__ __forceinline__ int rec_off(const CoopArgs& a, const RoundCtx& c, int r, int chunk, int t, int member) {
    const int slot = r % kSlots;
    return ((((c.g * kSlots + slot) * kChunks + chunk) * kT + t) * a.GP + member) * 16;
}

__device__ __forceinline__ u32x4 ld_l2(const RoundCtx& c, int off) {   // first read: served by the L2
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(c.rsrc, off, 0, 1));
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

// Buffer resource over the 16 tokens of tile tt of round r in a
// [n][per_tok] array; loads past the last token read zeros and stores past
// it are dropped by the hardware bounds check.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, int64_t per_tok_bytes, int64_t tok0,
                                                          int64_t n) {
    int64_t valid = n - tok0;
    valid = valid < 0 ? 0 : (valid > 16 ? 16 : valid);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(static_cast<const char*>(base)) + tok0 * per_tok_bytes,
                                             0, (int)(valid * per_tok_bytes), kBufDword3);
}

// Residual of round r, coalesced: the 4 waves of tile tt read the tile's
// 64 (token, stream) rows of the member slice, 4*KS chunks each, as
// 256*KS consecutive chunks; chunk g = (kg*KS + j)*64 + lane.
template <int KS>
__device__ __forceinline__ void load_round(Frags<KS>& f, const CoopArgs& a, const RoundCtx& c, int r) {
    const int64_t tok0 = tile_of(c, a, r) * kT + 16 * c.tt;
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(a.R, (int64_t)kHC * a.d * 2, tok0, a.n);
#pragma unroll
    for (int j = 0; j < KS; ++j) {
        const int g = (c.kg * KS + j) * 64 + c.l;
        const int row = g / Geo<KS>::kRow, col = g - row * Geo<KS>::kRow;
        const int off = (row * a.d + c.q * (32 * KS) + 8 * col) * 2;      // row = token*4 + stream
        f.r[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 2));
    }
}

// In place: coalesced layout -> MFMA A-operand layout (lane (row, grp)
// holds 8 features of stream grp of token row, k-step s of its k-group).
template <int KS>
__device__ __forceinline__ void to_operands(Frags<KS>& f, const RoundCtx& c, Lds<KS>& L) {
#pragma unroll
    for (int j = 0; j < KS; ++j) {
        const int g = (c.kg * KS + j) * 64 + c.l;
        const int row = g / Geo<KS>::kRow, col = g - row * Geo<KS>::kRow;
        L.u.stage[c.tt][(row >> 2) * Geo<KS>::kTok + (row & 3) * Geo<KS>::kRow + col] = f.r[j];
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < KS; ++s)
        f.r[s] = L.u.stage[c.tt][c.row * Geo<KS>::kTok + c.grp * Geo<KS>::kRow + c.kg * KS + s];
    __syncthreads();
}

// Sum over the gp lanes of each aligned lane group; the sum is read from
// the group's first lane, whose order of additions is fixed.  32 and 64
// lanes (member counts of the wide shapes) use DPP within rows of 16 and
// permlane swaps across rows; other sizes an xor butterfly.
__device__ __forceinline__ float group_sum(float v, int gp) {
    if (gp >= 32) {
        v = quad_sum(v);
        v = col4_sum(v);
        auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(x[0]) + __uint_as_float(x[1]);
        if (gp == 64) {
            auto y = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
            v = __uint_as_float(y[0]) + __uint_as_float(y[1]);
        }
        return v;
    }
    for (int m = 1; m < gp; m <<= 1) v += __shfl_xor(v, m);
    return v;
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
// f holds round r in MFMA operand layout.
template <int KS>
__device__ __forceinline__ void publish(const Frags<KS>& f, const CoopArgs& a, const RoundCtx& c, Lds<KS>& L,
                                        int r) {
    f32x4 acc[kTiles];
#pragma unroll
    for (int ct = 0; ct < kTiles; ++ct) acc[ct] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float sq[4] = {0.0f, 0.0f, 0.0f, 0.0f};
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
            sq[e] = __builtin_fmaf(hi, hi, __builtin_fmaf(lo, lo, sq[e]));
        }
    }
    float ss = (sq[0] + sq[1]) + (sq[2] + sq[3]);
    // sum of squares over the 4 lane groups (rows of 16 lanes)
    {
        auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(ss), __float_as_uint(ss), false, false);
        ss = __uint_as_float(x[0]) + __uint_as_float(x[1]);
        auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(ss), __float_as_uint(ss), false, false);
        ss = __uint_as_float(y[0]) + __uint_as_float(y[1]);
    }
    if (c.grp == 0) L.u.red[c.kg][16 * c.tt + c.row][24] = ss;
    // combine the three weight pieces (lo + mid first, then hi)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
        const int t = 16 * c.tt + 4 * c.grp + rr;
        const float v0 = (acc[2][rr] + acc[1][rr]) + acc[0][rr];
        const float t3 = acc[3][rr];
        const float t3x = dpp<0x128>(t3);
        const float v1 = (acc[4][rr] + t3x) + t3;
        L.u.red[c.kg][t][c.row] = v0;
        if (c.row < 8) L.u.red[c.kg][t][16 + c.row] = v1;
    }
    __syncthreads();
    const int tid = threadIdx.x;
    if (tid < kT * kChunks) {
        const int ch = tid / kT, t = tid - ch * kT;
        u32x4 v;
#pragma unroll
        for (int sl = 0; sl < 3; ++sl) {
            const int fi = field_at(ch, sl);
            float x = 0.0f;
            if (fi >= 0) x = ((L.u.red[0][t][fi] + L.u.red[1][t][fi]) + L.u.red[2][t][fi]) + L.u.red[3][t][fi];
            v[sl] = __float_as_uint(x);
        }
        v[3] = tag_of(c, r);
        st_dev(c, rec_off(a, c, r, ch, t, c.q), v);
    }
}

// Exchange loads of round r issued ahead of time (held in registers).
// Pre fields: record chunk index x = j*512 + tid over (chunk 0/1, token,
// member); owned tokens: x = j*512 + tid over (owned token, chunk, member).
template <int PI>
struct XLoads {
    u32x4 pre[PI];
    u32x4 own[2];
};

template <int PI, bool FUSED>
__device__ __forceinline__ void issue_x(XLoads<PI>& X, const CoopArgs& a, const RoundCtx& c, int r) {
    const int tid = threadIdx.x;
    if (FUSED) {
#pragma unroll
        for (int j = 0; j < PI; ++j) {
            const int x = j * kThreads + tid;
            const int pair = x >> a.gp_log2, m = x & (a.GP - 1);
            if (pair < kPrePairs && m < a.G) X.pre[j] = ld_l2(c, rec_off(a, c, r, pair / kT, pair % kT, m));
        }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int x = j * kThreads + tid;
        const int pair = x >> a.gp_log2, m = x & (a.GP - 1);
        const int o = pair / kChunks, ch = pair - o * kChunks;
        if (o < c.nown && m < a.G) X.own[j] = ld_l2(c, rec_off(a, c, r, ch, c.q + a.G * o, m));
    }
}

// Member sums of a loaded record chunk (3 floats): tag check (stale
// chunks are re-read at device scope), then the group butterfly.
__device__ __forceinline__ void chunk_sum(u32x4 v, bool have, const CoopArgs& a, const RoundCtx& c, int r, int chunk,
                                          int t, int m, float* s3, int* bad) {
    const uint32_t tag = tag_of(c, r);
    float x0 = 0.0f, x1 = 0.0f, x2 = 0.0f;
    if (have) {
        if (v[3] != tag) {
            v = reread(c.rsrc, rec_off(a, c, r, chunk, t, m), tag, a.hdr);
            if (v[3] != tag) *bad = 1;
        }
        x0 = __uint_as_float(v[0]);
        x1 = __uint_as_float(v[1]);
        x2 = __uint_as_float(v[2]);
    }
    s3[0] = group_sum(x0, a.GP);
    s3[1] = group_sum(x1, a.GP);
    s3[2] = group_sum(x2, a.GP);
}

// Exchange of round r: member sums of the pre-relevant records of every
// token (into L.xsum) and of all records of the owned tokens (into
// L.xown), in one fixed butterfly order shared by both, so pre formed here
// is bitwise the pre of the owner's mixes.  Returns true if any thread of
// the workgroup hit a timeout.
template <int PI, int KS, bool FUSED>
__device__ __forceinline__ bool exchange(const XLoads<PI>& X, const CoopArgs& a, const RoundCtx& c, Lds<KS>& L,
                                         int r) {
    const int tid = threadIdx.x;
    int bad = 0;
    if (FUSED) {
#pragma unroll
        for (int j = 0; j < PI; ++j) {
            if (j * kThreads < kPrePairs * a.GP) {          // block-uniform: this load carries pairs
                const int x = j * kThreads + tid;
                const int pair = x >> a.gp_log2, m = x & (a.GP - 1);
                float s3[3];
                chunk_sum(X.pre[j], pair < kPrePairs && m < a.G, a, c, r, pair / kT, pair % kT, m, s3, &bad);
                if (m == 0 && pair < kPrePairs) {
                    L.xsum[pair][0] = s3[0];
                    L.xsum[pair][1] = s3[1];
                    L.xsum[pair][2] = s3[2];
                }
            }
        }
    }
    const int npairs = c.nown * kChunks;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        if (j * kThreads < npairs * a.GP) {                 // block-uniform
            const int x = j * kThreads + tid;
            const int pair = x >> a.gp_log2, m = x & (a.GP - 1);
            const int o = pair / kChunks, ch = pair - o * kChunks;
            float s3[3];
            chunk_sum(X.own[j], pair < npairs && m < a.G, a, c, r, ch, c.q + a.G * o, m, s3, &bad);
            if (m == 0 && pair < npairs) {
                L.xown[pair][0] = s3[0];
                L.xown[pair][1] = s3[1];
                L.xown[pair][2] = s3[2];
            }
        }
    }
    return __syncthreads_or(bad) != 0;
}

// pre of every token of round r (into L.preL; the owner also writes the pre
// output) and the mixes of the owned tokens.
template <int KS, bool FUSED>
__device__ __forceinline__ void finals(const CoopArgs& a, const RoundCtx& c, Lds<KS>& L, int r) {
    const int tid = threadIdx.x;
    const int64_t tok0 = tile_of(c, a, r) * kT;
    if (FUSED && tid < kT * 4) {
        const int t = tid >> 2, j = tid & 3;
        const float sj = j < 3 ? L.xsum[t][j] : L.xsum[kT + t][0];     // m_0..m_2: chunk 0; m_3: chunk 1 slot 0
        const float sq = L.xsum[kT + t][1];                           // sum of squares: chunk 1 slot 1
        const float p = pre_gate(sj * rms_scale(sq, a.K, a.norm_eps), a.scale[0], a.base[j], a.eps);
        L.preL[t][j] = p;
        if (a.pre && t % a.G == c.q && tok0 + t < a.n) a.pre[(tok0 + t) * kHC + j] = p;
    }
    const int base = FUSED ? kT * 4 : 0;
    for (int x = tid - base; x >= 0 && x < c.nown * kMix; x += kThreads - base) {
        const int o = x / kMix, j = x - o * kMix;
        int ch, sl;
        field_pos(j, ch, sl);
        const float rs = rms_scale(L.xown[o * kChunks + 1][1], a.K, a.norm_eps);
        const int64_t t = tok0 + c.q + (int64_t)a.G * o;
        if (t < a.n) a.mixes[t * kMix + j] = L.xown[o * kChunks + ch][sl] * rs;
    }
    __syncthreads();        // preL is read by write_h; xsum / xown are rewritten next round
}

// h for this member's slice of round r: formed from the operand registers
// (f, MFMA layout), staged through LDS, stored with coalesced 4-byte stores.
template <int KS>
__device__ __forceinline__ void write_h(const Frags<KS>& f, const CoopArgs& a, const RoundCtx& c, Lds<KS>& L, int r) {
    {
        const int tl = 16 * c.tt + c.row;
        const double p0 = L.preL[tl][0], p1 = L.preL[tl][1], p2 = L.preL[tl][2], p3 = L.preL[tl][3];
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
            L.u.hst[c.tt][c.row * Geo<KS>::kHTok + 4 * (c.kg * KS + s) + c.grp] =
                pack2(bf16_rn_f64(lo), bf16_rn_f64(hi));
        }
    }
    __syncthreads();
    // the tile's 16 tokens x 16*KS words, by the tile's 4 waves
    const int64_t tok0 = tile_of(c, a, r) * kT + 16 * c.tt;
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(a.h, (int64_t)a.d * 2, tok0, a.n);
#pragma unroll
    for (int j = 0; j < KS; ++j) {
        const int x = j * 256 + c.kg * 64 + c.l;
        const int tk = x / (16 * KS), col = x - tk * (16 * KS);
        __builtin_amdgcn_raw_buffer_store_b32(L.u.hst[c.tt][tk * Geo<KS>::kHTok + col], rs,
                                              (tk * (a.d / 2) + c.q * (16 * KS) + col) * 4, 0, 2);
    }
    __syncthreads();        // the staging area is rewritten by the next round's transpose
}

// One pipeline iteration: exchange loads of round i, prefetch of round i+3
// into P, transpose + publication of round i+1 (M), exchange sums, pre,
// mixes and h of round i (H); then H <- M and M <- W.
template <int KS, int PI, bool FUSED>
__device__ __forceinline__ bool iteration(Frags<KS>& H, Frags<KS>& M, const Frags<KS>& W, Frags<KS>& P,
                                          const CoopArgs& a, const RoundCtx& c, Lds<KS>& L, int i) {
    XLoads<PI> X;
    issue_x<PI, FUSED>(X, a, c, i);
    if (i + 3 < c.nr) load_round<KS>(P, a, c, i + 3);
    if (i + 1 < c.nr) {
        to_operands<KS>(M, c, L);
        publish<KS>(M, a, c, L, i + 1);
    }
    if (exchange<PI, KS, FUSED>(X, a, c, L, i)) return false;
    finals<KS, FUSED>(a, c, L, i);
    if (FUSED) write_h<KS>(H, a, c, L, i);
    H = M;
    M = W;
    return true;
}

template <int KS, int PI, bool FUSED>
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
    c.nown = c.q < kT ? (kT - 1 - c.q) / a.G + 1 : 0;
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

    Frags<KS> H, M, A, B;
    load_round<KS>(H, a, c, 0);
    if (1 < c.nr) load_round<KS>(M, a, c, 1);
    if (2 < c.nr) load_round<KS>(A, a, c, 2);
    to_operands<KS>(H, c, L);
    publish<KS>(H, a, c, L, 0);
    for (int i = 0; i < c.nr; i += 2) {
        if (!iteration<KS, PI, FUSED>(H, M, A, B, a, c, L, i)) return;
        if (i + 1 >= c.nr) break;
        if (!iteration<KS, PI, FUSED>(H, M, B, A, a, c, L, i + 1)) return;
    }
}

// Per-call header update.  Clears the record area on the first use of a
// workspace, when the 20-bit call epoch wraps, and when this call's record
// area reaches past the part known to be clean (a previous call may have
// kept its mixes there), so a record never carries a current tag before
// this call writes it.  Past this call's record area the workspace may
// receive mixes, so only that area stays known clean.
__global__ __launch_bounds__(1024) void k_init(WsHeader* hdr, u32x4* part, int64_t nchunks) {
    __shared__ int clear;
    __shared__ uint32_t next;
    if (threadIdx.x == 0) {
        const uint32_t e = hdr->epoch;
        const bool fresh = hdr->magic != kMagic;
        uint32_t ne = fresh ? 1u : (e & kEpochMask) + 1u;
        clear = fresh || ne > kEpochMask || hdr->clean < nchunks;
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
        hdr->clean = nchunks;
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

static int pow2_at_least(int x) {
    int p = 1;
    while (p < x) p <<= 1;
    return p;
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
    p.ws_part = 256;
    p.ws_mix = p.ws_part + (size_t)p.NG * kSlots * kChunks * kT * pow2_at_least(p.G) * 16;
    p.ws_bytes = p.ws_mix + (((size_t)n * kMix * sizeof(float) + 255) & ~(size_t)255);
    return true;
}

template <int KS, int PI, bool FUSED>
static int launch_t(const CoopPlan& p, CoopArgs& a, hipStream_t s) {
    void* args[] = {&a};
    hipError_t e = hipLaunchCooperativeKernel((const void*)k_coop<KS, PI, FUSED>, dim3(p.G * p.NG),
                                              dim3(kThreads), args, 0, s);
    return e == hipSuccess ? 0 : -1;
}

// PI: 512-thread load instructions needed for the pre-relevant records,
// 2*kT*GP/512 rounded up to 1, 4 or 8.
template <int KS>
static int launch_ks(const CoopPlan& p, CoopArgs& a, bool fused, hipStream_t s) {
    const int need = (kPrePairs * a.GP + kThreads - 1) / kThreads;
    if (need <= 1) return fused ? launch_t<KS, 1, true>(p, a, s) : launch_t<KS, 1, false>(p, a, s);
    if (need <= 4) return fused ? launch_t<KS, 4, true>(p, a, s) : launch_t<KS, 4, false>(p, a, s);
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
    a.mixes = mixes ? mixes : reinterpret_cast<float*>(wsb + p.ws_mix);
    a.hdr = reinterpret_cast<WsHeader*>(wsb);
    a.part = reinterpret_cast<u32x4*>(wsb + p.ws_part);
    a.n = n;
    a.ntiles = p.ntiles;
    a.d = d;
    a.G = p.G;
    a.GP = pow2_at_least(p.G);
    a.gp_log2 = __builtin_ctz(a.GP);
    a.NG = p.NG;
    a.iters = iters;
    a.eps = eps;
    a.norm_eps = norm_eps;
    a.K = (float)(kHC * d);
    a.part_bytes = (int)(p.ws_mix - p.ws_part);
    k_init<<<1, 1024, 0, s>>>(a.hdr, a.part, (int64_t)(a.part_bytes / 16));
    if (hipGetLastError() != hipSuccess) return -1;
    int rc = -1;
    switch (p.KS) {
        case 1: rc = launch_ks<1>(p, a, fused, s); break;
        case 2: rc = launch_ks<2>(p, a, fused, s); break;
        case 3: rc = launch_ks<3>(p, a, fused, s); break;
        case 4: rc = launch_ks<4>(p, a, fused, s); break;
        case 5: rc = launch_ks<5>(p, a, fused, s); break;
    }
    if (rc || !fused) return rc;
    // post and comb (and pre when not written above): the split + Sinkhorn of
    // the mixes, in the same per-token code as hc_split_sinkhorn
    return launch_split(a.mixes, scale, base, nullptr, post, comb, n, iters, eps, s);
}

}  // namespace hc
