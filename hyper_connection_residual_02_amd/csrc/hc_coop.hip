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
//    registers, and forms the sums of squares (plain, and of the values
//    scaled by 2^-72 for streams whose plain sum overflows fp32) on the
//    matrix core as the diagonal of A A^T.
//  * The member's 26 partial sums per token are published to the workspace
//    as tagged 16-byte records (3 floats + a round tag), stored member-
//    fastest so that the G records of a (token, chunk) are contiguous.
//    Every member reads the pre-relevant records (m_0..m_3 and the sums of
//    squares) of all members with contiguous loads, adds them across lanes
//    in one fixed butterfly order, forms pre for all T tokens, and writes h
//    for its slice from the residual still in registers (staged through
//    LDS for coalesced stores): one HBM pass over the residual.  The owner
//    of each token (member t mod G) adds all 26 fields the same way and
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
//    XCD (workgroups are dispatched round-robin over the XCDs).  Records
//    are written and read at device scope (loads skip the L1, whose copy
//    of a slot's previous record a group-scope load can keep returning), so
//    placement only affects speed.
//  * Every wait is bounded in time; a timed-out wait raises a flag in the
//    workspace header and the workgroup stops.

#include <atomic>
#include <mutex>
#include <stddef.h>

#include "hc_device.hpp"
#include "hc_launch.hpp"

namespace hc {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kTT = 2;             // 16-token tiles per round
constexpr int kKG = 4;             // k-groups of a member's slice
constexpr int kT = 16 * kTT;       // tokens per round
constexpr int kTiles = 5;          // 5 x 16 = 80 MFMA columns (72 used)
constexpr int kChunks = 9;         // 16-byte chunks per partial record (26 fields + tag words)
constexpr int kSlots = 4;          // rounds of records kept per group
constexpr int kRed = 26;           // floats per token in the per-k-group LDS partials
constexpr int kPrePairs = 2 * kT;  // (chunk, token) pairs holding the pre-relevant fields
constexpr int kOwnPairs = kChunks * kT;   // (owned token, chunk) pairs at most (G = 1)
constexpr uint64_t kMagic = 0x6863776b73703031ull;   // marks an initialised workspace
constexpr uint32_t kEpochMask = 0xFFFFFu;            // 20-bit call epoch in each tag
constexpr int kBufDword3 = 0x00020000;               // raw buffer resource, dword 3
constexpr int kOOB = 0x7FFFFFF0;   // buffer offset past every resource: loads read 0, stores drop

// Workspace header (first 256 bytes): magic, call epoch, error flags, the
// length (16-byte records) of the record area known to hold only tagged
// records or zeros, and the per-group arrival words of the wave-specialised
// kernel's start-up.
constexpr int kMaxGroups = 32;     // token groups of the wave-specialised kernel (G >= 8)
struct WsHeader {
    uint64_t magic;
    uint32_t epoch;
    uint32_t err;       // this call: a bounded wait gave up (the call's workgroups stop)
    int64_t clean;
    uint32_t clear;     // this call clears its record area before use
    uint32_t failed;    // sticky: a call on this workspace gave up; cleared by the host status query
    uint32_t garr[kMaxGroups];   // group g, this call: members arrived (low 16 bits) and
                                 // members not on the group's XCD (high 16 bits)
};

static_assert(sizeof(WsHeader) <= 256, "the header occupies the first 256 bytes of the workspace");

// Epoch of call number `call` (process-wide call counter): 1 .. kEpochMask.
__host__ __device__ inline uint32_t epoch_of(uint64_t call) { return 1u + (uint32_t)(call % kEpochMask); }

// Header update at the start of a call.  The record area must be cleared
// on the first use of a workspace, when the call epoch does not increase
// (the 20-bit epoch wrapped, or calls were numbered elsewhere), and when
// this call's record area reaches past the part known to be clean (a
// previous call may have kept its mixes there), so that a record never
// carries a current tag before this call writes it.  Past this call's
// record area the workspace may receive mixes, so only that area stays
// known clean.  Returns whether to clear.
__device__ inline bool header_update(WsHeader* hdr, uint64_t call, int64_t nchunks, int ngroups) {
    const uint32_t ep = epoch_of(call);
    const bool fresh = hdr->magic != kMagic;
    const bool clear = fresh || ep <= hdr->epoch || hdr->clean < nchunks;
    if (fresh) hdr->failed = 0u;
    hdr->magic = kMagic;
    hdr->epoch = ep;
    hdr->err = 0u;
    hdr->clean = nchunks;
    for (int g = 0; g < ngroups && g < kMaxGroups; ++g) hdr->garr[g] = 0u;
    hdr->clear = clear ? 1u : 0u;
    return clear;
}

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
    uint64_t call;      // process-wide number of this call (sets the record epoch)
    const u32x4* Wp;    // weights already split into MFMA pieces (hc_pack_weights), or null
    uint64_t spin;      // bound of an exchange wait, in s_memrealtime ticks (100 MHz)
    uint32_t force_tag; // 0; nonzero (diagnostics only) makes every exchange record look stale
    // hc_post_mix_pre in one pass (k_spec, PO): R' = hc_post(x, R, post, comb)
    // is formed from each round of R on its way through LDS, written to Rout
    // (which may be R), and projected in place of R.
    const uint16_t* x;  // sublayer output [n][d]
    const float* postp; // the previous sublayer's post [n][4] and comb [n][4][4]
    const float* combp;
    uint16_t* Rout;
};

// A bounded wait of this call gave up: peers stop when they see err, and
// the sticky failed word tells the host (hc_workspace_status).
__device__ __forceinline__ void give_up(const CoopArgs& a) {
    __hip_atomic_store(&a.hdr->err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&a.hdr->failed, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Field f of a partial record (0..23 = the 24 dot products, 24 = sum of
// squares, 25 = sum of squares of the values times 2^-72) by chunk and
// slot.  The pre-relevant fields (0..3, 24 and 25) are in chunks 0 and 1.
__device__ __forceinline__ int field_at(int chunk, int slot) {
    if (chunk == 0) return slot;                                    // m0 m1 m2
    if (chunk == 1) return slot == 0 ? 3 : 23 + slot;               // m3 ss sb
    const int f = 4 + 3 * (chunk - 2) + slot;                       // m4 .. m23
    return f <= 23 ? f : -1;
}
__device__ __forceinline__ void field_pos(int f, int& chunk, int& slot) {
    if (f < 3) { chunk = 0; slot = f; }
    else if (f == 3) { chunk = 1; slot = 0; }
    else if (f >= 24) { chunk = 1; slot = f - 23; }
    else { chunk = 2 + (f - 4) / 3; slot = (f - 4) % 3; }
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
    float s0, bpre;         // hc_scale[0] and hc_base of the lane's pre stream, read once: a parameter
                            // load inside the loop would be the youngest memory op, and
                            // waiting for it would wait for every prefetch
};

// hc_base[thread % 4] from four uniform (scalar) loads: a per-lane vector
// load would be waited for where it is first used inside the round loop,
// and that wait would also wait for every store still in flight.
__device__ __forceinline__ float base_of_lane(const float* base, int k) {
    const float b0 = base[0], b1 = base[1], b2 = base[2], b3 = base[3];
    return k == 0 ? b0 : (k == 1 ? b1 : (k == 2 ? b2 : b3));
}

__device__ __forceinline__ uint32_t tag_of(const RoundCtx& c, int r) {
    return (c.epoch << 12) | ((uint32_t)r & 0xFFFu);
}

// Byte offset of record chunk (member, token t, chunk) of round r.
__device__ __forceinline__ int rec_off(const CoopArgs& a, const RoundCtx& c, int r, int chunk, int t, int member) {
    const int slot = r % kSlots;
    return ((((c.g * kSlots + slot) * kChunks + chunk) * kT + t) * a.GP + member) * 16;
}

__device__ __forceinline__ u32x4 ld_l2(const RoundCtx& c, int off) {   // first read: device scope, skips the L1
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(c.rsrc, off, 0, 16));
}
__device__ __forceinline__ u32x4 ld_dev(const RoundCtx& c, int off) {  // re-read: device scope
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

// Buffer resource over the 16 tokens of tile tt of round r in a
// [n][per_tok] array; loads past the last token read zeros and stores past
// it are dropped by the hardware bounds check.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, int64_t per_tok_bytes, int64_t tok0,
                                                          int64_t n, int64_t ntok = 16) {
    int64_t valid = base ? n - tok0 : 0;
    valid = valid < 0 ? 0 : (valid > ntok ? ntok : valid);
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

// Sums of squares of a 16-token MFMA tile.  With the A operand also as B
// an MFMA gives A A^T, whose diagonal holds each token row's sum of squares
// (products of bf16 values are exact in fp32); diagonal element (i, i) sits
// in lane i + 16 * (i / 4), component i % 4.
__device__ __forceinline__ void sq_step(const u32x4& av, f32x4& sq) {
    const bf16x8 ab = __builtin_bit_cast(bf16x8, av);
    sq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ab, ab, sq, 0, 0, 0);
}
__device__ __forceinline__ void sq_step_scaled(const u32x4& av, f32x4& sb) {
    u32x4 sv;
#pragma unroll
    for (int e = 0; e < 4; ++e) sv[e] = scaled_x2(av[e]);
    const bf16x8 ab = __builtin_bit_cast(bf16x8, sv);
    sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ab, ab, sb, 0, 0, 0);
}
// The scaled sum of the tile (values times 2^-72) from its plain sum ss:
// while ss is finite, ss * 2^-144 (whatever underflows is below 2^-126, far
// under one ulp of a total that has overflowed unscaled, the only case in
// which the scaled sum is used); where any token row of the wave overflowed,
// `redo` recomputes the scaled sums from the operands (a wave-uniform,
// rare branch).  Valid on the diagonal lanes.
template <typename Redo>
__device__ __forceinline__ float scaled_sum(int row, int grp, float ss, Redo&& redo) {
    const bool diag = (row >> 2) == grp;
    float sb = (ss * 0x1p-72f) * 0x1p-72f;
    if (__builtin_amdgcn_ballot_w64(diag && !(ss <= 3.40282347e38f))) sb = redo()[row & 3];
    return sb;
}

// ---------------------------------------------------- stage A: publish r
// f holds round r in MFMA operand layout.
template <int KS>
__device__ __forceinline__ void publish(const Frags<KS>& f, const CoopArgs& a, const RoundCtx& c, Lds<KS>& L,
                                        int r) {
    f32x4 acc[kTiles];
#pragma unroll
    for (int ct = 0; ct < kTiles; ++ct) acc[ct] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    f32x4 sq = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // weight operands double-buffered from LDS: the reads for k-step s+1
    // are in flight while the MFMAs of step s run
    bf16x8 bw[2][kTiles];
#pragma unroll
    for (int ct = 0; ct < kTiles; ++ct) bw[0][ct] = L.wf[c.kg * KS][ct][c.l];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const bf16x8 av = __builtin_bit_cast(bf16x8, f.r[s]);
        if (s + 1 < KS) {
#pragma unroll
            for (int ct = 0; ct < kTiles; ++ct) bw[(s + 1) & 1][ct] = L.wf[c.kg * KS + s + 1][ct][c.l];
        }
#pragma unroll
        for (int ct = 0; ct < kTiles; ++ct)
            acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bw[s & 1][ct], acc[ct], 0, 0, 0);
        sq_step(f.r[s], sq);
    }
    {
        const float ss = sq[c.row & 3];
        const float sb = scaled_sum(c.row, c.grp, ss, [&] {
            f32x4 v = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < KS; ++s) sq_step_scaled(f.r[s], v);
            return v;
        });
        if ((c.row >> 2) == c.grp) {
            L.u.red[c.kg][16 * c.tt + c.row][24] = ss;
            L.u.red[c.kg][16 * c.tt + c.row][25] = sb;
        }
    }
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
    // 9 records per token from the first 288 threads; the other threads'
    // stores go past the resource and are dropped (no branch around the
    // store keeps the memory counters countable)
    const int tid = threadIdx.x;
    const int ch = tid / kT, t = tid - ch * kT;
    u32x4 v;
#pragma unroll
    for (int sl = 0; sl < 3; ++sl) {
        const int fi = field_at(ch, sl);      // -1 for ch >= kChunks
        float x = 0.0f;
        if (fi >= 0) x = ((L.u.red[0][t][fi] + L.u.red[1][t][fi]) + L.u.red[2][t][fi]) + L.u.red[3][t][fi];
        v[sl] = __float_as_uint(x);
    }
    v[3] = tag_of(c, r);
    st_dev(c, ch < kChunks ? rec_off(a, c, r, ch, t, c.q) : kOOB, v);
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
            const bool ok = pair < kPrePairs && m < a.G;
            X.pre[j] = ld_l2(c, ok ? rec_off(a, c, r, pair / kT, pair % kT, m) : kOOB);
        }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int x = j * kThreads + tid;
        const int pair = x >> a.gp_log2, m = x & (a.GP - 1);
        const int o = pair / kChunks, ch = pair - o * kChunks;
        const bool ok = o < c.nown && m < a.G;
        X.own[j] = ld_l2(c, ok ? rec_off(a, c, r, ch, c.q + a.G * o, m) : kOOB);
    }
}

// Position of pre-relevant load j / owned load j of this thread: (chunk,
// token, member), and whether it names a real record.
__device__ __forceinline__ bool pre_pos(const CoopArgs& a, int j, int& chunk, int& t, int& m) {
    const int x = j * kThreads + (int)threadIdx.x;
    const int pair = x >> a.gp_log2;
    m = x & (a.GP - 1);
    chunk = pair / kT;
    t = pair - chunk * kT;
    return pair < kPrePairs && m < a.G;
}
__device__ __forceinline__ bool own_pos(const CoopArgs& a, const RoundCtx& c, int j, int& chunk, int& t, int& m) {
    const int x = j * kThreads + (int)threadIdx.x;
    const int pair = x >> a.gp_log2;
    m = x & (a.GP - 1);
    const int o = pair / kChunks;
    chunk = pair - o * kChunks;
    t = c.q + a.G * o;
    return o < c.nown && m < a.G;
}

// Member sums of the 3 floats of a record (zeros where there is none).
__device__ __forceinline__ void chunk_sum(const u32x4& v, const CoopArgs& a, float* s3) {
    s3[0] = group_sum(__uint_as_float(v[0]), a.GP);
    s3[1] = group_sum(__uint_as_float(v[1]), a.GP);
    s3[2] = group_sum(__uint_as_float(v[2]), a.GP);
}

// Exchange of round r: member sums of the pre-relevant records of every
// token (into L.xsum) and of all records of the owned tokens (into
// L.xown), in one fixed reduction order shared by both, so pre formed here
// is bitwise the pre of the owner's mixes.  A wave any of whose records
// still carries an older tag re-reads those records at device scope until
// they are current (bounded in time).  Returns true if any thread of the
// workgroup hit a timeout.
template <int PI, int KS, bool FUSED>
__device__ __forceinline__ bool exchange(XLoads<PI>& X, const CoopArgs& a, const RoundCtx& c, Lds<KS>& L,
                                         int r) {
    const uint32_t tag = tag_of(c, r) ^ a.force_tag;
    int chunk, t, m;
    bool stale = false;
    if (FUSED) {
#pragma unroll
        for (int j = 0; j < PI; ++j) stale |= pre_pos(a, j, chunk, t, m) && X.pre[j][3] != tag;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) stale |= own_pos(a, c, j, chunk, t, m) && X.own[j][3] != tag;
    int bad = 0;
    if (__builtin_amdgcn_ballot_w64(stale)) {           // wave-uniform, rare
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        for (;;) {
            bool again = false;
            if (FUSED) {
#pragma unroll
                for (int j = 0; j < PI; ++j)
                    if (pre_pos(a, j, chunk, t, m) && X.pre[j][3] != tag) {
                        X.pre[j] = ld_dev(c, rec_off(a, c, r, chunk, t, m));
                        again |= X.pre[j][3] != tag;
                    }
            }
#pragma unroll
            for (int j = 0; j < 2; ++j)
                if (own_pos(a, c, j, chunk, t, m) && X.own[j][3] != tag) {
                    X.own[j] = ld_dev(c, rec_off(a, c, r, chunk, t, m));
                    again |= X.own[j][3] != tag;
                }
            if (!__builtin_amdgcn_ballot_w64(again)) break;
            if (__builtin_amdgcn_s_memrealtime() - t0 > a.spin ||
                __hip_atomic_load(&a.hdr->err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
                give_up(a);
                bad = 1;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    const int tid = threadIdx.x;
    if (FUSED) {
#pragma unroll
        for (int j = 0; j < PI; ++j) {
            if (j * kThreads < kPrePairs * a.GP) {          // block-uniform: this load carries pairs
                const bool ok = pre_pos(a, j, chunk, t, m);
                float s3[3];
                chunk_sum(X.pre[j], a, s3);                 // zeros where !ok (load past the resource)
                if (m == 0 && ok) {
                    const int pair = chunk * kT + t;
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
            const int pair = x >> a.gp_log2;
            const bool ok = own_pos(a, c, j, chunk, t, m);
            float s3[3];
            chunk_sum(X.own[j], a, s3);
            if (m == 0 && ok) {
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
    if (FUSED) {
        // threads < 128: pre of (token tid/4, stream tid%4); the others
        // compute a copy of it and their store is dropped
        const int t = (tid >> 2) & (kT - 1), j = tid & 3;
        const float sj = j < 3 ? L.xsum[t][j] : L.xsum[kT + t][0];     // m_0..m_2: chunk 0; m_3: chunk 1 slot 0
        // sums of squares: chunk 1 slots 1 and 2
        const MixScale ms = mix_scale(L.xsum[kT + t][1], L.xsum[kT + t][2], a.K, a.norm_eps);
        const float p = pre_gate(mix_value(sj, ms), c.s0, c.bpre, a.eps);
        if (tid < kT * 4) L.preL[t][j] = p;
        // the owner writes pre (a null pre gives an empty resource)
        const __amdgpu_buffer_rsrc_t rp = tile_rsrc(a.pre, kHC * 4, tok0, a.n, kT);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(p), rp,
                                              tid < kT * 4 && t % a.G == c.q ? (t * kHC + j) * 4 : kOOB, 0, 0);
    }
    // mixes of the owned tokens; a fixed number of passes, with the stores
    // of threads past the owned mixes dropped by the resource bound
    const int base = FUSED ? kT * 4 : 0;
    const __amdgpu_buffer_rsrc_t rm = tile_rsrc(a.mixes, kMix * 4, tok0, a.n, kT);
    constexpr int kPasses = (kT * kMix + (kThreads - (FUSED ? kT * 4 : 0)) - 1) / (kThreads - (FUSED ? kT * 4 : 0));
#pragma unroll
    for (int it = 0; it < kPasses; ++it) {
        const int x = tid - base + it * (kThreads - base);
        const bool ok = x >= 0 && x < c.nown * kMix;
        const int xx = ok ? x : 0;
        const int o = xx / kMix, j = xx - o * kMix;
        int ch, sl;
        field_pos(j, ch, sl);
        const MixScale ms = mix_scale(L.xown[o * kChunks + 1][1], L.xown[o * kChunks + 1][2], a.K, a.norm_eps);
        const float v = mix_value(L.xown[o * kChunks + ch][sl], ms);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rm, ok ? ((c.q + a.G * o) * kMix + j) * 4 : kOOB,
                                              0, 0);
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
    // past the group's last round these load zeros (empty resource) and
    // publish records that nobody reads; no branch keeps the memory
    // counters countable, so waits stay partial
    load_round<KS>(P, a, c, i + 3);
    to_operands<KS>(M, c, L);
    publish<KS>(M, a, c, L, i + 1);
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
    c.w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);     // wave-uniform: scalar
    c.l = threadIdx.x & 63;
    c.row = c.l & 15;
    c.grp = c.l >> 4;
    c.tt = c.w & 1;
    c.kg = c.w >> 1;
    c.nown = c.q < kT ? (kT - 1 - c.q) / a.G + 1 : 0;
    c.epoch = epoch_of(a.call);
    c.rsrc = __builtin_amdgcn_make_buffer_rsrc(a.part, 0, a.part_bytes, kBufDword3);
    if (c.g >= a.ntiles) return;
    c.s0 = FUSED ? a.scale[0] : 0.0f;
    c.bpre = FUSED ? base_of_lane(a.base, threadIdx.x & 3) : 0.0f;
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
    load_round<KS>(M, a, c, 1);
    load_round<KS>(A, a, c, 2);
    to_operands<KS>(H, c, L);
    publish<KS>(H, a, c, L, 0);
    for (int i = 0; i < c.nr; i += 2) {
        if (!iteration<KS, PI, FUSED>(H, M, A, B, a, c, L, i)) return;
        if (i + 1 >= c.nr) break;
        if (!iteration<KS, PI, FUSED>(H, M, B, A, a, c, L, i + 1)) return;
    }
}

// ====================================================== wave-specialised kernel
// Used when a group has 8..32 members.  The 8 waves of a workgroup split
// into two roles that run one round apart, with one workgroup barrier per
// round ("tick"):
//
//  * MFMA waves (0..3): wave w handles stream w of the member slice and
//    keeps that stream's weight slice in registers (MFMA B layout), so the
//    weights never go through LDS.  In tick t a wave writes the records of
//    round t-1 from the per-wave partials of the previous tick, issues the
//    residual of round t+2 as direct global->LDS loads into slot (t+2) % 3,
//    multiplies round t out of slot t % 3 into per-wave partials, and waits
//    until round t+1 has landed in LDS.
//  * Exchange waves (4..7): wave x handles tokens 8x..8x+7 of a round.  In
//    tick t it reads the records of round t-2, forms pre for its tokens
//    (and the mixes of the token it owns), writes h of round t-2 from the
//    residual it copied out of slot (t-2) % 3 two ticks earlier, and copies
//    round t out of slot t % 3 for use two ticks later.
//
// The direct-to-LDS loads are issued with inline assembly, so the
// compiler's memory fences at the barriers do not wait for them; the MFMA
// waves wait for them explicitly with a vmcnt count that is exact for the
// fixed sequence of memory instructions of a tick.
namespace spec {

// Phase tracing of the wave-specialised kernel, compiled in only with
// HC_PHASE_TRACE (the library built by `hyper_connection_residual_02_amd.build
// --phase-trace`; hc_phase_trace copies the tables out).  Lane 0 of each
// wave adds the s_memrealtime ticks (100 MHz) since its previous mark to the
// phase just ended, in LDS; at the end every workgroup writes its waves'
// totals and its tick count to kTrace.  Phases of the MFMA waves: 0 waiting
// at the tick's barrier, 1 publication, 2 DMA issue, 3 products, 4 waiting
// for the next round's DMA (with PO: and for the four waves' arrival), 5
// (PO) hc_post of the next round.  Exchange waves: 0 barrier, 1 exchange
// (tag check, member sums, pre, the owned token's mixes), 2 h, 3 residual
// copy, 4 record-load issue, 5 (PO) R' stores.  Each workgroup also stamps
// the clock at four points (kTraceTs): entry, the end of the start-up
// protocol (run by the first exchange wave), the start of the round loop
// (after the weights and the first residual loads) and the end.
#ifdef HC_PHASE_TRACE
constexpr int kTrPhases = 6;
constexpr int kTrMaxBlocks = 1024;
constexpr int kTrWords = kWaves * (kTrPhases + 1);       // per workgroup: per wave the phases, then ticks
__device__ uint64_t kTrace[kTrMaxBlocks * kTrWords];
__device__ uint64_t kTraceTs[kTrMaxBlocks * 4];
__shared__ uint32_t tr_tot[kWaves][kTrPhases];
__shared__ uint32_t tr_last[kWaves];
__shared__ uint64_t tr_ts[4];
__device__ __forceinline__ void tr_stamp(int i, unsigned tid = 0) {
    if (threadIdx.x == tid) tr_ts[i] = __builtin_amdgcn_s_memrealtime();
}
__device__ __forceinline__ void tr_start() {
    if ((threadIdx.x & 63) == 0) {
        const int w = threadIdx.x >> 6;
        for (int i = 0; i < kTrPhases; ++i) tr_tot[w][i] = 0u;
        tr_last[w] = (uint32_t)__builtin_amdgcn_s_memrealtime();
    }
}
__device__ __forceinline__ void tr_mark(int ph) {
    if ((threadIdx.x & 63) == 0) {
        const int w = threadIdx.x >> 6;
        const uint32_t now = (uint32_t)__builtin_amdgcn_s_memrealtime();
        tr_tot[w][ph] += now - tr_last[w];
        tr_last[w] = now;
    }
}
__device__ __forceinline__ void tr_finish(int ticks) {
    if ((threadIdx.x & 63) == 0 && blockIdx.x < (unsigned)kTrMaxBlocks) {
        const int w = threadIdx.x >> 6;
        uint64_t* o = &kTrace[(size_t)blockIdx.x * kTrWords + w * (kTrPhases + 1)];
        for (int i = 0; i < kTrPhases; ++i) o[i] = tr_tot[w][i];
        o[kTrPhases] = (uint64_t)ticks;
        if (w == 0) {
            tr_ts[3] = __builtin_amdgcn_s_memrealtime();
            for (int i = 0; i < 4; ++i) kTraceTs[(size_t)blockIdx.x * 4 + i] = tr_ts[i];
        }
    }
}
#else
__device__ __forceinline__ void tr_stamp(int, unsigned = 0) {}
__device__ __forceinline__ void tr_start() {}
__device__ __forceinline__ void tr_mark(int) {}
__device__ __forceinline__ void tr_finish(int) {}
#endif

constexpr int kMW = 4;                  // MFMA waves
constexpr int kTokX = kT / 4;           // tokens per exchange wave
constexpr int kXL = 8;                  // exchange loads per lane and pass: 32 members / 4 lane groups

// Slot geometry.  A slot holds one round of the member's residual slice,
// 32 token rows.  PO (the sublayer-boundary variant, hc_post_mix_pre): rows
// carry no pad (their 16-byte chunks are XOR-swizzled instead, see roff),
// so that three slots still fit beside a two-slot ring of the round's x
// rows and the previous sublayer's post and comb, and the partials are
// single-buffered.
template <int KS, bool PO = false>
struct Geo {
    static constexpr int kRowB = PO ? 4 * 64 * KS : 4 * 64 * KS + 16;   // bytes per token row of R
    static constexpr int kRDma = PO ? 8 * KS : (kT * kRowB + 1023) / 1024;   // 1 KB loads of R per round
    static constexpr int kPostOff = 2 * KS * 1024;             // PO, x slot: x rows (64*KS bytes each) first,
    static constexpr int kCombOff = kPostOff + kT * 16;        // then post (16 B per token), comb (64 B)
    static constexpr int kXSlotB = kCombOff + kT * 64;
    static constexpr int kNeed = PO ? 10 * KS + 3 : kRDma;     // 1 KB loads per round
    static constexpr int kDmaW = (kNeed + kMW - 1) / kMW;      // per MFMA wave
    static constexpr int kSlotB = PO ? kRDma * 1024 : kDmaW * kMW * 1024;
    static constexpr int kNSlot = 3;                           // residual rounds held in LDS
    static constexpr int kNRed = PO ? 1 : 2;                   // partial buffers
    static constexpr int kBlk = 8 * KS;                        // 4-feature blocks per token and stream
    static constexpr int kItems = kTokX * kBlk;                // h items (token, block) per exchange wave
    static constexpr int kPass = (kItems + 63) / 64;           // KS = 5: 320 items, 5 full passes
    static constexpr int kPostItems = kT * 4 * KS;             // PO: hc_post items (token, 8 features)
};

template <int KS, bool PO = false>
struct Lds {
    uint8_t slot[Geo<KS, PO>::kNSlot][Geo<KS, PO>::kSlotB];
    uint8_t xs[PO ? 2 : 1][PO ? Geo<KS, PO>::kXSlotB : 16];   // PO: x, post, comb of rounds by parity
    float red[Geo<KS, PO>::kNRed][kMW][kT][kRed];   // per-MFMA-wave partials (by round parity if two)
    float xpre[4][kTokX][4];               // pre of each exchange wave's tokens
    float xown[4][10][4];                  // member sums of the owned token's records
    int stop;                              // set when a wait timed out
    uint32_t acnt;                         // PO: MFMA-wave arrivals, one per wave and tick
};

// Byte offset of byte b of token row tk's residual in a slot.  PO rows have
// no pad: their 16-byte chunk c sits at chunk c ^ (tk & 15), a permutation
// inside each aligned run of 16 chunks (a row has 16*KS), so that the 16
// rows of an MFMA operand read still fall on distinct LDS banks.
template <int KS, bool PO>
__device__ __forceinline__ int roff(int tk, int b) {
    if (!PO) return tk * Geo<KS, PO>::kRowB + b;
    return tk * Geo<KS, PO>::kRowB + ((((b >> 4) ^ (tk & 15))) << 4) + (b & 15);
}

typedef __attribute__((ext_vector_type(4))) uint32_t v4u;

// Raw buffer resource words over [base, base + bytes); made wave-uniform.
__device__ __forceinline__ v4u rsrc_words(uintptr_t base, uint32_t bytes) {
    v4u r;
    r.x = __builtin_amdgcn_readfirstlane((uint32_t)base);
    r.y = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32) & 0xFFFFu);
    r.z = __builtin_amdgcn_readfirstlane(bytes);
    r.w = (uint32_t)kBufDword3;
    return r;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p);
}

// One 16-byte-per-lane load from the buffer straight into LDS at
// lds + 16 * lane (M0 holds the LDS address; saved and restored).
__device__ __forceinline__ void dma16(v4u rs, uint32_t lds, uint32_t voff) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(rs), "s"(lds)
        : "memory");
}

// Index (16-byte units) of lane l's piece vector for member q, stream w,
// k-step st, column tile ct in the packed weights: [q][w][st][ct][lane].
template <int KS>
__device__ __forceinline__ int64_t packed_index(int q, int w, int st, int ct, int l) {
    return ((((int64_t)q * kHC + w) * KS + st) * kTiles + ct) * 64 + l;
}

template <int KS, bool PO = false>
struct MState {
    bf16x8 w[KS][kTiles];                  // weight slice of stream w, MFMA B layout
    uint32_t dvoff[Geo<KS, PO>::kDmaW];    // lane byte offsets of this wave's loads within a round
};

template <int KS>
struct XState {
    u32x2 rb[2][Geo<KS>::kPass][kHC];      // residual for h, two rounds (by parity)
    u32x4 P[kXL];                          // records of the next exchange (issued a tick early)
    u32x4 O[kXL];
    int pb, ob;                            // lane offsets of the pre and owner loads of load s = 0 in a
                                           // round's slot (load s adds s * kLoadStride)
};

// Record stores and loads.  Loads are device scope (sc1): they skip the
// L1, which may hold a copy of a slot's previous record (a group-scope load
// can keep returning that copy).  LOCAL: every member of the group runs on
// one XCD, so plain stores, which stay in that XCD's L2, are enough (about
// half the latency of a device-scope store); otherwise stores are device
// scope too.
template <bool LOCAL>
__device__ __forceinline__ u32x4 ld_rec(const RoundCtx& c, int off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(c.rsrc, off, 0, 16));
}
template <bool LOCAL>
__device__ __forceinline__ void st_rec(const RoundCtx& c, int off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((__vector_size__(16))) int, v), c.rsrc,
                                           off, 0, LOCAL ? 0 : 16);
}

// Weight slice of stream w split into MFMA B fragments: k-step st, lane
// (column i, k-block grp) holds features 32*st + 8*grp .. +7 of stream w of
// the member slice, as the bf16 piece (hi, mid or lo) of column tile ct.
// Each fragment is pinned in registers, which keeps the compiler from
// re-forming the pieces inside the round loop.
template <int KS, bool PO = false>
__device__ __forceinline__ void m_split_weights(MState<KS, PO>& S, const CoopArgs& a, const RoundCtx& c) {
    const int64_t K = (int64_t)kHC * a.d;
    // piece (0 hi, 1 mid, 2 lo, -1 none) and weight row of column tile ct
    auto tile_piece = [&](int ct, int& piece, int& j) {
        if (ct < 3) { piece = ct; j = c.row; }
        else if (ct == 3) { piece = c.row < 8 ? 0 : 1; j = 16 + (c.row & 7); }
        else { piece = c.row < 8 ? 2 : -1; j = 16 + c.row; }
    };
    // the fp32 weights of k-step st for every column tile
    auto fetch = [&](int st, f32x4 (&raw)[kTiles][2]) {
#pragma unroll
        for (int ct = 0; ct < kTiles; ++ct) {
            int piece, j;
            tile_piece(ct, piece, j);
            const int jj = piece < 0 ? 0 : j;
            const f32x4* src = reinterpret_cast<const f32x4*>(a.W + jj * K + (int64_t)c.w * a.d +
                                                              c.q * (32 * KS) + 32 * st + 8 * c.grp);
            raw[ct][0] = src[0];
            raw[ct][1] = src[1];
        }
    };
    // Loads of k-step st+1 are issued before the pieces of k-step st are
    // formed (the pin is a scheduling barrier, so a load placed after it
    // would wait for every earlier one): two weight round trips in flight
    // instead of one per column tile.
    f32x4 raw[2][kTiles][2];
    fetch(0, raw[0]);
#pragma unroll
    for (int st = 0; st < KS; ++st) {
        if (st + 1 < KS) fetch(st + 1, raw[(st + 1) & 1]);
#pragma unroll
        for (int ct = 0; ct < kTiles; ++ct) {
            int piece, j;
            tile_piece(ct, piece, j);
            const f32x4 w0 = raw[st & 1][ct][0], w1 = raw[st & 1][ct][1];
            bf16x8 v;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = e < 4 ? w0[e] : w1[e - 4];
                const __bf16 hi = (__bf16)x;
                const float r1 = x - (float)hi;
                const __bf16 mid = (__bf16)r1;
                const __bf16 lo = (__bf16)(r1 - (float)mid);
                v[e] = piece == 0 ? hi : (piece == 1 ? mid : (piece == 2 ? lo : (__bf16)0.0f));
            }
            u32x4 pinned = __builtin_bit_cast(u32x4, v);
            asm volatile("" : "+v"(pinned));
            S.w[st][ct] = __builtin_bit_cast(bf16x8, pinned);
        }
    }
}

// The same fragments from weights split once by k_pack, stored in this
// register layout: every load is issued before the first pin.
template <int KS, bool PO = false>
__device__ __forceinline__ void m_load_packed(MState<KS, PO>& S, const CoopArgs& a, const RoundCtx& c) {
    u32x4 pk[KS][kTiles];
#pragma unroll
    for (int st = 0; st < KS; ++st)
#pragma unroll
        for (int ct = 0; ct < kTiles; ++ct) pk[st][ct] = a.Wp[packed_index<KS>(c.q, c.w, st, ct, c.l)];
#pragma unroll
    for (int st = 0; st < KS; ++st)
#pragma unroll
        for (int ct = 0; ct < kTiles; ++ct) {
            u32x4 pinned = pk[st][ct];
            asm volatile("" : "+v"(pinned));
            S.w[st][ct] = __builtin_bit_cast(bf16x8, pinned);
        }
}

// Source of the 1 KB load instruction I of a round: 0 the residual, and
// with PO 1 the rows of x, 2 post (32 lanes), 3 comb.  Instructions past
// the round's (PO: the last wave's last one to three) repeat instruction
// I - 3 of the same wave: the same bytes to the same place, so that every
// wave issues kDmaW loads per round and the wait counts stay exact.
template <int KS, bool PO>
__host__ __device__ constexpr int dma_kind(int I) {
    if (!PO) return I < Geo<KS, PO>::kRDma ? 0 : -1;
    if (I >= 10 * KS + 3) I -= 3;
    if (I < 8 * KS) return 0;
    if (I < 10 * KS) return 1;
    return I == 10 * KS ? 2 : 3;
}
template <int KS, bool PO>
__host__ __device__ constexpr int dma_real(int I) { return PO && I >= 10 * KS + 3 ? I - 3 : I; }

// The loads of one MFMA wave W (PO), each instruction's source and
// destination fixed at compile time (no per-instruction branches).
struct DmaSrc {
    v4u rs, rx, rp, rc;
    uint32_t rbase, xbase;
    int lane;
};
template <int KS, int W, int I0, int N>
struct DmaRun {
    template <typename Off>
    __device__ __forceinline__ static void go(const DmaSrc& d, const Off& off) {
        if constexpr (N > 0) {
            using GG = Geo<KS, true>;
            constexpr int I = dma_real<KS, true>(W * GG::kDmaW + I0);
            constexpr int kind = dma_kind<KS, true>(I);
            if constexpr (kind == 0) {
                dma16(d.rs, d.rbase + I * 1024, off[I0]);
            } else if constexpr (kind == 1) {
                dma16(d.rx, d.xbase + (I - 8 * KS) * 1024, off[I0]);
            } else if constexpr (kind == 2) {
                // half an instruction's worth: only lanes 0..31 write, so
                // that comb can follow right after post
                if (d.lane < kT) dma16(d.rp, d.xbase + GG::kPostOff, off[I0]);
            } else {
                dma16(d.rc, d.xbase + GG::kCombOff + (I - 10 * KS - 1) * 1024, off[I0]);
            }
            DmaRun<KS, W, I0 + 1, N - 1>::go(d, off);
        }
    }
};

// The member's weight slice (packed, or split here) and the lane offsets of
// the residual loads (m_dma).  m_dma_offsets alone is enough to start
// loading rounds: k_spec and k_part issue their first rounds before
// fetching the weights, so that both round trips overlap.
template <int KS, bool PO = false>
__device__ __forceinline__ void m_weights(MState<KS, PO>& S, const CoopArgs& a, const RoundCtx& c) {
    if (a.Wp) m_load_packed<KS, PO>(S, a, c);
    else m_split_weights<KS, PO>(S, a, c);
}
template <int KS, bool PO = false>
__device__ __forceinline__ void m_dma_offsets(MState<KS, PO>& S, const CoopArgs& a, const RoundCtx& c) {
    using GG = Geo<KS, PO>;
#pragma unroll
    for (int i = 0; i < GG::kDmaW; ++i) {
        const int I = dma_real<KS, PO>(c.w * GG::kDmaW + i);
        const int kind = dma_kind<KS, PO>(I);
        uint32_t v = (uint32_t)kOOB;
        if (kind == 0) {
            // residual: token tk, stream k, byte off of the member's slice
            const int pos = I * 1024 + 16 * c.l;
            const int tk = pos / GG::kRowB, wb = pos - tk * GG::kRowB;
            const int lb = PO ? (((wb >> 4) ^ (tk & 15)) << 4) : wb;      // roff's inverse
            const int k = lb / (64 * KS), off = lb - k * (64 * KS);
            if (tk < kT && k < kHC) v = (uint32_t)(tk * 8 * a.d + k * 2 * a.d + c.q * (64 * KS) + off);
        } else if (kind == 1) {
            // x: token tk, byte off of the member's slice
            const int pos = (I - 8 * KS) * 1024 + 16 * c.l;
            const int tk = pos / (64 * KS), off = pos - tk * (64 * KS);
            v = (uint32_t)(tk * 2 * a.d + c.q * (64 * KS) + off);
        } else if (kind == 2) {
            v = (uint32_t)(16 * c.l);                                  // post, 16 B per token
        } else if (kind == 3) {
            v = (uint32_t)((I - 10 * KS - 1) * 1024 + 16 * c.l);      // comb, 64 B per token
        }
        S.dvoff[i] = v;
    }
}

// Round r of this group (rounds past the end: zeros) into slot r % 3; with
// PO the round's x rows and the previous sublayer's post and comb go to x
// slot r % 2, each from a resource bounded to the round's tokens.
template <int KS, bool PO = false>
__device__ __forceinline__ void m_dma(const MState<KS, PO>& S, const CoopArgs& a, const RoundCtx& c,
                                      Lds<KS, PO>& L, int r) {
    using GG = Geo<KS, PO>;
    const int64_t tok0 = tile_of(c, a, r) * kT;
    int64_t valid = a.n - tok0;
    valid = valid < 0 ? 0 : (valid > kT ? kT : valid);
    const int64_t t0 = valid > 0 ? tok0 : 0;
    const v4u rs = rsrc_words(reinterpret_cast<uintptr_t>(a.R) + (uintptr_t)t0 * 8 * a.d,
                              (uint32_t)(valid * 8 * a.d));
    const uint32_t rbase = lds_addr(&L.slot[r % GG::kNSlot][0]);
    if constexpr (!PO) {
        const uint32_t base = rbase + c.w * GG::kDmaW * 1024;
#pragma unroll
        for (int i = 0; i < GG::kDmaW; ++i) dma16(rs, base + i * 1024, S.dvoff[i]);
    } else {
        const v4u rx = rsrc_words(reinterpret_cast<uintptr_t>(a.x) + (uintptr_t)t0 * 2 * a.d,
                                  (uint32_t)(valid * 2 * a.d));
        const v4u rp = rsrc_words(reinterpret_cast<uintptr_t>(a.postp) + (uintptr_t)t0 * 16, (uint32_t)(valid * 16));
        const v4u rc = rsrc_words(reinterpret_cast<uintptr_t>(a.combp) + (uintptr_t)t0 * 64, (uint32_t)(valid * 64));
        const DmaSrc d{rs, rx, rp, rc, rbase, lds_addr(&L.xs[r & 1][0]), c.l};
        switch (c.w) {                        // wave-uniform
            case 0: DmaRun<KS, 0, 0, GG::kDmaW>::go(d, S.dvoff); break;
            case 1: DmaRun<KS, 1, 0, GG::kDmaW>::go(d, S.dvoff); break;
            case 2: DmaRun<KS, 2, 0, GG::kDmaW>::go(d, S.dvoff); break;
            default: DmaRun<KS, 3, 0, GG::kDmaW>::go(d, S.dvoff); break;
        }
    }
}

// Record layout of this kernel, per (group, slot): member-major.  A
// member's 288 records are chunks 0 and 1 (the pre-relevant fields) of the
// 32 tokens, token-major (1 KB), then chunks 2..8 of the 32 tokens,
// token-major (3.5 KB).  An exchange load then reads whole 256-byte runs of
// one member, the owner's loads two runs per member, and a publication
// store instruction 1 KB in one run.
constexpr int kRecPre = 2 * kT;                 // records of the pre-relevant run
constexpr int kRecMember = kChunks * kT;        // records per member and round
__device__ __forceinline__ int srec_index(int chunk, int t) {
    return chunk < 2 ? 2 * t + chunk : kRecPre + (kChunks - 2) * t + (chunk - 2);
}
__device__ __forceinline__ int srec_off(const CoopArgs& a, const RoundCtx& c, int r, int member, int rec) {
    const int slot = r % kSlots;
    return (((c.g * kSlots + slot) * a.GP + member) * kRecMember + rec) * 16;
}

// Where the two records a lane publishes per round come from: for record p
// of the lane (p = 0, 1) and slot sl, the offset of its field in one MFMA
// wave's partials (token * kRed + field; field 0 for the empty slot), and a
// bit per (p, sl) telling whether the slot holds a field.  Computed once
// before the round loop, so that the publication's LDS reads carry no
// per-lane branches and issue back to back.
struct PubMap {
    int off[2][3];
    uint32_t live;
};

// rec_of(id, tk, ch): token and chunk of record id of a member's round.
template <typename RecOf>
__device__ __forceinline__ PubMap pub_map(RecOf rec_of) {
    PubMap m;
    m.live = 0u;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int idx = p * (kMW * 64) + (int)threadIdx.x;
        const int id = idx < kRecMember ? idx : 0;      // lanes past the records compute record 0, dropped
        int tk, ch;
        rec_of(id, tk, ch);
#pragma unroll
        for (int sl = 0; sl < 3; ++sl) {
            const int fi = field_at(ch, sl);
            m.off[p][sl] = tk * kRed + (fi >= 0 ? fi : 0);
            if (fi >= 0) m.live |= 1u << (3 * p + sl);
        }
    }
    return m;
}

// Record p of the lane for the partials of round parity b: the four MFMA
// waves' partials of each field added in wave order.
template <int KS, bool PO = false>
__device__ __forceinline__ u32x4 pub_value(const Lds<KS, PO>& L, int b, const PubMap& m, int p) {
    const float* red = &L.red[b][0][0][0];
    constexpr int kW = kT * kRed;          // floats between two waves' partials
    float x[3];
#pragma unroll
    for (int sl = 0; sl < 3; ++sl) {
        const int o = m.off[p][sl];
        x[sl] = ((red[o] + red[o + kW]) + red[o + 2 * kW]) + red[o + 3 * kW];
    }
    // every lane uses all three sums here, so the compiler cannot move the
    // reads under the per-lane selects below (it would branch around each)
    asm volatile("" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]));
    u32x4 v;
#pragma unroll
    for (int sl = 0; sl < 3; ++sl) v[sl] = (m.live >> (3 * p + sl)) & 1u ? __float_as_uint(x[sl]) : 0u;
    v[3] = 0u;
    return v;
}

// Token and chunk of record id in this kernel's member-major order.
__device__ __forceinline__ void srec_of(int id, int& tk, int& ch) {
    const int q = id - kRecPre;
    tk = id < kRecPre ? id >> 1 : q / (kChunks - 2);
    ch = id < kRecPre ? id & 1 : 2 + (q - (kChunks - 2) * (q / (kChunks - 2)));
}

// Records of round r from the partials of the four MFMA waves (two store
// instructions per wave, always; past the group's rounds they are dropped).
// Lane idx writes record idx of this member.
template <int KS, bool LOCAL, bool PO = false>
__device__ __forceinline__ void m_publish(const CoopArgs& a, const RoundCtx& c, Lds<KS, PO>& L, const PubMap& M,
                                          int r) {
    const int tid = threadIdx.x;
    const bool live = r >= 0 && r < c.nr;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int idx = p * (kMW * 64) + tid;
        u32x4 v = pub_value<KS, PO>(L, Geo<KS, PO>::kNRed == 1 ? 0 : (r & 1), M, p);
        v[3] = tag_of(c, r);
        st_rec<LOCAL>(c, live && idx < kRecMember ? srec_off(a, c, r, c.q, idx) : kOOB, v);
    }
}

// Partial mixes and sums of squares of stream w for round r (slot r % 3).
template <int KS, bool PO = false>
__device__ __forceinline__ void m_mfma(const MState<KS, PO>& S, const RoundCtx& c, Lds<KS, PO>& L, int r) {
    const uint8_t* slot = &L.slot[r % Geo<KS, PO>::kNSlot][0];
    const int b = Geo<KS, PO>::kNRed == 1 ? 0 : (r & 1);
    auto operand = [&](int tt, int st) {
        return *reinterpret_cast<const u32x4*>(slot + roff<KS, PO>(16 * tt + c.row, c.w * (64 * KS) + 64 * st +
                                                                                         16 * c.grp));
    };
    // the products of both 16-token tiles go to the matrix core before
    // either tile's sums are read back, so that the read-back of one
    // overlaps the other's products (each accumulator sees the k-steps in
    // the same order as before)
    f32x4 accs[kTT][kTiles], sqs[kTT];
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt) {
#pragma unroll
        for (int ct = 0; ct < kTiles; ++ct) accs[tt][ct] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        sqs[tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int st = 0; st < KS; ++st) {
            const u32x4 av = operand(tt, st);
            const bf16x8 ab = __builtin_bit_cast(bf16x8, av);
#pragma unroll
            for (int ct = 0; ct < kTiles; ++ct)
                accs[tt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ab, S.w[st][ct], accs[tt][ct], 0, 0, 0);
            sq_step(av, sqs[tt]);
        }
    }
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt) {
        const f32x4* acc = accs[tt];
        const f32x4 sq = sqs[tt];
        {
            const float ss = sq[c.row & 3];
            const float sb = scaled_sum(c.row, c.grp, ss, [&] {
                f32x4 v = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int st = 0; st < KS; ++st) sq_step_scaled(operand(tt, st), v);
                return v;
            });
            if ((c.row >> 2) == c.grp) {
                L.red[b][c.w][16 * tt + c.row][24] = ss;
                L.red[b][c.w][16 * tt + c.row][25] = sb;
            }
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int t = 16 * tt + 4 * c.grp + rr;
            const float v0 = (acc[2][rr] + acc[1][rr]) + acc[0][rr];
            const float t3 = acc[3][rr];
            const float t3x = dpp<0x128>(t3);
            const float v1 = (acc[4][rr] + t3x) + t3;
            L.red[b][c.w][t][c.row] = v0;
            if (c.row < 8) L.red[b][c.w][t][16 + c.row] = v1;
        }
    }
}

// The one sync inside a tick (PO), on an LDS counter rather than a
// workgroup barrier, so that the two wave roles keep their own pace: in tick
// t each MFMA wave counts itself in on `acnt` once its own loads of round
// t+1 have landed (a wave only waits for the loads it issued) and its
// publication of round t-1 has read the partials; when the count reaches
// 4(t+2) round t+1 may be read by every wave and the partials rewritten
// (the prologue's arrival, for round 0, is the first).  A wait is bounded in
// time like every other wait (about 2 s) and stops early when the call has
// given up; it returns true then.
__device__ __forceinline__ void m_arrive(uint32_t* cnt) {
    if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ bool m_wait(const CoopArgs& a, const uint32_t* cnt, uint32_t target) {
    if (__hip_atomic_load(cnt, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) return false;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    for (;;) {
        __builtin_amdgcn_s_sleep(1);
        if (__hip_atomic_load(cnt, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) return false;
        if (__builtin_amdgcn_s_memrealtime() - t0 > 200000000ull ||
            __hip_atomic_load(&a.hdr->err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
            give_up(a);
            return true;
        }
    }
}

// hc_post of round r in its slot (PO): R'_{k,c} = bf16(post_k x_c +
// sum_j comb[j][k] R_{j,c}) for the four streams of every feature of the
// member's slice ("Mix projection" page, Block.hc_post), with the
// arithmetic of the standalone hc_post (post_words_lean: the same double
// sums and rounding), so the results are bitwise its results.  R' replaces
// R in the slot, so the products, the sums of squares and h of this round
// see R'; the exchange waves write it to Rout from their copy of the round
// (x_store).  A lane's item is (token, 8 features) of all four streams in
// the full runs and (token, 4 features) in the half runs: the round's
// 128*KS items of 8 features are 2*KS runs of 64, the MFMA waves take run
// j by wave j % 4 and, when the run count is not a multiple of four, the
// last two runs as four runs of 64 half items, one per wave, so that the
// four waves do the same work.
template <int KS>
__device__ __forceinline__ void post_item(uint8_t* slot, const uint8_t* xs, int tk, int b0, bool half,
                                          int hoff) {
    using GG = Geo<KS, true>;
    const f32x4 q = *reinterpret_cast<const f32x4*>(xs + GG::kPostOff + 16 * tk);
    f32x4 cb[kHC];
#pragma unroll
    for (int j = 0; j < kHC; ++j) cb[j] = *reinterpret_cast<const f32x4*>(xs + GG::kCombOff + 64 * tk + 16 * j);
    if (!half) {
        uint32_t rv[kHC][4], xv[4], out[kHC][4];
#pragma unroll
        for (int k = 0; k < kHC; ++k) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(slot + roff<KS, true>(tk, k * (64 * KS) + b0));
#pragma unroll
            for (int w = 0; w < 4; ++w) rv[k][w] = v[w];
        }
        const u32x4 x4 = *reinterpret_cast<const u32x4*>(xs + tk * (64 * KS) + b0);
#pragma unroll
        for (int w = 0; w < 4; ++w) xv[w] = x4[w];
        post_words_lean<4>(q, cb, xv, rv, out);
#pragma unroll
        for (int k = 0; k < kHC; ++k)
            *reinterpret_cast<u32x4*>(slot + roff<KS, true>(tk, k * (64 * KS) + b0)) =
                u32x4{out[k][0], out[k][1], out[k][2], out[k][3]};
    } else {
        uint32_t rv[kHC][2], xv[2], out[kHC][2];
#pragma unroll
        for (int k = 0; k < kHC; ++k) {
            const u32x2 v = *reinterpret_cast<const u32x2*>(slot + roff<KS, true>(tk, k * (64 * KS) + b0 + hoff));
            rv[k][0] = v[0];
            rv[k][1] = v[1];
        }
        const u32x2 x2 = *reinterpret_cast<const u32x2*>(xs + tk * (64 * KS) + b0 + hoff);
        xv[0] = x2[0];
        xv[1] = x2[1];
        post_words_lean<2>(q, cb, xv, rv, out);
#pragma unroll
        for (int k = 0; k < kHC; ++k)
            *reinterpret_cast<u32x2*>(slot + roff<KS, true>(tk, k * (64 * KS) + b0 + hoff)) = u32x2{out[k][0], out[k][1]};
    }
}

template <int KS>
__device__ __forceinline__ void m_post(const CoopArgs& a, const RoundCtx& c, Lds<KS, true>& L, int r) {
    using GG = Geo<KS, true>;
    constexpr int kCh = 4 * KS;            // 8-feature chunks per (token, stream) of the slice
    static_assert(GG::kPostItems % 64 == 0, "whole runs of 64 hc_post items");
    constexpr int kRuns = GG::kPostItems / 64;
    constexpr int kFull = kRuns % kMW == 0 ? kRuns : kRuns - 2;     // runs taken whole
    static_assert(kRuns % kMW == 0 || kRuns % kMW == 2, "runs split evenly over the MFMA waves");
    uint8_t* slot = &L.slot[r % GG::kNSlot][0];
    const uint8_t* xs = &L.xs[r & 1][0];
#pragma unroll 1
    for (int j = c.w; j < kFull; j += kMW) {                 // c.w is wave-uniform
        int it = j * 64 + c.l;
        // formed anew in every round: held across the round loop, the
        // item's offsets would take registers
        asm volatile("" : "+v"(it));
        const int tk = it / kCh, ch = it - tk * kCh;
        post_item<KS>(slot, xs, tk, 16 * ch, false, 0);
    }
    if constexpr (kFull < kRuns) {
        // the last two runs as 256 half items, 64 per wave
        int hi = c.w * 64 + c.l;
        asm volatile("" : "+v"(hi));
        const int it = kFull * 64 + (hi >> 1);
        const int tk = it / kCh, ch = it - tk * kCh;
        post_item<KS>(slot, xs, tk, 16 * ch, true, 8 * (hi & 1));
    }
}

// Lane layout of the exchange loads: lane l = e + 16 g reads, in load s,
// the record of member 4s + g for entry e, so that a member sum is an
// in-lane sum over the kXL loads followed by a sum over the 4 lane groups
// (two swaps), with no dependent cross-lane chain.  Pre loads: entry e is
// chunk e % 2 of token 8xw + e / 2.  Owner loads: entry e is chunk e of the
// owned token (e < 9).  Members past G read past the resource (zeros).  The
// pre and owner paths add in the same order, so pre formed from the pre
// loads is bitwise the pre of the owner's mixes.
__device__ __forceinline__ int x_member(const RoundCtx& c, int s) { return 4 * s + (c.l >> 4); }

// Member sum of record slot sl of kXL loads (every lane of the wave with
// the same entry gets the same total).
__device__ __forceinline__ float member_sum(const u32x4 (&v)[kXL], int sl) {
    float x = __uint_as_float(v[0][sl]);
#pragma unroll
    for (int s = 1; s < kXL; ++s) x += __uint_as_float(v[s][sl]);
    auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(h[0]) + __uint_as_float(h[1]);
    auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

template <bool FUSED>
__device__ __forceinline__ bool pre_live(const CoopArgs& a, const RoundCtx& c, int s) {
    return FUSED && x_member(c, s) < a.G;
}
__device__ __forceinline__ bool own_live(const CoopArgs& a, const RoundCtx& c, int xw, int s) {
    return xw < c.nown && x_member(c, s) < a.G && (c.l & 15) < kChunks;
}
// Record loads of round r for exchange wave xw: the pre-relevant records
// (chunks 0 and 1) of tokens 8xw..8xw+7 and all records of owned token xw.
// Offsets: load s reads member 4s + lane / 16, so its offset within a
// round's slot is that of load 0 plus s * kLoadStride; the lane part is
// computed once (x_offsets) and each load costs one add.
constexpr int kLoadStride = 4 * kRecMember * 16;
template <int KS>
__device__ __forceinline__ void x_offsets(XState<KS>& X, const CoopArgs& a, const RoundCtx& c, int xw) {
    const int e = c.l & 15, mem0 = c.l >> 4;
    X.pb = (mem0 * kRecMember + srec_index(e & 1, kTokX * xw + (e >> 1))) * 16;
    X.ob = (mem0 * kRecMember + srec_index(e, c.q + a.G * xw)) * 16;
}
template <int KS, bool FUSED, bool LOCAL>
__device__ __forceinline__ void x_issue(XState<KS>& X, const CoopArgs& a, const RoundCtx& c, int xw, int r) {
    const int slot = ((c.g * kSlots + r % kSlots) * a.GP) * kRecMember * 16;    // srec_off of member 0, record 0
#pragma unroll
    for (int s = 0; s < kXL; ++s)
        X.P[s] = ld_rec<LOCAL>(c, pre_live<FUSED>(a, c, s) ? slot + X.pb + s * kLoadStride : kOOB);
    // the owned token's records: only the waves that own a token load them
    // (the others' would all fall outside the resource)
    if (xw < c.nown) {
#pragma unroll
        for (int s = 0; s < kXL; ++s)
            X.O[s] = ld_rec<LOCAL>(c, own_live(a, c, xw, s) ? slot + X.ob + s * kLoadStride : kOOB);
    } else {
#pragma unroll
        for (int s = 0; s < kXL; ++s) X.O[s] = u32x4{0u, 0u, 0u, 0u};
    }
}

// Exchange of round r for exchange wave xw, from the loads issued by
// x_issue: pre of tokens 8xw..8xw+7 (into L.xpre, and the pre output of the
// tokens this member owns) and the mixes of owned token xw.  A record that
// still carries an older tag is re-read until current (bounded in time).
// Returns true on a timeout.
template <int KS, bool FUSED, bool LOCAL, bool PO = false>
__device__ __forceinline__ bool x_exchange(XState<KS>& X, const CoopArgs& a, const RoundCtx& c, Lds<KS, PO>& L, int xw,
                                           int r) {
    const uint32_t tag = tag_of(c, r) ^ a.force_tag;
    const int l = c.l, e = l & 15;
    const int otk = c.q + a.G * xw;
    const int64_t tok0 = tile_of(c, a, r) * kT;
    bool stale = false;
#pragma unroll
    for (int s = 0; s < kXL; ++s) stale |= pre_live<FUSED>(a, c, s) && X.P[s][3] != tag;
#pragma unroll
    for (int s = 0; s < kXL; ++s) stale |= own_live(a, c, xw, s) && X.O[s][3] != tag;
    bool bad = false;
    if (__builtin_amdgcn_ballot_w64(stale)) {              // wave-uniform: a peer is late
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        for (;;) {
            // re-read every record of the exchange at once: a record that was
            // already current comes back unchanged (its slot is not rewritten
            // before every member has finished this round)
            x_issue<KS, FUSED, LOCAL>(X, a, c, xw, r);
            bool again = false;
#pragma unroll
            for (int s = 0; s < kXL; ++s) again |= pre_live<FUSED>(a, c, s) && X.P[s][3] != tag;
#pragma unroll
            for (int s = 0; s < kXL; ++s) again |= own_live(a, c, xw, s) && X.O[s][3] != tag;
            if (!__builtin_amdgcn_ballot_w64(again)) break;
            if (__builtin_amdgcn_s_memrealtime() - t0 > a.spin ||
                __hip_atomic_load(&a.hdr->err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
                give_up(a);
                bad = true;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    // lanes with an even entry e = 2j: pre of (token 8xw + j, stream g); the
    // odd neighbour holds the token's chunk 1 (m3 and the sums of squares)
    float pre_mine = 0.0f;
    const int k = l >> 4, j = e >> 1;
    if (FUSED) {
        const float v0 = member_sum(X.P, 0), v1 = member_sum(X.P, 1), v2 = member_sum(X.P, 2);
        const float n0 = dpp<0xF5>(v0), n1 = dpp<0xF5>(v1), n2 = dpp<0xF5>(v2);      // quad_perm [1,1,3,3]
        const float mk = k == 0 ? v0 : (k == 1 ? v1 : (k == 2 ? v2 : n0));
        pre_mine = pre_gate(mix_value(mk, mix_scale(n1, n2, a.K, a.norm_eps)), c.s0, c.bpre, a.eps);
        if ((e & 1) == 0) L.xpre[xw][j][k] = pre_mine;
    }
    // owned token q + G xw (waves that own one): entry e = chunk e, then
    // its mixes from lanes 0..23
    if (xw < c.nown) {
        const float v0 = member_sum(X.O, 0), v1 = member_sum(X.O, 1), v2 = member_sum(X.O, 2);
        if (l < kChunks) {
            L.xown[xw][l][0] = v0;
            L.xown[xw][l][1] = v1;
            L.xown[xw][l][2] = v2;
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");     // the wave reads back its own LDS writes
        const int f = l < kMix ? l : 0;
        int ch, sl;
        field_pos(f, ch, sl);
        const float v = mix_value(L.xown[xw][ch][sl], mix_scale(L.xown[xw][1][1], L.xown[xw][1][2], a.K, a.norm_eps));
        const __amdgpu_buffer_rsrc_t rm = tile_rsrc(a.mixes, kMix * 4, tok0, a.n, kT);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rm, l < kMix ? (otk * kMix + l) * 4 : kOOB, 0, 0);
    }
    if (FUSED) {
        // pre output of the tokens this member owns
        const int tk = kTokX * xw + j;
        const __amdgpu_buffer_rsrc_t rp = tile_rsrc(a.pre, kHC * 4, tok0, a.n, kT);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(pre_mine), rp,
                                              (e & 1) == 0 && tk % a.G == c.q ? (tk * kHC + k) * 4 : kOOB, 0, 0);
    }
    return bad;
}

// h of round r for exchange wave xw from the residual copy rb (items of 4
// features: token tk, block b).
template <int KS, bool PO = false>
__device__ __forceinline__ void x_h(const u32x2 (&rb)[Geo<KS>::kPass][kHC], const CoopArgs& a, const RoundCtx& c,
                                    Lds<KS, PO>& L, int xw, int r) {
    const int64_t tok0 = tile_of(c, a, r) * kT;
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(a.h, (int64_t)a.d * 2, tok0, a.n, kT);
    // pre of every pass's token, read from LDS together (one wait, not one
    // per pass)
    f32x4 pqs[Geo<KS>::kPass];
#pragma unroll
    for (int p = 0; p < Geo<KS>::kPass; ++p) {
        const int item = p * 64 + c.l;
        const int it = item < Geo<KS>::kItems ? item : 0;
        pqs[p] = *reinterpret_cast<const f32x4*>(&L.xpre[xw][it / Geo<KS>::kBlk][0]);
    }
#pragma unroll
    for (int p = 0; p < Geo<KS>::kPass; ++p) {
        const int item = p * 64 + c.l;
        const bool valid = item < Geo<KS>::kItems;
        const int it = valid ? item : 0;
        const int tk = it / Geo<KS>::kBlk, b = it - tk * Geo<KS>::kBlk;
        const f32x4 pq = pqs[p];
        const double p0 = pq[0], p1 = pq[1], p2 = pq[2], p3 = pq[3];
        auto sum = [&](int w, int e) {
            auto v = [&](uint32_t word) { return (double)(e ? bf_hi(word) : bf_lo(word)); };
            double y = p0 * v(rb[p][0][w]);
            y = __builtin_fma(p1, v(rb[p][1][w]), y);
            y = __builtin_fma(p2, v(rb[p][2][w]), y);
            return __builtin_fma(p3, v(rb[p][3][w]), y);
        };
        u32x2 out;
        float f[2][2];
        bool mid = false;
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            f[w][0] = f32_mid(sum(w, 0), mid);
            f[w][1] = f32_mid(sum(w, 1), mid);
        }
        if (__builtin_amdgcn_ballot_w64(mid)) {
#pragma unroll
            for (int w = 0; w < 2; ++w) out[w] = pack2(bf16_rn_f64(sum(w, 0)), bf16_rn_f64(sum(w, 1)));
        } else {
#pragma unroll
            for (int w = 0; w < 2; ++w) out[w] = pack2(bf16_rn(f[w][0]), bf16_rn(f[w][1]));
        }
        const int off = valid ? ((kTokX * xw + tk) * a.d + c.q * (32 * KS) + 4 * b) * 2 : kOOB;
        // non-temporal (nt): h is not read again by this call, and streaming
        // it out leaves fewer dirty lines for the next kernel to write back
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((__vector_size__(8))) int, out),
                                              rs, off, 0, 2);
    }
}

// Copy of round r's residual (slot r % 3) for this wave's h items.
template <int KS, bool PO = false>
__device__ __forceinline__ void x_copy(u32x2 (&rb)[Geo<KS>::kPass][kHC], const RoundCtx& c, Lds<KS, PO>& L, int xw,
                                       int r) {
    const uint8_t* slot = &L.slot[r % Geo<KS, PO>::kNSlot][0];
#pragma unroll
    for (int p = 0; p < Geo<KS>::kPass; ++p) {
        const int item = p * 64 + c.l;
        const int it = item < Geo<KS>::kItems ? item : 0;
        const int tk = it / Geo<KS>::kBlk, b = it - tk * Geo<KS>::kBlk;
#pragma unroll
        for (int k = 0; k < kHC; ++k)
            rb[p][k] = *reinterpret_cast<const u32x2*>(slot + roff<KS, PO>(kTokX * xw + tk, k * (64 * KS) + 8 * b));
    }
}

// PO: round r's R' to Rout from the copy just taken (the exchange waves'
// items cover the whole round), with non-temporal stores: this call does
// not read it back.  Taking the stores off the MFMA waves keeps them out of
// the way of those waves' residual loads.
template <int KS>
__device__ __forceinline__ void x_store(const u32x2 (&rb)[Geo<KS>::kPass][kHC], const CoopArgs& a,
                                        const RoundCtx& c, int xw, int r) {
    const int64_t tok0 = tile_of(c, a, r) * kT;
    int64_t valid = a.n - tok0;
    valid = valid < 0 ? 0 : (valid > kT ? kT : valid);
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        a.Rout + (valid > 0 ? tok0 : 0) * 4 * a.d, 0, (int)(valid * 8 * a.d), kBufDword3);
#pragma unroll
    for (int p = 0; p < Geo<KS>::kPass; ++p) {
        const int it = p * 64 + c.l;
        const int tk = it / Geo<KS>::kBlk, b = it - tk * Geo<KS>::kBlk;
        const int vo = (kTokX * xw + tk) * 8 * a.d + c.q * (64 * KS) + 8 * b;
#pragma unroll
        for (int k = 0; k < kHC; ++k)      // stream k's offset in the scalar operand
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((__vector_size__(8))) int, rb[p][k]),
                                                  ro, vo, k * 2 * a.d, 2);
    }
}

// Exchange-wave part of tick t; P is the parity of t (selects the residual
// copy).  Returns true on a timeout.
template <int KS, bool FUSED, bool LOCAL, int P, bool PO = false>
__device__ __forceinline__ bool x_tick(XState<KS>& X, const CoopArgs& a, const RoundCtx& c, Lds<KS, PO>& L, int t) {
    const int xw = c.w - kMW;
    bool bad = false;
    const bool xr = t >= 2 && t - 2 < c.nr;
    if (xr) bad = x_exchange<KS, FUSED, LOCAL, PO>(X, a, c, L, xw, t - 2);
    tr_mark(1);
    if (FUSED && xr && !bad) x_h<KS, PO>(X.rb[P], a, c, L, xw, t - 2);
    tr_mark(2);
    if (FUSED) x_copy<KS, PO>(X.rb[P], c, L, xw, t);
    tr_mark(3);
    if constexpr (PO) {
        if (t < c.nr) x_store<KS>(X.rb[P], a, c, xw, t);
        tr_mark(5);
    }
    // records of round t-1 (published at the start of this tick) for the
    // next tick's exchange: their latency overlaps the barrier
    if (t >= 1 && t - 1 < c.nr) x_issue<KS, FUSED, LOCAL>(X, a, c, xw, t - 1);
    tr_mark(4);
    return bad;
}

// The two roles run separate loops with the same barrier sequence: a
// prologue barrier, then one barrier per tick t = 0 .. nr+1 (the exchange of
// the last round happens in tick nr+1); after each barrier both read the
// stop flag, so both leave after the same tick.  The store scope of the
// records (LOCAL) is known only at the prologue barrier, so each role's
// loop is instantiated for both and chosen there.
//
// PO (hc_post_mix_pre): in tick t the MFMA waves publish round t-1, issue
// round t+2 (residual, x, post, comb) into the slots round t-1 left, count
// themselves in once their loads of round t+1 have landed, multiply round t
// (turned into R' last tick), and then turn round t+1 into R' in place
// (m_post), which the tick's closing barrier orders before round t+1's
// products and the exchange waves' copy of it.
template <int KS, bool FUSED, bool LOCAL, bool PO>
__device__ __forceinline__ void m_loop(MState<KS, PO>& S, const PubMap& M, const CoopArgs& a, const RoundCtx& c,
                                       Lds<KS, PO>& L) {
    const int last = c.nr + 1;
    for (int t = 0;; ++t) {
        // records first (peers are waiting for them), then the residual
        // loads, then the products of round t
        m_publish<KS, LOCAL, PO>(a, c, L, M, t - 1);
        tr_mark(1);
        if constexpr (PO) {
            // round t+2 into the slots round t-1 left; round t (R' since
            // last tick) is multiplied; round t+1 is turned into R'
            m_dma<KS, PO>(S, a, c, L, t + 2);
            tr_mark(2);
            // round t+1 landed (issued last tick): younger than its loads
            // are at most last tick's R' stores, this tick's two record
            // stores and its loads, and the R' stores are older than the
            // last kDmaW + 2, so waiting down to kDmaW + 2 covers round
            // t+1 (and those stores)
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(Geo<KS, PO>::kDmaW + 2) : "memory");
            m_arrive(&L.acnt);
            // every MFMA wave's publication has read the (single) partials
            const bool bad = m_wait(a, &L.acnt, 4u * (t + 2));
            if (bad) L.stop = 1;
            tr_mark(4);
            m_mfma<KS, PO>(S, c, L, t);
            tr_mark(3);
            if (t + 1 < c.nr && !bad) m_post<KS>(a, c, L, t + 1);
            tr_mark(5);
        } else {
            m_dma<KS>(S, a, c, L, t + 2);
            tr_mark(2);
            m_mfma<KS>(S, c, L, t);
            tr_mark(3);
            // round t+1 (issued last tick, its loads the youngest memory
            // instructions of that tick) must be in LDS before the barrier:
            // younger than them are only this tick's two record stores and
            // its loads
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(Geo<KS>::kDmaW + 2) : "memory");
            tr_mark(4);
        }
        __syncthreads();
        tr_mark(0);
        if (L.stop || t + 1 > last) break;
    }
}

template <int KS, bool FUSED, bool LOCAL, bool PO>
__device__ __forceinline__ void x_loop(XState<KS>& X, const CoopArgs& a, const RoundCtx& c, Lds<KS, PO>& L) {
    const int last = c.nr + 1;
    for (int t = 0;; t += 2) {
        if (x_tick<KS, FUSED, LOCAL, 0, PO>(X, a, c, L, t)) L.stop = 1;
        __syncthreads();
        tr_mark(0);
        if (L.stop || t + 1 > last) break;
        if (x_tick<KS, FUSED, LOCAL, 1, PO>(X, a, c, L, t + 1)) L.stop = 1;
        __syncthreads();
        tr_mark(0);
        if (L.stop || t + 2 > last) break;
    }
}

// Start of the call, run by the first exchange wave while the MFMA waves
// load their weights and the first two rounds.  The workspace header was
// updated by k_hdr, launched just before this kernel on the same stream, so
// it already holds this call's epoch and says whether the record area is to
// be cleared.  The member clears its share of its group's record area (if
// so) and counts itself in on the group's arrival word, and the group
// starts once all G of its members have arrived: no record is written
// before the group's area is clean, and no workgroup waits for one outside
// its own group (there is no grid-wide count, so one group's members being
// held back by other work does not stall the others).  Placement: with NG a
// multiple of 8, the members of group g are the workgroups b = g (mod 8),
// which the dispatcher places on XCD b % 8 (checked against the XCC id
// register); a group whose members all sit on that XCD keeps its records in
// the XCD's L2.  The wait is bounded (about two seconds): a member that is
// not resident in time makes the call give up (error flag, reported by
// hc_workspace_status).  The count carries data only when the members
// cleared records: then the zeros are released before it and acquired after
// it.  Otherwise it is relaxed, which spares every member an L2 write-back
// and each poll an L2 invalidation.  Result in *mode: 1 local, 0 not, -1
// gave up.
__device__ __forceinline__ void start_protocol(const CoopArgs& a, const RoundCtx& c, int* mode) {
    const bool cleared = __hip_atomic_load(&a.hdr->clear, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
    if (cleared) {
        // this member's part of group g's records (a group's records are
        // contiguous: [g][slot][member][record])
        const int64_t nchunks = a.part_bytes / 16;
        const int64_t gchunks = nchunks / a.NG;
        const int64_t per = (gchunks + a.G - 1) / a.G;
        const int64_t gend = (int64_t)(c.g + 1) * gchunks;
        const int64_t lo = (int64_t)c.g * gchunks + per * c.q, hi = lo + per < gend ? lo + per : gend;
        for (int64_t i = lo + c.l; i < hi; i += 64) a.part[i] = u32x4{0u, 0u, 0u, 0u};
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    }
    if (c.l == 0) {
        const uint32_t xcc = __builtin_amdgcn_s_getreg((20) | (0 << 6) | (15 << 11)) & 0xFu;
        const uint32_t add = 1u + (xcc != (blockIdx.x & 7u) ? 0x10000u : 0u);
        uint32_t* gw = &a.hdr->garr[c.g];
        __hip_atomic_fetch_add(gw, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        bool ok = true;
        uint32_t v;
        while (((v = __hip_atomic_load(gw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) & 0xFFFFu) < (uint32_t)a.G) {
            if (__builtin_amdgcn_s_memrealtime() - t0 > 200000000ull ||
                __hip_atomic_load(&a.hdr->err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
                give_up(a);
                ok = false;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        if (cleared) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        const bool local = a.NG % 8 == 0 && (v >> 16) == 0u;
        *mode = ok ? (local ? 1 : 0) : -1;
    }
    tr_stamp(1, 64 * kMW);
}

template <int KS, bool FUSED, bool PO = false>
__global__ __launch_bounds__(kThreads, 1) void k_spec(CoopArgs a) {
    __shared__ __attribute__((aligned(16))) Lds<KS, PO> L;
    __shared__ int local_mode;
    tr_stamp(0);
    RoundCtx c;
    c.g = blockIdx.x % a.NG;
    c.q = blockIdx.x / a.NG;
    c.w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    c.l = threadIdx.x & 63;
    c.row = c.l & 15;
    c.grp = c.l >> 4;
    c.tt = 0;
    c.kg = 0;
    c.nown = c.q < kT ? (kT - 1 - c.q) / a.G + 1 : 0;
    c.epoch = epoch_of(a.call);
    c.rsrc = __builtin_amdgcn_make_buffer_rsrc(a.part, 0, a.part_bytes, kBufDword3);
    c.nr = (int)((a.ntiles - c.g + a.NG - 1) / a.NG);
    c.s0 = FUSED ? a.scale[0] : 0.0f;
    c.bpre = FUSED ? base_of_lane(a.base, (threadIdx.x & 63) >> 4) : 0.0f;
    // a group with no token tile: all its members leave (none waits on them)
    if (c.g >= a.ntiles) return;
    if (threadIdx.x == 0) {
        L.stop = 0;
        L.acnt = 0u;
    }
    __syncthreads();
    if (c.w < kMW) {
        MState<KS, PO> S;
        m_dma_offsets<KS, PO>(S, a, c);
        const PubMap M = pub_map(srec_of);
        m_dma<KS, PO>(S, a, c, L, 0);
        m_dma<KS, PO>(S, a, c, L, 1);
        m_weights<KS, PO>(S, a, c);
        // round 0 landed (older than round 1 and the weight loads, which
        // have landed too by now)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(Geo<KS, PO>::kDmaW) : "memory");
        if constexpr (PO) {
            // round 0 into R' before the first tick
            m_arrive(&L.acnt);
            const bool bad = m_wait(a, &L.acnt, 4u);
            if (!bad) m_post<KS>(a, c, L, 0);
            else L.stop = 1;
        }
        __syncthreads();
        const int mode = local_mode;
        if (mode < 0) {
            // no load may still be writing this workgroup's LDS when it ends
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            return;
        }
        tr_start();
        tr_stamp(2);
        if (mode) m_loop<KS, FUSED, true, PO>(S, M, a, c, L);
        else m_loop<KS, FUSED, false, PO>(S, M, a, c, L);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
        if (c.w == kMW) start_protocol(a, c, &local_mode);
        XState<KS> X;
        x_offsets<KS>(X, a, c, c.w - kMW);
        __syncthreads();
        const int mode = local_mode;
        if (mode < 0) return;
        tr_start();
        if (mode) x_loop<KS, FUSED, true, PO>(X, a, c, L);
        else x_loop<KS, FUSED, false, PO>(X, a, c, L);
    }
    tr_finish(c.nr + 2);
}


}  // namespace spec

// The phase tables of the last wave-specialised launches (HC_PHASE_TRACE
// builds): up to count words of [workgroup][wave][phase 0..5, ticks] (1,024
// workgroups), then [workgroup][4 timestamps]; returns the words copied, or
// -1 without tracing or on a copy failure.
int phase_trace_copy(uint64_t* out, size_t count) {
#ifdef HC_PHASE_TRACE
    const size_t nt = (size_t)spec::kTrMaxBlocks * spec::kTrWords, ns = (size_t)spec::kTrMaxBlocks * 4;
    const size_t n1 = count < nt ? count : nt;
    const size_t n2 = count > nt ? (count - nt < ns ? count - nt : ns) : 0;
    if (hipMemcpyFromSymbol(out, HIP_SYMBOL(spec::kTrace), n1 * sizeof(uint64_t), 0, hipMemcpyDeviceToHost) !=
        hipSuccess)
        return -1;
    if (n2 && hipMemcpyFromSymbol(out + nt, HIP_SYMBOL(spec::kTraceTs), n2 * sizeof(uint64_t), 0,
                                  hipMemcpyDeviceToHost) != hipSuccess)
        return -1;
    return (int)(n1 + n2);
#else
    (void)out;
    (void)count;
    return -1;
#endif
}

namespace spec {

// ============================================== two-pass path (short runs)
// For a call of few tokens the persistent kernel's fixed costs (the start-up
// count, filling and draining its three-round pipeline, the exchange waits)
// dominate.  There the same arithmetic runs as two ordinary launches with no
// waits between workgroups:
//
//  * k_part: the MFMA waves' loop of k_spec on its own (same weight slices
//    and pieces, same direct-to-LDS residual ring, same products, same order
//    of the four stream partials).  Member q of tile group g writes the 26
//    partial sums of each token of its rounds as 9 records of 16 bytes
//    (3 floats and a zero word) to the workspace, at
//    [token][member][chunk].  A zero word never equals a tag of the
//    persistent kernels (their epochs start at 1), so a workspace that both
//    paths use stays valid for either.
//  * k_fin: one wave per token adds the members' records in the exchange
//    order of k_spec (lane e + 16 g holds chunk e of members 4 s + g, summed
//    over s in order, then across the lane groups by the same two swaps),
//    forms the mixes, pre and the split + Sinkhorn with the shared per-token
//    code, and the block's four waves then form h from a second read of the
//    residual (bitwise hc_pre's result for that pre).
//
// Mixes, pre, post, comb and h are therefore bitwise those of k_spec for the
// same token, whichever path a call takes.

constexpr int kFinTok = 4;      // tokens per k_fin block (one reducing wave each)

// Records of round r from the four MFMA waves' partials, to the two-pass
// record area (two store instructions per lane, always, as m_publish: the
// wait count of the loop depends on it).  Rounds past the group's end store
// nothing.
template <int KS>
__device__ __forceinline__ void p_publish(const CoopArgs& a, const RoundCtx& c, Lds<KS>& L, const PubMap& M,
                                          int r) {
    const int tid = threadIdx.x;
    const bool live = r >= 0 && r < c.nr;
    const int64_t tok0 = live ? tile_of(c, a, r) * kT : 0;
    int64_t valid = live ? a.n - tok0 : 0;
    valid = valid < 0 ? 0 : (valid > kT ? kT : valid);
    const int64_t tok_bytes = (int64_t)a.GP * kChunks * 16;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<char*>(a.part) + tok0 * tok_bytes, 0, (int)(valid * tok_bytes), kBufDword3);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int idx = p * (kMW * 64) + tid;
        const int tk = idx / kChunks, ch = idx - tk * kChunks;
        const u32x4 v = pub_value<KS>(L, r & 1, M, p);
        const int off = idx < kRecMember ? ((tk * a.GP + c.q) * kChunks + ch) * 16 : kOOB;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((__vector_size__(16))) int, v), rs,
                                               off, 0, 0);
    }
}

// Token and chunk of record id of a member's round in the two-pass record
// order (token-major).
__device__ __forceinline__ void prec_of(int id, int& tk, int& ch) {
    tk = id / kChunks;
    ch = id - tk * kChunks;
}

// Pass 1: workgroup b is member b % G of tile group b / G (tiles g, g + NG,
// ...).  Four waves, one per stream, as the MFMA waves of k_spec; tick t
// publishes round t-1, issues round t+2 and multiplies round t.
template <int KS>
__global__ __launch_bounds__(kMW * 64, 1) void k_part(CoopArgs a) {
    __shared__ __attribute__((aligned(16))) Lds<KS> L;
    RoundCtx c;
    c.q = blockIdx.x % a.G;
    c.g = blockIdx.x / a.G;
    c.w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    c.l = threadIdx.x & 63;
    c.row = c.l & 15;
    c.grp = c.l >> 4;
    c.tt = 0;
    c.kg = 0;
    c.nown = 0;
    c.epoch = 0;
    c.nr = (int)((a.ntiles - c.g + a.NG - 1) / a.NG);
    c.s0 = 0.0f;
    c.bpre = 0.0f;
    MState<KS> S;
    m_dma_offsets<KS>(S, a, c);
    const PubMap M = pub_map(prec_of);
    // rounds past the group's last are neither loaded nor multiplied (a
    // call of a few tokens has one round per group); the first rounds'
    // loads go out before the weights are fetched, so that both round trips
    // overlap; each wait below still covers the loads of every round used
    m_dma<KS>(S, a, c, L, 0);
    if (1 < c.nr) m_dma<KS>(S, a, c, L, 1);
    m_weights<KS>(S, a, c);
    // the rounds' loads are older than the weight loads, which have landed
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int t = 0;; ++t) {
        p_publish<KS>(a, c, L, M, t - 1);
        if (t + 2 < c.nr) {
            m_dma<KS>(S, a, c, L, t + 2);
            m_mfma<KS>(S, c, L, t);
            // round t+1 in LDS: younger than its loads are only this tick's
            // two record stores and the loads of round t+2
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(Geo<KS>::kDmaW + 2) : "memory");
        } else {
            if (t < c.nr) m_mfma<KS>(S, c, L, t);
            // younger than round t+1's loads (if any) are only this tick's
            // two record stores
            asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
        }
        __syncthreads();
        if (t >= c.nr) break;          // tick nr published the last round
    }
    // no load may still be writing this workgroup's LDS when it ends
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Weight packing (hc_pack_weights): block q, wave w forms member q's
// pieces of stream w with the projection's own conversion and stores the registers
// as they are, so a packed call's weights are bitwise an unpacked call's.
template <int KS>
__global__ __launch_bounds__(kMW * 64) void k_pack(CoopArgs a, u32x4* out) {
    RoundCtx c;
    c.q = blockIdx.x;
    c.g = 0;
    c.w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    c.l = threadIdx.x & 63;
    c.row = c.l & 15;
    c.grp = c.l >> 4;
    MState<KS> S;
    m_split_weights<KS>(S, a, c);
#pragma unroll
    for (int st = 0; st < KS; ++st)
#pragma unroll
        for (int ct = 0; ct < kTiles; ++ct)
            out[packed_index<KS>(c.q, c.w, st, ct, c.l)] = __builtin_bit_cast(u32x4, S.w[st][ct]);
}

// Pass 2: a group of blocks per 4 tokens.  With splits > 1 column parts
// (short calls, where the grid needs filling) the group has splits + 1
// blocks: part sp < splits covers column part sp of h, and part splits runs
// the split + Sinkhorn and writes the mixes, so the Sinkhorn's long
// dependent chain runs beside h rather than after it.  With one column part
// the group is one block that forms h and then runs the split + Sinkhorn
// (a separate block would only repeat the reduction).  In every block wave
// w reduces token 4 * group + w, and each thread issues the residual loads
// of its first h chunk before the reduction (they do not depend on it).
template <bool FUSED>
__global__ __launch_bounds__(256) void k_fin(CoopArgs a, int splits) {
    __shared__ float sums[kFinTok][kChunks][4];
    __shared__ __attribute__((aligned(16))) float mixL[kFinTok][kMix];
    __shared__ __attribute__((aligned(16))) float preL[kFinTok][4];
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63, e = l & 15, g = l >> 4;
    const bool sep = FUSED && splits > 1;         // a block of its own for the split + Sinkhorn
    const int parts = sep ? splits + 1 : 1;
    const int64_t tg = blockIdx.x / parts;
    const int sp = blockIdx.x - (int)(tg * parts);
    const bool sk_only = sep && sp == splits;     // this block runs only the split + Sinkhorn
    const bool coef = !sep || sk_only;            // this block writes the mixes and the split
    const int64_t t = tg * kFinTok + w;
    const bool tv = t < a.n;

    // h chunks of this block: item i is token i / cs of the block, chunk
    // sp * cs + i % cs of d / 8
    const int d8 = a.d / 8;
    const int cs = d8 / splits;
    const int64_t t0 = tg * kFinTok;
    const int64_t nt = a.n - t0 < kFinTok ? a.n - t0 : kFinTok;
    const int items = FUSED && !sk_only ? (int)nt * cs : 0;
    const u32x4* R = reinterpret_cast<const u32x4*>(a.R);
    int i = threadIdx.x;
    int tk = 0;
    int64_t row = 0, hrow = 0;
    u32x4 r0, r1, r2, r3;
    auto fetch = [&]() {
        tk = i / cs;
        const int c8 = sp * cs + (i - tk * cs);
        row = (t0 + tk) * kHC * (int64_t)d8 + c8;
        hrow = (t0 + tk) * d8 + c8;
        r0 = __builtin_nontemporal_load(R + row);
        r1 = __builtin_nontemporal_load(R + row + d8);
        r2 = __builtin_nontemporal_load(R + row + 2 * (int64_t)d8);
        r3 = __builtin_nontemporal_load(R + row + 3 * (int64_t)d8);
    };
    if (i < items) fetch();

    // member sums of token t's records in the exchange order of k_spec
    const int64_t tok_bytes = (int64_t)a.GP * kChunks * 16;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<char*>(a.part) + (tv ? t : 0) * tok_bytes, 0, tv ? (int)tok_bytes : 0, kBufDword3);
    u32x4 v[kXL];
#pragma unroll
    for (int s = 0; s < kXL; ++s) {
        const int m = 4 * s + g;
        const int off = (e < kChunks && m < a.G) ? (m * kChunks + e) * 16 : kOOB;
        v[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
    }
    const float x0 = member_sum(v, 0), x1 = member_sum(v, 1), x2 = member_sum(v, 2);
    if (l < kChunks) {
        sums[w][l][0] = x0;
        sums[w][l][1] = x1;
        sums[w][l][2] = x2;
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");     // the wave reads back its own LDS writes
    {
        const int f = l < kMix ? l : 0;
        int ch, sl;
        field_pos(f, ch, sl);
        const float m = mix_value(sums[w][ch][sl], mix_scale(sums[w][1][1], sums[w][1][2], a.K, a.norm_eps));
        if (l < kMix) mixL[w][l] = m;
        if (a.mixes && coef && tv && l < kMix) a.mixes[t * kMix + l] = m;
    }
    if (!FUSED) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    const float s0 = a.scale[0];
    // the split + Sinkhorn of token t (all four 16-lane rows compute it;
    // row 0 writes)
    auto split = [&]() {
        float p, q, cc;
        split_sinkhorn16(&mixL[w][0], s0, a.scale[1], a.scale[2], a.base, a.iters, a.eps, p, q, cc);
        if (tv && l < 16) {
            a.comb[t * (kHC * kHC) + e] = cc;
            if (e < kHC) {
                a.post[t * kHC + e] = q;
                if (a.pre) a.pre[t * kHC + e] = p;
            }
        }
    };
    if (sk_only) {
        split();
        return;
    }
    if (l < kHC) preL[w][l] = pre_gate(mixL[w][l], s0, a.base[l], a.eps);
    __syncthreads();

    // h of this block's tokens, column part sp
    u32x4* h = reinterpret_cast<u32x4*>(a.h);
    while (i < items) {
        const u32x4 out = pre_chunk8(*reinterpret_cast<const f32x4*>(&preL[tk][0]), r0, r1, r2, r3);
        const int64_t hr = hrow;
        i += 256;
        if (i < items) fetch();
        __builtin_nontemporal_store(out, h + hr);
    }
    if (coef) split();
}

}  // namespace spec

// Header update alone, launched before every call of the wave-specialised
// kernel.  Kernel order on the stream makes the update visible to all of
// k_spec's workgroups before any starts, with no grid-wide handshake inside
// k_spec (a wait on workgroup 0 costs every workgroup the slowest start).
// A replayed graph repeats the call number and so the epoch; the update then
// orders the record area cleared, which k_spec's workgroups do in parallel.
__global__ void k_hdr(WsHeader* hdr, int64_t nchunks, uint64_t call, int ngroups) {
    if (threadIdx.x == 0) header_update(hdr, call, nchunks, ngroups);
}

// Header update and record-area clearing before a call of the cooperative
// kernel of narrow or wide streams (before the wave-specialised kernel,
// k_hdr updates the header and the kernel's workgroups clear the record
// area themselves).
__global__ __launch_bounds__(1024) void k_init(WsHeader* hdr, u32x4* part, int64_t nchunks, uint64_t call) {
    __shared__ int clear;
    if (threadIdx.x == 0) clear = header_update(hdr, call, nchunks, 0);
    __syncthreads();
    if (clear)
        for (int64_t i = threadIdx.x; i < nchunks; i += blockDim.x) part[i] = u32x4{0u, 0u, 0u, 0u};
}

// ------------------------------------------------------------------ host
// Calls are numbered process-wide; the number sets the epoch in the record
// tags, so no per-call initialisation launch is needed.
static std::atomic<uint64_t> g_calls{0};

// Bound of an exchange wait: 2 s of the 100 MHz s_memrealtime counter.
constexpr uint64_t kSpin = 200000000ull;

// Diagnostics: the next t_force persistent-kernel launches of this thread
// take every exchange record for stale and bound their waits to zero time,
// so their waits give up at once (hc_debug_force_timeout).
static thread_local int t_force = 0;
void set_force_timeout(int calls) { t_force = calls; }

// Persistent-kernel launches of one device in this process run one after
// another: a launch on another stream than the previous one first waits
// for the previous one (an event), so two persistent grids never share the
// compute units, each needing all of its group's workgroups resident.
struct Gate {
    std::mutex mu;
    hipEvent_t ev = nullptr;
    hipStream_t last = nullptr;
    bool used = false;
};
static Gate g_gate[64];

int ws_status(const void* ws, bool clear) {
    WsHeader h;
    if (hipMemcpy(&h, ws, sizeof h, hipMemcpyDeviceToHost) != hipSuccess) return -1;
    if (h.magic != kMagic || h.failed == 0u) return 0;
    if (clear) {
        const uint32_t z = 0u;
        if (hipMemcpy(static_cast<char*>(const_cast<void*>(ws)) + offsetof(WsHeader, failed), &z, sizeof z,
                      hipMemcpyHostToDevice) != hipSuccess)
            return -1;
    }
    return 1;
}

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

// Calls of at most this many tokens (at widths the wave-specialised kernel
// serves) take the two-pass path.
#ifndef HC_TWO_PASS_MAX_N
#define HC_TWO_PASS_MAX_N 2048
#endif
constexpr int64_t kTwoPassMaxN = HC_TWO_PASS_MAX_N;

// Wave-specialised kernel: groups of 8..32 members.
static bool spec_width(int G) { return G >= 8 && G <= 32; }

bool coop_plan(int64_t n, int d, CoopPlan& p) {
    const int KS = coop_ks(d);
    if (!KS) return false;
    p.KS = KS;
    p.G = d / (32 * KS);
    p.TM = kTT;
    p.ntiles = (n + kT - 1) / kT;
    const int cus = num_cus();
    int ng = cus / p.G;
    if (ng < 1) ng = 1;
    if (spec_width(p.G) && ng > kMaxGroups) ng = kMaxGroups;     // one header arrival word per group
    if (ng > p.ntiles) ng = (int)(p.ntiles > 0 ? p.ntiles : 1);
    p.NG = ng;
    p.gate = true;
    p.ws_part = 256;
    p.two_pass = spec_width(p.G) && n <= kTwoPassMaxN;
    p.splits = 1;
    if (p.two_pass) {
        // records [n][GP][9] of 16 bytes; nothing else in the workspace
        p.ws_mix = p.ws_part + (size_t)n * pow2_at_least(p.G) * kChunks * 16;
        p.ws_bytes = (p.ws_mix + 255) & ~(size_t)255;
        const int64_t blocks = (n + spec::kFinTok - 1) / spec::kFinTok;
        const int d8 = d / 8;
        while (blocks * p.splits < 2 * cus && p.splits < 8 && d8 % (2 * p.splits) == 0) p.splits *= 2;
        return true;
    }
    p.ws_mix = p.ws_part + (size_t)p.NG * kSlots * kChunks * kT * pow2_at_least(p.G) * 16;
    p.ws_bytes = p.ws_mix + (((size_t)n * kMix * sizeof(float) + 255) & ~(size_t)255);
    return true;
}

template <int KS, int PI, bool FUSED>
static int launch_t(const CoopPlan& p, CoopArgs& a, hipStream_t s) {
    void* args[] = {&a};
    hipError_t e = hipLaunchKernel((const void*)k_coop<KS, PI, FUSED>, dim3(p.G * p.NG), dim3(kThreads), args, 0, s);
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

static bool use_spec(const CoopPlan& p) { return spec_width(p.G); }

size_t packed_weights_bytes(int d) {
    const int KS = coop_ks(d);
    if (!KS || !spec_width(d / (32 * KS))) return 0;
    return (size_t)(d / (32 * KS)) * kHC * KS * kTiles * 64 * 16;
}

int launch_pack(const float* W, void* out, int d, hipStream_t s) {
    const int KS = coop_ks(d);
    CoopArgs a{};
    a.W = W;
    a.d = d;
    a.Wp = nullptr;
    const int G = d / (32 * KS);
    u32x4* o = static_cast<u32x4*>(out);
    switch (KS) {
        case 1: spec::k_pack<1><<<G, spec::kMW * 64, 0, s>>>(a, o); break;
        case 2: spec::k_pack<2><<<G, spec::kMW * 64, 0, s>>>(a, o); break;
        case 3: spec::k_pack<3><<<G, spec::kMW * 64, 0, s>>>(a, o); break;
        case 4: spec::k_pack<4><<<G, spec::kMW * 64, 0, s>>>(a, o); break;
        case 5: spec::k_pack<5><<<G, spec::kMW * 64, 0, s>>>(a, o); break;
        default: return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <int KS>
static int launch_two_pass(const CoopPlan& p, CoopArgs& a, bool fused, hipStream_t s) {
    spec::k_part<KS><<<p.G * p.NG, spec::kMW * 64, 0, s>>>(a);
    if (hipGetLastError() != hipSuccess) return -1;
    const int splits = fused ? p.splits : 1;
    const int64_t blocks = (a.n + spec::kFinTok - 1) / spec::kFinTok * (fused && splits > 1 ? splits + 1 : 1);
    if (fused) spec::k_fin<true><<<(unsigned)blocks, 256, 0, s>>>(a, splits);
    else spec::k_fin<false><<<(unsigned)blocks, 256, 0, s>>>(a, splits);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <int KS>
static int launch_spec(const CoopPlan& p, CoopArgs& a, bool fused, bool post, hipStream_t s) {
    void* args[] = {&a};
    const void* f = post    ? (const void*)spec::k_spec<KS, true, true>
                    : fused ? (const void*)spec::k_spec<KS, true>
                            : (const void*)spec::k_spec<KS, false>;
    hipError_t e = hipLaunchKernel(f, dim3(p.G * p.NG), dim3(kThreads), args, 0, s);
    return e == hipSuccess ? 0 : -1;
}

int launch_coop(const CoopPlan& p, const void* R, const float* W, const float* scale, const float* base,
                void* h, float* pre, float* post, float* comb, float* mixes, void* ws, int64_t n, int d,
                int iters, float eps, float norm_eps, bool fused, hipStream_t s, const PostIn* prev,
                const void* Wp) {
    char* wsb = static_cast<char*>(ws);
    // The sublayer boundary in one pass: the persistent kernel forms R' from
    // each round of R in LDS (k_spec, PO), so R is read once for hc_post,
    // the projection and h.
    const bool one_pass = prev && fused && !p.two_pass && use_spec(p);
    if (prev && !one_pass) {
        // hc_post, then the projection of its output.  (Applying hc_post to
        // each round inside k_part, while the residual is in LDS, was
        // slower: its exact-rounding work then runs on the few CUs of a
        // short call instead of the whole chip.)
        if (launch_post(prev->x, R, prev->post, prev->comb, prev->Rout, n, d, s)) return -1;
        return launch_coop(p, prev->Rout, W, scale, base, h, pre, post, comb, mixes, ws, n, d, iters, eps,
                           norm_eps, fused, s, nullptr, Wp);
    }
    CoopArgs a{};
    a.Wp = static_cast<const u32x4*>(Wp);
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
    a.call = g_calls.fetch_add(1, std::memory_order_relaxed) + 1;
    a.spin = kSpin;
    a.force_tag = 0u;
    if (one_pass) {
        a.x = static_cast<const uint16_t*>(prev->x);
        a.postp = prev->post;
        a.combp = prev->comb;
        a.Rout = static_cast<uint16_t*>(prev->Rout);
    }
    int rc = -1;
    if (p.two_pass) {
        // mixes go only where the caller asked for them; pass 2 does the split
        a.mixes = mixes;
        switch (p.KS) {
            case 1: return launch_two_pass<1>(p, a, fused, s);
            case 2: return launch_two_pass<2>(p, a, fused, s);
            case 3: return launch_two_pass<3>(p, a, fused, s);
            case 4: return launch_two_pass<4>(p, a, fused, s);
            case 5: return launch_two_pass<5>(p, a, fused, s);
        }
        return -1;
    }
    // the persistent kernels: waits between workgroups
    if (t_force > 0) {
        --t_force;
        a.spin = 0;
        a.force_tag = 0x80000000u;
    }
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) return -1;
    const bool capturing = cs != hipStreamCaptureStatusNone;
    Gate* gate = nullptr;
    std::unique_lock<std::mutex> lk;
    if (p.gate && !capturing) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
        gate = &g_gate[dev];
        lk = std::unique_lock<std::mutex>(gate->mu);
        if (!gate->ev && hipEventCreateWithFlags(&gate->ev, hipEventDisableTiming) != hipSuccess) {
            gate->ev = nullptr;
            return -1;
        }
        if (gate->used && gate->last != s && hipStreamWaitEvent(s, gate->ev, 0) != hipSuccess) return -1;
    }
    if (!use_spec(p)) {
        k_init<<<1, 1024, 0, s>>>(a.hdr, a.part, (int64_t)(a.part_bytes / 16), a.call);
        if (hipGetLastError() != hipSuccess) return -1;
    }
    if (use_spec(p)) {
        // the header update is a launch of its own: k_spec's workgroups read
        // it without a grid-wide handshake, and a replayed graph repeats it
        k_hdr<<<1, 64, 0, s>>>(a.hdr, (int64_t)(a.part_bytes / 16), a.call, a.NG);
        if (hipGetLastError() != hipSuccess) return -1;
        switch (p.KS) {
            case 1: rc = launch_spec<1>(p, a, fused, one_pass, s); break;
            case 2: rc = launch_spec<2>(p, a, fused, one_pass, s); break;
            case 3: rc = launch_spec<3>(p, a, fused, one_pass, s); break;
            case 4: rc = launch_spec<4>(p, a, fused, one_pass, s); break;
            case 5: rc = launch_spec<5>(p, a, fused, one_pass, s); break;
        }
    } else switch (p.KS) {
        case 1: rc = launch_ks<1>(p, a, fused, s); break;
        case 2: rc = launch_ks<2>(p, a, fused, s); break;
        case 3: rc = launch_ks<3>(p, a, fused, s); break;
        case 4: rc = launch_ks<4>(p, a, fused, s); break;
        case 5: rc = launch_ks<5>(p, a, fused, s); break;
    }
    if (gate && !rc) {
        if (hipEventRecord(gate->ev, s) != hipSuccess) return -1;
        gate->last = s;
        gate->used = true;
    }
    if (rc || !fused) return rc;
    // post and comb (and pre when not written above): the split + Sinkhorn of
    // the mixes, in the same per-token code as hc_split_sinkhorn
    return launch_split(a.mixes, scale, base, nullptr, post, comb, n, iters, eps, s);
}

}  // namespace hc
