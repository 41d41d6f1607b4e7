// hc_device.hpp -- device helpers shared by the libhc kernels (gfx950 only).
//
// bf16 <-> float/double conversions, the correctly rounded double -> bf16
// conversion used for every bf16 output, cross-lane reductions inside a
// 16-lane row (DPP), and the per-token split + epsilon-Sinkhorn that the
// standalone and fused kernels share so that both give bitwise the same
// coefficients.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hc {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr int kHC = 4;                      // streams per token (hc_mult)
constexpr int kMix = (2 + kHC) * kHC;       // 24 mix numbers per token

// ---------------------------------------------------------------- bf16 bits
// A 32-bit word holds two bf16 values: element 0 in the low half.
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t bf16_rn(float f) {
    __bf16 b = (__bf16)f;
    return (uint32_t)__builtin_bit_cast(uint16_t, b);
}

// double -> bf16 bits, correctly rounded (nearest even), from a single
// conceptual rounding of y.  The fast path rounds y to float and then to
// bf16; that double rounding can only go wrong when the float lands exactly
// on a bf16 halfway point while y itself does not, in which case the float
// is nudged one float ulp towards y before the second rounding.
// Branch-free (selects only), so a wave computes it in a few instructions.
__device__ __forceinline__ uint32_t bf16_rn_f64(double y) {
    const float f = (float)y;
    const double back = (double)f;
    const uint32_t u = __float_as_uint(f);
    const bool nudge = ((u & 0xFFFFu) == 0x8000u) & (back != y);
    const uint32_t toward = (__builtin_fabs(y) > __builtin_fabs(back)) ? 1u : 0xFFFFFFFFu;
    return bf16_rn(__uint_as_float(u + (nudge ? toward : 0u)));
}

// Fast path of bf16_rn_f64: the float rounding of y gives the correctly
// rounded bf16 unless that float lands exactly on a bf16 halfway point.
// Returns the float and raises `mid` when it does; a wave in which any lane
// raised it redoes its item with bf16_rn_f64 (a few percent of items), so
// results are those of bf16_rn_f64 bit for bit.
__device__ __forceinline__ float f32_mid(double y, bool& mid) {
    const float f = (float)y;
    mid |= (__float_as_uint(f) & 0xFFFFu) == 0x8000u;
    return f;
}

// Pack two bf16 bit patterns into one word (element 0 low).
__device__ __forceinline__ uint32_t pack2(uint32_t lo, uint32_t hi) { return lo | (hi << 16); }

// Two floats to one word of bf16 bits, each rounded to nearest even (one
// v_cvt_pk_bf16_f32; the same rounding as bf16_rn on each): pack2(bf16_rn(lo),
// bf16_rn(hi)) in one instruction.
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rn(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v){lo, hi}, bf16x2v));
}

// h of one 16-byte chunk (8 consecutive features) from the four streams'
// chunks r0..r3 and the token's pre p ("Mix projection" page, Block.hc_pre):
// each output is the correctly rounded bf16 of sum_k p_k R_k, accumulated in
// double (every product is exact there) in the fixed order p0 R0 + p1 R1 +
// p2 R2 + p3 R3.  A wave redoes its chunks with bf16_rn_f64 when any lane
// hit a float halfway point, so the result does not depend on the path.
__device__ __forceinline__ u32x4 pre_chunk8(const f32x4 p, const u32x4 r0, const u32x4 r1, const u32x4 r2,
                                            const u32x4 r3) {
    const double p0 = p[0], p1 = p[1], p2 = p[2], p3 = p[3];
    // element e of word w (e = 0: low half): sum over the 4 streams
    auto sum = [&](int w, int e) {
        auto v = [&](uint32_t word) { return (double)(e ? bf_hi(word) : bf_lo(word)); };
        double y = p0 * v(r0[w]);
        y = __builtin_fma(p1, v(r1[w]), y);
        y = __builtin_fma(p2, v(r2[w]), y);
        return __builtin_fma(p3, v(r3[w]), y);
    };
    u32x4 out;
    float f[4][2];
    bool mid = false;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        f[w][0] = f32_mid(sum(w, 0), mid);
        f[w][1] = f32_mid(sum(w, 1), mid);
    }
    if (__builtin_amdgcn_ballot_w64(mid)) {
#pragma unroll
        for (int w = 0; w < 4; ++w) out[w] = pack2(bf16_rn_f64(sum(w, 0)), bf16_rn_f64(sum(w, 1)));
    } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) out[w] = pack2(bf16_rn(f[w][0]), bf16_rn(f[w][1]));
    }
    return out;
}

// hc_post of one 16-byte chunk (8 consecutive features) of one token
// ("Mix projection" page, Block.hc_post): out[k] holds the chunk of output
// stream k, each element the correctly rounded bf16 of post_k x +
// sum_j comb[j][k] R_j, accumulated in double (every product is exact
// there) in the fixed order post_k x, then j = 0..3.  q = post of the token,
// cb[j] = row j of its comb, xv = the chunk of x, r[j] = the chunk of R_j.
// Waves in which any lane hit a float halfway point redo their chunks with
// bf16_rn_f64, so the result does not depend on the path.
__device__ __forceinline__ void post_chunk8(const f32x4 q, const f32x4 (&cb)[kHC], const u32x4 xv,
                                            const u32x4 (&r)[kHC], u32x4 (&out)[kHC]) {
    auto sum = [&](int k, int w, int e) {
        auto v = [&](uint32_t word) { return (double)(e ? bf_hi(word) : bf_lo(word)); };
        double y = (double)q[k] * v(xv[w]);
#pragma unroll
        for (int j = 0; j < kHC; ++j) y = __builtin_fma((double)cb[j][k], v(r[j][w]), y);
        return y;
    };
    float f[kHC][4][2];
    bool mid = false;
#pragma unroll
    for (int k = 0; k < kHC; ++k)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            f[k][w][0] = f32_mid(sum(k, w, 0), mid);
            f[k][w][1] = f32_mid(sum(k, w, 1), mid);
        }
    if (__builtin_amdgcn_ballot_w64(mid)) {
#pragma unroll
        for (int k = 0; k < kHC; ++k)
#pragma unroll
            for (int w = 0; w < 4; ++w) out[k][w] = pack2(bf16_rn_f64(sum(k, w, 0)), bf16_rn_f64(sum(k, w, 1)));
    } else {
#pragma unroll
        for (int k = 0; k < kHC; ++k)
#pragma unroll
            for (int w = 0; w < 4; ++w) out[k][w] = pack2(bf16_rn(f[k][w][0]), bf16_rn(f[k][w][1]));
    }
}

// post_chunk8 with the work ordered by input word: for each 32-bit word w
// (two features) the eight outputs of the four streams, so that only that
// word's inputs are live as doubles.  NW words per stream (4: a 16-byte
// chunk, 2: half of one).  The same double sums, so the same bits (each
// output is bf16_rn_f64 of its sum whichever path a wave takes), for
// callers short of registers.
template <int NW>
__device__ __forceinline__ void post_words_lean(const f32x4 q, const f32x4 (&cb)[kHC], const uint32_t (&xv)[NW],
                                                const uint32_t (&r)[kHC][NW], uint32_t (&out)[kHC][NW]) {
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        auto sum = [&](int k, int e) {
            auto v = [&](uint32_t word) { return (double)(e ? bf_hi(word) : bf_lo(word)); };
            double y = (double)q[k] * v(xv[w]);
#pragma unroll
            for (int j = 0; j < kHC; ++j) y = __builtin_fma((double)cb[j][k], v(r[j][w]), y);
            return y;
        };
        float f[kHC][2];
        bool mid = false;
#pragma unroll
        for (int k = 0; k < kHC; ++k) {
            f[k][0] = f32_mid(sum(k, 0), mid);
            f[k][1] = f32_mid(sum(k, 1), mid);
        }
        if (__builtin_amdgcn_ballot_w64(mid)) {
#pragma unroll
            for (int k = 0; k < kHC; ++k) out[k][w] = pack2(bf16_rn_f64(sum(k, 0)), bf16_rn_f64(sum(k, 1)));
        } else {
#pragma unroll
            for (int k = 0; k < kHC; ++k) out[k][w] = bf16x2_rn(f[k][0], f[k][1]);
        }
    }
}

// ------------------------------------------------ 16-lane row reductions
// DPP controls (gfx9 encoding): quad_perm patterns and row_ror 4 / 8, all of
// which read a lane inside the same row, so no lane is out of bounds and
// the bound_ctrl setting only lets the compiler fold the move into the
// instruction that uses it.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
// Sum / max over the 4 lanes of a quad (lanes 4j..4j+3 of a 16-lane row).
__device__ __forceinline__ float quad_sum(float v) {
    v = v + dpp<0xB1>(v);
    return v + dpp<0x4E>(v);
}
__device__ __forceinline__ float quad_max(float v) {
    v = fmaxf(v, dpp<0xB1>(v));
    return fmaxf(v, dpp<0x4E>(v));
}
// Sum over lanes e, e+4, e+8, e+12 (mod 16) of a 16-lane row.
__device__ __forceinline__ float col4_sum(float v) {
    v = v + dpp<0x128>(v);
    return v + dpp<0x124>(v);
}

// Logistic function in float: hardware exp2 and reciprocal (each within
// about one ulp), so the gate costs a handful of instructions.  Every
// kernel that forms a gate calls this one function, so all entry points
// agree bit for bit.
__device__ __forceinline__ float sigmoidf_(float z) {
    const float e = __builtin_amdgcn_exp2f(-z * 1.4426950408889634f);
    return __builtin_amdgcn_rcpf(1.0f + e);
}

// The read and write gates of the split, shared by every kernel that forms
// them so that all entry points agree bit for bit.
__device__ __forceinline__ float pre_gate(float m, float s0, float b, float eps) {
    return sigmoidf_(m * s0 + b) + eps;
}
__device__ __forceinline__ float post_gate(float m, float s1, float b) { return 2.0f * sigmoidf_(m * s1 + b); }

// RMS normaliser of the mix formula: 1 / sqrt(sum_sq / K + norm_eps), with
// the hardware reciprocal square root (about one ulp).  One function for
// every kernel, so the mixes and pre of all entry points agree bit for bit.
__device__ __forceinline__ float rms_scale(float sum_sq, float K, float norm_eps) {
    return __builtin_amdgcn_rsqf(sum_sq * __builtin_amdgcn_rcpf(K) + norm_eps);
}

// Overflow-safe normaliser.  A bf16 stream can hold values up to 2^128,
// whose squares overflow fp32 long before the stream itself overflows, so
// every kernel also forms sb, the sum of squares of the values scaled by
// 2^-72 (scaled_x2 below).  While the plain sum ss is finite the mix is
// dot * rms_scale(ss) exactly as before; once ss has overflowed,
// 1/sqrt(ss/K) = 2^-72/sqrt(sb/K) (norm_eps is then far below one ulp), and
// the 2^-72 is applied to the dot product first so that no intermediate
// leaves the normal range.  A mix is mix_value(dot, mix_scale(ss, sb, ...)).
struct MixScale {
    float mul, rs;
};
__device__ __forceinline__ MixScale mix_scale(float ss, float sb, float K, float norm_eps) {
    const bool big = !(ss <= 3.40282347e38f);          // overflowed (or not a number)
    MixScale m;
    m.mul = big ? 0x1p-72f : 1.0f;
    m.rs = big ? __builtin_amdgcn_rsqf(sb * __builtin_amdgcn_rcpf(K)) : rms_scale(ss, K, norm_eps);
    return m;
}
__device__ __forceinline__ float mix_value(float dot, MixScale s) { return (dot * s.mul) * s.rs; }

// Two packed bf16 values times 2^-72, for the scaled sum of squares: the
// magnitude bits minus 72 << 7 in each half, saturating at zero, so a value
// below 2^-55 becomes zero or subnormal (its square is then far below one
// ulp of a sum that has overflowed fp32 unscaled).  The sign is dropped.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t scaled_x2(uint32_t w) {
    const u16x2 m = __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_sub_sat(m, (u16x2){0x2400, 0x2400}));
}

// ------------------------------------------------- split + epsilon-Sinkhorn
// One token per 16-lane row; lane e = (lane & 15) holds comb entry
// (j, k) = (e / 4, e % 4).  m points at the token's 24 mixes (any memory
// the lane can read).  Follows the hc_split_sinkhorn listing of the
// "Reading weights" page: pre = sigmoid(s0*m_j + b_j) + eps,
// post = 2 sigmoid(s1*m_{4+j} + b_{4+j}), logits s2*m_{8+4j+k} + b_{8+4j+k};
// row softmax + eps, column normalisation, then (iters - 1) x (row, column)
// normalisations, each dividing by (sum + eps).
// Outputs: pre_o / post_o valid in lanes e < 4 (stream e); comb_o in all.
__device__ __forceinline__ void split_sinkhorn16(const float* m, float s0, float s1, float s2,
                                                 const float* __restrict__ base, int iters,
                                                 float eps, float& pre_o, float& post_o,
                                                 float& comb_o) {
    const int e = threadIdx.x & 15;
    const int j4 = e & 3;
    pre_o = pre_gate(m[j4], s0, base[j4], eps);
    post_o = post_gate(m[kHC + j4], s1, base[kHC + j4]);
    float c = m[2 * kHC + e] * s2 + base[2 * kHC + e];
    // row softmax (max subtracted for range only), then + eps
    float mx = quad_max(c);
    float ex = expf(c - mx);
    float rs = quad_sum(ex);
    c = ex / rs + eps;
    // column normalisation
    float cs = col4_sum(c);
    c = c * __builtin_amdgcn_rcpf(cs + eps);
    for (int it = 1; it < iters; ++it) {
        rs = quad_sum(c);
        c = c * __builtin_amdgcn_rcpf(rs + eps);
        cs = col4_sum(c);
        c = c * __builtin_amdgcn_rcpf(cs + eps);
    }
    comb_o = c;
}

}  // namespace hc
