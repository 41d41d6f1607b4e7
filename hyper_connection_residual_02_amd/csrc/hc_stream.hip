// hc_stream.hip -- the streaming kernels: hc_pre, hc_post and the
// chained-stack stand-in sublayer (diagonal scale).
//
// All three are HBM-bound elementwise passes.  Each thread owns one 16-byte
// chunk (8 consecutive features) of one token and touches every stream of
// that chunk, so every global access is a coalesced 16-byte vector access.
// When a wave's 64 chunks all belong to one token (d a multiple of 512) the
// token's coefficients are wave-uniform and come through scalar loads.
//
// Numerics: each output is the correctly rounded bf16 of its defining sum.
// A product of an fp32 coefficient and a bf16 value has at most 32
// significant bits, so it is exact in double; the sum of the (at most 5)
// products is accumulated in double and rounded once (bf16_rn_f64, with its
// float fast path taken per wave).

#include "hc_device.hpp"
#include "hc_launch.hpp"

namespace hc {

// Work item = (token t, 16-byte chunk c8 of d).  A wave of 64 items covers
// 512 features of one token when d8 % 64 == 0 ("uniform" mode); otherwise
// items are numbered flat and each lane loads its own coefficients.
struct ItemMap {
    uint32_t d8;       // chunks per token row
    uint64_t items;    // n * d8
};

__device__ __forceinline__ void item_of(uint64_t it, uint32_t d8, uint64_t& t, uint32_t& c8) {
    if (it < 0xFFFFFFFFull) {
        uint32_t i32 = (uint32_t)it;
        t = i32 / d8;
        c8 = i32 - (uint32_t)t * d8;
    } else {
        t = it / d8;
        c8 = (uint32_t)(it - t * d8);
    }
}

// ------------------------------------------------------------------ hc_pre
// "Mix projection" page, Block.hc_pre: h_c = bf16(sum_k pre_k R_{k,c}).
template <bool UNIFORM>
__global__ __launch_bounds__(256) void k_pre(const u32x4* __restrict__ R, const float* __restrict__ pre,
                                             u32x4* __restrict__ h, ItemMap map) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t it = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; it < map.items; it += stride) {
        uint64_t t;
        uint32_t c8;
        item_of(it, map.d8, t, c8);
        if (UNIFORM) t = __builtin_amdgcn_readfirstlane((uint32_t)t) | ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(t >> 32)) << 32);
        const f32x4 p = *reinterpret_cast<const f32x4*>(pre + t * kHC);
        const uint64_t row = t * kHC * (uint64_t)map.d8 + c8;
        const u32x4 r0 = __builtin_nontemporal_load(R + row);
        const u32x4 r1 = __builtin_nontemporal_load(R + row + map.d8);
        const u32x4 r2 = __builtin_nontemporal_load(R + row + 2 * (uint64_t)map.d8);
        const u32x4 r3 = __builtin_nontemporal_load(R + row + 3 * (uint64_t)map.d8);
        const u32x4 out = pre_chunk8(p, r0, r1, r2, r3);
        __builtin_nontemporal_store(out, h + t * map.d8 + c8);
    }
}

// ----------------------------------------------------------------- hc_post
// "Mix projection" page, Block.hc_post:
//   R'_{k,c} = bf16(post_k x_c + sum_j comb[j][k] R_{j,c}).
template <bool UNIFORM>
__global__ __launch_bounds__(256) void k_post(const u32x4* __restrict__ x, const u32x4* R,
                                              const float* __restrict__ post, const float* __restrict__ comb,
                                              u32x4* Rout, ItemMap map) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    uint64_t it = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (it >= map.items) return;
    struct Item {
        uint64_t t;
        uint32_t c8;
        u32x4 xv, r[kHC];
    };
    // the next item's loads are in flight while this item is computed; past
    // the end the last item is loaded again (no branch around the loads, so
    // the wait for the current item counts only its own loads)
    auto fetch = [&](uint64_t i, Item& I) {
        item_of(i < map.items ? i : map.items - 1, map.d8, I.t, I.c8);
        if (UNIFORM)
            I.t = __builtin_amdgcn_readfirstlane((uint32_t)I.t) |
                  ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(I.t >> 32)) << 32);
        const uint64_t row = I.t * kHC * (uint64_t)map.d8 + I.c8;
        I.xv = __builtin_nontemporal_load(x + I.t * map.d8 + I.c8);
#pragma unroll
        for (int j = 0; j < kHC; ++j) I.r[j] = __builtin_nontemporal_load(R + row + j * (uint64_t)map.d8);
    };
    Item cur, nxt;
    fetch(it, cur);
    for (; it < map.items; it += stride) {
        fetch(it + stride, nxt);
        const uint64_t t = cur.t;
        const f32x4 q = *reinterpret_cast<const f32x4*>(post + t * kHC);
        f32x4 cb[kHC];
#pragma unroll
        for (int j = 0; j < kHC; ++j) cb[j] = *reinterpret_cast<const f32x4*>(comb + (t * kHC + j) * kHC);
        const uint64_t row = t * kHC * (uint64_t)map.d8 + cur.c8;
        u32x4 out[kHC];
        post_chunk8(q, cb, cur.xv, cur.r, out);
#pragma unroll
        for (int k = 0; k < kHC; ++k) __builtin_nontemporal_store(out[k], Rout + row + k * (uint64_t)map.d8);
        cur = nxt;
    }
}

// hc_post for short calls: items of 4 features (half a chunk; map.d8 holds
// the token row's 8-byte pieces), so that a call of a few tokens spreads
// over twice as many threads and each thread's chain of double sums is half
// as long.  post_words_lean<2> forms the same double sums and rounding, so
// the results are k_post's bit for bit.
template <bool UNIFORM>
__global__ __launch_bounds__(256) void k_post4(const u32x2* __restrict__ x, const u32x2* R,
                                               const float* __restrict__ post, const float* __restrict__ comb,
                                               u32x2* Rout, ItemMap map) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t it = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; it < map.items; it += stride) {
        uint64_t t;
        uint32_t c4;
        item_of(it, map.d8, t, c4);
        if (UNIFORM)
            t = __builtin_amdgcn_readfirstlane((uint32_t)t) |
                ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(t >> 32)) << 32);
        const uint64_t row = t * kHC * (uint64_t)map.d8 + c4;
        const u32x2 xp = __builtin_nontemporal_load(x + t * map.d8 + c4);
        uint32_t xw[2] = {xp[0], xp[1]};
        uint32_t rw[kHC][2];
#pragma unroll
        for (int j = 0; j < kHC; ++j) {
            const u32x2 v = __builtin_nontemporal_load(R + row + j * (uint64_t)map.d8);
            rw[j][0] = v[0];
            rw[j][1] = v[1];
        }
        const f32x4 q = *reinterpret_cast<const f32x4*>(post + t * kHC);
        f32x4 cb[kHC];
#pragma unroll
        for (int j = 0; j < kHC; ++j) cb[j] = *reinterpret_cast<const f32x4*>(comb + (t * kHC + j) * kHC);
        uint32_t out[kHC][2];
        post_words_lean<2>(q, cb, xw, rw, out);
#pragma unroll
        for (int k = 0; k < kHC; ++k)
            __builtin_nontemporal_store(u32x2{out[k][0], out[k][1]}, Rout + row + k * (uint64_t)map.d8);
    }
}

// ----------------------------------------------------------- diag_scale
// x_c = bf16(h_c * D_c): the product of two bf16 values is exact in float.
__global__ __launch_bounds__(256) void k_diag(const u32x4* __restrict__ h, const u32x4* __restrict__ D,
                                              u32x4* __restrict__ x, ItemMap map) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t it = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; it < map.items; it += stride) {
        uint64_t t;
        uint32_t c8;
        item_of(it, map.d8, t, c8);
        const u32x4 hv = __builtin_nontemporal_load(h + t * map.d8 + c8);
        const u32x4 dv = D[c8];
        u32x4 out;
#pragma unroll
        for (int w = 0; w < 4; ++w)
            out[w] = pack2(bf16_rn(bf_lo(hv[w]) * bf_lo(dv[w])), bf16_rn(bf_hi(hv[w]) * bf_hi(dv[w])));
        __builtin_nontemporal_store(out, x + t * map.d8 + c8);
    }
}

// ------------------------------------------------------------- launchers
static int grid_for(uint64_t items, int per_cu_blocks) {
    uint64_t blocks = (items + 255) / 256;
    uint64_t cap = (uint64_t)num_cus() * per_cu_blocks;
    if (blocks > cap) blocks = cap;
    return (int)(blocks ? blocks : 1);
}

int launch_pre(const void* R, const float* pre, void* h, int64_t n, int d, hipStream_t s) {
    ItemMap m{(uint32_t)(d / 8), (uint64_t)n * (uint64_t)(d / 8)};
    const int g = grid_for(m.items, 8);
    if (m.d8 % 64 == 0)
        k_pre<true><<<g, 256, 0, s>>>((const u32x4*)R, pre, (u32x4*)h, m);
    else
        k_pre<false><<<g, 256, 0, s>>>((const u32x4*)R, pre, (u32x4*)h, m);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_post(const void* x, const void* R, const float* post, const float* comb, void* Rout,
                int64_t n, int d, hipStream_t s) {
    ItemMap m{(uint32_t)(d / 8), (uint64_t)n * (uint64_t)(d / 8)};
    if (m.items < 256ull * (uint64_t)num_cus()) {
        // fewer 16-byte items than one 256-thread workgroup per CU: half
        // items, one per thread
        ItemMap h{(uint32_t)(d / 4), (uint64_t)n * (uint64_t)(d / 4)};
        const int g = grid_for(h.items, 16);
        if (h.d8 % 64 == 0)
            k_post4<true><<<g, 256, 0, s>>>((const u32x2*)x, (const u32x2*)R, post, comb, (u32x2*)Rout, h);
        else
            k_post4<false><<<g, 256, 0, s>>>((const u32x2*)x, (const u32x2*)R, post, comb, (u32x2*)Rout, h);
        return hipGetLastError() == hipSuccess ? 0 : -1;
    }
    // Long runs: two workgroups per CU, whose waves each stream many items
    // and so keep fewer DRAM pages open at once (2.7 % faster than 16 per CU
    // at 65,536 tokens); short runs need the wider grid to fill the chip.
    const int g = grid_for(m.items, m.items >= (1ull << 24) ? 2 : 16);
    if (m.d8 % 64 == 0)
        k_post<true><<<g, 256, 0, s>>>((const u32x4*)x, (const u32x4*)R, post, comb, (u32x4*)Rout, m);
    else
        k_post<false><<<g, 256, 0, s>>>((const u32x4*)x, (const u32x4*)R, post, comb, (u32x4*)Rout, m);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_diag(const void* h, const void* D, void* x, int64_t n, int d, hipStream_t s) {
    ItemMap m{(uint32_t)(d / 8), (uint64_t)n * (uint64_t)(d / 8)};
    k_diag<<<grid_for(m.items, 8), 256, 0, s>>>((const u32x4*)h, (const u32x4*)D, (u32x4*)x, m);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace hc
