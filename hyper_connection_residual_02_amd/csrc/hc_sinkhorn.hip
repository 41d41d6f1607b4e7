// hc_sinkhorn.hip -- standalone split of the mixes into pre / post / comb
// with the epsilon-Sinkhorn iteration ("Reading weights" page, the
// hc_split_sinkhorn kernel listing).  One token per 16-lane row, so a
// 256-thread block handles 16 tokens per step; the per-token arithmetic is
// the shared split_sinkhorn16, identical to the fused kernel's.
#include "hc_device.hpp"
#include "hc_launch.hpp"

namespace hc {

__global__ __launch_bounds__(256) void k_split(const float* __restrict__ mixes, const float* __restrict__ scale,
                                               const float* __restrict__ base, float* pre,
                                               float* __restrict__ post, float* __restrict__ comb, int64_t n,
                                               int iters, float eps) {
    const float s0 = scale[0], s1 = scale[1], s2 = scale[2];
    const int e = threadIdx.x & 15;
    for (int64_t t0 = (int64_t)blockIdx.x * 16; t0 < n; t0 += (int64_t)gridDim.x * 16) {
        const int64_t t = t0 + (threadIdx.x >> 4);
        const bool valid = t < n;
        // rows past the end compute a copy of the last token so that every
        // lane of a row takes part in the cross-lane reductions
        const int64_t tt = valid ? t : n - 1;
        float p, q, c;
        split_sinkhorn16(mixes + tt * kMix, s0, s1, s2, base, iters, eps, p, q, c);
        if (valid) {
            comb[t * (kHC * kHC) + e] = c;
            if (e < kHC) {
                if (pre) pre[t * kHC + e] = p;
                post[t * kHC + e] = q;
            }
        }
    }
}

int launch_split(const float* mixes, const float* scale, const float* base, float* pre, float* post,
                 float* comb, int64_t n, int iters, float eps, hipStream_t s) {
    int64_t blocks = (n + 15) / 16;
    const int64_t cap = (int64_t)num_cus() * 8;
    if (blocks > cap) blocks = cap;
    k_split<<<(int)blocks, 256, 0, s>>>(mixes, scale, base, pre, post, comb, n, iters, eps);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace hc
