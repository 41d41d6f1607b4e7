// hc_probe.hip -- the bandwidth probe behind the streaming ceilings the
// kernels are measured against (hc_probe_stream).
//
// A plain stream over a buffer with the access pattern of the library's
// streaming kernels: each lane moves 16-byte chunks with non-temporal
// loads and stores, two chunks in flight, over a grid of a chosen number
// of workgroups per compute unit (two, as the streaming kernels use on long
// runs, by default) walking the buffer with a grid stride.  dst non-null:
// a device copy src -> dst (read and write).  dst null: a read-only stream,
// whose words are folded into a value the kernel keeps live, so that no
// load is dropped.

#include "hc_device.hpp"
#include "hc_launch.hpp"

namespace hc {

namespace {

__global__ __launch_bounds__(256) void k_probe(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                               uint64_t chunks) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0u;
    for (; i + stride < chunks; i += 2 * stride) {
        const u32x4 a = __builtin_nontemporal_load(src + i);
        const u32x4 b = __builtin_nontemporal_load(src + i + stride);
        if (dst) {
            __builtin_nontemporal_store(a, dst + i);
            __builtin_nontemporal_store(b, dst + i + stride);
        } else {
            acc ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3];
        }
    }
    if (i < chunks) {
        const u32x4 a = __builtin_nontemporal_load(src + i);
        if (dst) __builtin_nontemporal_store(a, dst + i);
        else acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
    }
    asm volatile("" ::"v"(acc));       // the read-only stream's loads stay
}

}  // namespace

int launch_probe(const void* src, void* dst, uint64_t bytes, int wg_per_cu, hipStream_t s) {
    const uint64_t chunks = bytes / 16;
    if (chunks == 0) return 0;
    uint64_t blocks = (chunks + 255) / 256;
    const uint64_t cap = (uint64_t)num_cus() * (uint64_t)wg_per_cu;
    if (blocks > cap) blocks = cap;
    k_probe<<<(unsigned)blocks, 256, 0, s>>>(static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), chunks);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace hc
