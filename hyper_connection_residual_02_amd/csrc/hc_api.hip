// hc_api.hip -- the C-ABI of libhc: argument checks (host only, before any
// HIP call) and dispatch to the kernels.  See include/hc.h for the contract
// of each entry point.
#include <math.h>
#include <mutex>

#include "../../include/hc.h"
#include "hc_launch.hpp"

namespace hc {

// ------------------------------------------------------- device properties
static std::mutex g_mu;
static int g_cus[64];

int num_cus() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_cus[dev] == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
        g_cus[dev] = v;
    }
    return g_cus[dev];
}

// ------------------------------------------------ static scratch (no-alloc)
// Workspace of hc_fused_mix_pre_noalloc, for callers that cannot allocate:
// one array per device, held until the process ends.  In host code
// `scratch` names a host-side stand-in, never the device memory: the
// device address comes from hipGetSymbolAddress, taken once per device with
// that device current, and only that address is passed to kernels.
static __device__ __align__(256) uint8_t scratch[HC_SCRATCH_BYTES];
static void* g_scratch[64];

// Device address of this device's scratch array, or null if it cannot be
// resolved (no device, or the symbol lookup failed).
void* scratch_ptr() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch[dev] = p;
    }
    return g_scratch[dev];
}

}  // namespace hc

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 40;   // bound on n*hc*d (sizes stay far from overflow)

bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool al4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

struct Span {
    uintptr_t lo, hi;   // [lo, hi)
};
Span span(const void* p, uint64_t bytes) { return Span{(uintptr_t)p, (uintptr_t)p + bytes}; }
bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

bool finite_nonneg(float v) { return isfinite(v) && v >= 0.0f; }

int check_nd(int64_t n, int32_t hc, int32_t d) {
    if (n < 0 || d <= 0 || d % 8 != 0) return HC_ERR_SHAPE;
    if (hc != 4 && !hc::gen_hc(hc)) return HC_ERR_UNSUPPORTED;
    if (n > 0 && n > kMaxElems / ((int64_t)hc * d)) return HC_ERR_SHAPE;
    return HC_OK;
}

}  // namespace

extern "C" {

const char* hc_status_str(int s) {
    switch (s) {
        case HC_OK: return "HC_OK";
        case HC_ERR_NULL: return "HC_ERR_NULL: a required pointer is NULL";
        case HC_ERR_SHAPE: return "HC_ERR_SHAPE: bad n or d (n >= 0, d > 0, d % 8 == 0)";
        case HC_ERR_ALIGN: return "HC_ERR_ALIGN: tensor pointers must be 16-byte aligned (scale/base 4-byte)";
        case HC_ERR_UNSUPPORTED: return "HC_ERR_UNSUPPORTED: hc must be 1..8 (4 for packed weights), sinkhorn_iters >= 1, d tileable";
        case HC_ERR_WORKSPACE: return "HC_ERR_WORKSPACE: workspace missing or too small";
        case HC_ERR_ALIAS: return "HC_ERR_ALIAS: an output overlaps an input or another output";
        case HC_ERR_VALUE: return "HC_ERR_VALUE: epsilon must be finite and >= 0";
        case HC_ERR_LAUNCH: return "HC_ERR_LAUNCH: the HIP runtime refused a kernel launch";
        case HC_ERR_DEVICE: return "HC_ERR_DEVICE: device query failed";
        case HC_ERR_TIMEOUT: return "HC_ERR_TIMEOUT: a call on this workspace stopped early (a bounded wait between workgroups gave up); its outputs are undefined";
        case HC_ERR_SCRATCH: return "HC_ERR_SCRATCH: the call needs more workspace than the static scratch holds (hc_scratch_bytes)";
        default: return "HC_ERR_?: unknown status";
    }
}

const char* hc_version(void) { return "0.1.0"; }

int hc_pre(const void* R, const float* pre, void* h, int64_t n, int32_t hc_, int32_t d, void* stream) {
    int st = check_nd(n, hc_, d);
    if (st) return st;
    if (n == 0) return HC_OK;
    if (!R || !pre || !h) return HC_ERR_NULL;
    if (!al16(R) || !al16(pre) || !al16(h)) return HC_ERR_ALIGN;
    const uint64_t nd = (uint64_t)n * d;
    Span sh = span(h, nd * 2);
    if (overlap(sh, span(R, nd * hc_ * 2)) || overlap(sh, span(pre, (uint64_t)n * hc_ * 4))) return HC_ERR_ALIAS;
    // one workgroup per token (or four), h only, up to 32,768 features; the
    // grid-stride kernels beyond
    int e;
    if (hc::norm_waves(d))
        e = hc::launch_pre_norm(R, pre, nullptr, h, nullptr, n, hc_, d, 0.0f, (hipStream_t)stream);
    else
        e = hc_ == 4 ? hc::launch_pre(R, pre, h, n, d, (hipStream_t)stream)
                     : hc::launch_gen_pre(R, pre, h, n, hc_, d, (hipStream_t)stream);
    return e ? HC_ERR_LAUNCH : HC_OK;
}

int hc_rmsnorm(const void* h, const float* gamma, void* y, int64_t n, int32_t d, float norm_eps, void* stream) {
    int st = check_nd(n, 1, d);
    if (st) return st;
    if (!finite_nonneg(norm_eps)) return HC_ERR_VALUE;
    if (hc::norm_waves(d) == 0) return HC_ERR_UNSUPPORTED;
    if (n == 0) return HC_OK;
    if (!h || !gamma || !y) return HC_ERR_NULL;
    if (!al16(h) || !al16(gamma) || !al16(y)) return HC_ERR_ALIGN;
    const uint64_t nd = (uint64_t)n * d;
    Span sy = span(y, nd * 2);
    if (overlap(sy, span(h, nd * 2)) || overlap(sy, span(gamma, (uint64_t)d * 4))) return HC_ERR_ALIAS;
    const int e = hc::launch_pre_norm(h, nullptr, gamma, nullptr, y, n, 0, d, norm_eps, (hipStream_t)stream);
    return e ? HC_ERR_LAUNCH : HC_OK;
}

int hc_pre_norm(const void* R, const float* pre, const float* gamma, void* h, void* y, int64_t n, int32_t hc_,
                int32_t d, float norm_eps, void* stream) {
    int st = check_nd(n, hc_, d);
    if (st) return st;
    if (!finite_nonneg(norm_eps)) return HC_ERR_VALUE;
    if (hc::norm_waves(d) == 0) return HC_ERR_UNSUPPORTED;
    if (n == 0) return HC_OK;
    if (!R || !pre || !gamma || !y) return HC_ERR_NULL;
    if (!al16(R) || !al16(pre) || !al16(gamma) || !al16(y) || (h && !al16(h))) return HC_ERR_ALIGN;
    const uint64_t nd = (uint64_t)n * d;
    const Span in[3] = {span(R, nd * hc_ * 2), span(pre, (uint64_t)n * hc_ * 4), span(gamma, (uint64_t)d * 4)};
    Span sy = span(y, nd * 2);
    for (const Span& x : in)
        if (overlap(sy, x) || (h && overlap(span(h, nd * 2), x))) return HC_ERR_ALIAS;
    if (h && overlap(sy, span(h, nd * 2))) return HC_ERR_ALIAS;
    const int e = hc::launch_pre_norm(R, pre, gamma, h, y, n, hc_, d, norm_eps, (hipStream_t)stream);
    return e ? HC_ERR_LAUNCH : HC_OK;
}

int hc_post(const void* x, const void* R, const float* post, const float* comb, void* R_out, int64_t n,
            int32_t hc_, int32_t d, void* stream) {
    int st = check_nd(n, hc_, d);
    if (st) return st;
    if (n == 0) return HC_OK;
    if (!x || !R || !post || !comb || !R_out) return HC_ERR_NULL;
    if (!al16(x) || !al16(R) || !al16(post) || !al16(comb) || !al16(R_out)) return HC_ERR_ALIGN;
    const uint64_t nd = (uint64_t)n * d;
    Span so = span(R_out, nd * hc_ * 2);
    if (R_out != R && overlap(so, span(R, nd * hc_ * 2))) return HC_ERR_ALIAS;
    if (overlap(so, span(x, nd * 2)) || overlap(so, span(post, (uint64_t)n * hc_ * 4)) ||
        overlap(so, span(comb, (uint64_t)n * hc_ * hc_ * 4)))
        return HC_ERR_ALIAS;
    const int e = hc_ == 4 ? hc::launch_post(x, R, post, comb, R_out, n, d, (hipStream_t)stream)
                           : hc::launch_gen_post(x, R, post, comb, R_out, n, hc_, d, (hipStream_t)stream);
    return e ? HC_ERR_LAUNCH : HC_OK;
}

int hc_diag_scale(const void* h, const void* D, void* x, int64_t n, int32_t d, void* stream) {
    int st = check_nd(n, 4, d);
    if (st) return st;
    if (n == 0) return HC_OK;
    if (!h || !D || !x) return HC_ERR_NULL;
    if (!al16(h) || !al16(D) || !al16(x)) return HC_ERR_ALIGN;
    const uint64_t nd = (uint64_t)n * d;
    Span sx = span(x, nd * 2);
    if (overlap(sx, span(h, nd * 2)) || overlap(sx, span(D, (uint64_t)d * 2))) return HC_ERR_ALIAS;
    return hc::launch_diag(h, D, x, n, d, (hipStream_t)stream) ? HC_ERR_LAUNCH : HC_OK;
}

int hc_split_sinkhorn(const float* mixes, const float* hc_scale, const float* hc_base, float* pre, float* post,
                      float* comb, int64_t n, int32_t hc_, int32_t sinkhorn_iters, float hc_eps, void* stream) {
    if (n < 0) return HC_ERR_SHAPE;
    if ((hc_ != 4 && !hc::gen_hc(hc_)) || sinkhorn_iters < 1) return HC_ERR_UNSUPPORTED;
    if (!finite_nonneg(hc_eps)) return HC_ERR_VALUE;
    const uint64_t M = (uint64_t)(2 + hc_) * hc_;
    if (n > kMaxElems / (int64_t)M) return HC_ERR_SHAPE;
    if (n == 0) return HC_OK;
    if (!mixes || !hc_scale || !hc_base || !pre || !post || !comb) return HC_ERR_NULL;
    if (!al16(mixes) || !al16(pre) || !al16(post) || !al16(comb) || !al4(hc_scale) || !al4(hc_base))
        return HC_ERR_ALIGN;
    const Span ins[] = {span(mixes, (uint64_t)n * M * 4), span(hc_scale, 12), span(hc_base, M * 4)};
    const Span outs[] = {span(pre, (uint64_t)n * hc_ * 4), span(post, (uint64_t)n * hc_ * 4),
                         span(comb, (uint64_t)n * hc_ * hc_ * 4)};
    for (const Span& o : outs)
        for (const Span& i : ins)
            if (overlap(o, i)) return HC_ERR_ALIAS;
    if (overlap(outs[0], outs[1]) || overlap(outs[0], outs[2]) || overlap(outs[1], outs[2])) return HC_ERR_ALIAS;
    const int e = hc_ == 4 ? hc::launch_split(mixes, hc_scale, hc_base, pre, post, comb, n, sinkhorn_iters, hc_eps,
                                              (hipStream_t)stream)
                           : hc::launch_gen_split(mixes, hc_scale, hc_base, pre, post, comb, n, hc_, sinkhorn_iters,
                                                  hc_eps, (hipStream_t)stream);
    return e ? HC_ERR_LAUNCH : HC_OK;
}

size_t hc_fused_workspace_bytes(int64_t n, int32_t hc_, int32_t d) {
    if (check_nd(n, hc_, d) != HC_OK || n == 0) return 0;
    if (hc_ != 4) return hc::gen_ws_bytes(n, hc_, d);
    hc::CoopPlan p;
    if (!hc::coop_plan(n, d, p)) return 0;
    return p.ws_bytes;
}

static int coop_common(const void* R, const float* hc_fn, void* workspace, size_t ws_bytes, int64_t n, int32_t hc_,
                       int32_t d, float norm_eps, hc::CoopPlan& p) {
    int st = check_nd(n, hc_, d);
    if (st) return st;
    if (!finite_nonneg(norm_eps)) return HC_ERR_VALUE;
    if (n == 0) return HC_OK;
    if (hc::coop_ks(d) == 0) return HC_ERR_UNSUPPORTED;
    if (!R || !hc_fn) return HC_ERR_NULL;
    if (!workspace) return HC_ERR_WORKSPACE;
    if (!al16(R) || !al16(hc_fn) || ((uintptr_t)workspace & 255u)) return HC_ERR_ALIGN;
    if (!hc::coop_plan(n, d, p)) return HC_ERR_UNSUPPORTED;
    if (ws_bytes < p.ws_bytes) return HC_ERR_WORKSPACE;
    return HC_OK;
}

int hc_mixes(const void* R, const float* hc_fn, float* mixes, int64_t n, int32_t hc_, int32_t d, float norm_eps,
             void* workspace, size_t workspace_bytes, void* stream) {
    if (hc_ != 4) {
        // other stream counts: one plain kernel, no workspace
        int st = check_nd(n, hc_, d);
        if (st) return st;
        if (!finite_nonneg(norm_eps)) return HC_ERR_VALUE;
        if (n == 0) return HC_OK;
        if (!R || !hc_fn || !mixes) return HC_ERR_NULL;
        if (!al16(R) || !al16(hc_fn) || !al16(mixes)) return HC_ERR_ALIGN;
        const uint64_t K = (uint64_t)hc_ * d, M = (uint64_t)(2 + hc_) * hc_;
        const Span sm = span(mixes, (uint64_t)n * M * 4);
        if (overlap(sm, span(R, (uint64_t)n * K * 2)) || overlap(sm, span(hc_fn, M * K * 4))) return HC_ERR_ALIAS;
        return hc::launch_gen_mixes(R, hc_fn, mixes, n, hc_, d, norm_eps, (hipStream_t)stream) ? HC_ERR_LAUNCH
                                                                                              : HC_OK;
    }
    hc::CoopPlan p;
    int st = coop_common(R, hc_fn, workspace, workspace_bytes, n, hc_, d, norm_eps, p);
    if (st || n == 0) return st;
    if (!mixes) return HC_ERR_NULL;
    if (!al16(mixes)) return HC_ERR_ALIGN;
    const uint64_t K = (uint64_t)4 * d;
    const Span sm = span(mixes, (uint64_t)n * 96);
    if (overlap(sm, span(R, (uint64_t)n * K * 2)) || overlap(sm, span(hc_fn, 24 * K * 4)) ||
        overlap(sm, span(workspace, p.ws_bytes)))
        return HC_ERR_ALIAS;
    return hc::launch_coop(p, R, hc_fn, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, mixes, workspace, n, d,
                           1, 0.0f, norm_eps, false, (hipStream_t)stream)
               ? HC_ERR_LAUNCH
               : HC_OK;
}

}  // extern "C"

// hc_fused_mix_pre (and, with prev, hc_post_mix_pre) for stream counts other
// than four: the checks of the four-stream call with hc-sized buffers, then
// the plain kernels in sequence.
static int gen_fused(const hc::PostIn* prev, const void* R, const float* hc_fn, const float* hc_scale,
                     const float* hc_base, void* h, float* pre, float* post, float* comb, float* mixes,
                     void* workspace, size_t workspace_bytes, int64_t n, int32_t hc_, int32_t d,
                     int32_t sinkhorn_iters, float hc_eps, float norm_eps, void* stream) {
    int st = check_nd(n, hc_, d);
    if (st) return st;
    if (sinkhorn_iters < 1) return HC_ERR_UNSUPPORTED;
    if (!finite_nonneg(hc_eps) || !finite_nonneg(norm_eps)) return HC_ERR_VALUE;
    if (n == 0) return HC_OK;
    if (!R || !hc_fn || !hc_scale || !hc_base || !h || !post || !comb) return HC_ERR_NULL;
    if (prev && (!prev->x || !prev->post || !prev->comb || !prev->Rout)) return HC_ERR_NULL;
    if (!workspace) return HC_ERR_WORKSPACE;
    // the call needs gen_ws_min_bytes; with gen_ws_bytes it also splits the
    // weights once (long calls), and uses that much
    const size_t full = hc::gen_ws_bytes(n, hc_, d);
    if (workspace_bytes < hc::gen_ws_min_bytes(n, hc_, d)) return HC_ERR_WORKSPACE;
    const size_t wsb = workspace_bytes >= full ? full : hc::gen_ws_min_bytes(n, hc_, d);
    if (!al16(R) || !al16(hc_fn) || ((uintptr_t)workspace & 255u) || !al4(hc_scale) || !al4(hc_base) || !al16(h) ||
        !al16(post) || !al16(comb) || (pre && !al16(pre)) || (mixes && !al16(mixes)))
        return HC_ERR_ALIGN;
    if (prev && (!al16(prev->x) || !al16(prev->post) || !al16(prev->comb))) return HC_ERR_ALIGN;
    const uint64_t K = (uint64_t)hc_ * d, M = (uint64_t)(2 + hc_) * hc_;
    const void* Rin = prev ? prev->Rout : R;   // the stream the projection reads
    const Span sR = span(R, (uint64_t)n * K * 2), sRin = span(Rin, (uint64_t)n * K * 2);
    if (prev && Rin != R && overlap(sRin, sR)) return HC_ERR_ALIAS;
    Span ins[8];
    int ni = 0;
    ins[ni++] = sR;
    ins[ni++] = span(hc_fn, M * K * 4);
    ins[ni++] = span(hc_scale, 12);
    ins[ni++] = span(hc_base, M * 4);
    ins[ni++] = span(workspace, wsb);
    if (prev) {
        ins[ni++] = span(prev->x, (uint64_t)n * d * 2);
        ins[ni++] = span(prev->post, (uint64_t)n * hc_ * 4);
        ins[ni++] = span(prev->comb, (uint64_t)n * hc_ * hc_ * 4);
    }
    Span outs[6];
    int no = 0;
    if (prev) outs[no++] = sRin;
    outs[no++] = span(h, (uint64_t)n * d * 2);
    outs[no++] = span(post, (uint64_t)n * hc_ * 4);
    outs[no++] = span(comb, (uint64_t)n * hc_ * hc_ * 4);
    if (pre) outs[no++] = span(pre, (uint64_t)n * hc_ * 4);
    if (mixes) outs[no++] = span(mixes, (uint64_t)n * M * 4);
    for (int i = 0; i < no; ++i) {
        // R_out (the first output of hc_post_mix_pre) may be R itself
        for (int k = 0; k < ni; ++k)
            if (!(prev && i == 0 && k == 0 && Rin == R) && overlap(outs[i], ins[k])) return HC_ERR_ALIAS;
        for (int j = i + 1; j < no; ++j)
            if (overlap(outs[i], outs[j])) return HC_ERR_ALIAS;
    }
    hipStream_t s = (hipStream_t)stream;
    if (prev && hc::launch_gen_post(prev->x, R, prev->post, prev->comb, prev->Rout, n, hc_, d, s))
        return HC_ERR_LAUNCH;
    return hc::launch_gen_fused(Rin, hc_fn, hc_scale, hc_base, h, pre, post, comb, mixes, workspace, wsb, n, hc_, d,
                                sinkhorn_iters, hc_eps, norm_eps, s)
               ? HC_ERR_LAUNCH
               : HC_OK;
}

// hc_fused_mix_pre with the weights as given (hc_fn) or already split
// (packed, from hc_pack_weights).
// The pre-sublayer RMSNorm of hc_fused_mix_pre_norm: y and gamma, checked
// by the caller.  h may then be null: y stands in for it in the checks and
// receives h, which the norm kernel then normalises in place.
struct NormOut {
    void* y;
    const float* gamma;
};

static int fused_impl(const void* R, const float* hc_fn, const void* packed, size_t packed_bytes,
                      const float* hc_scale, const float* hc_base, void* h_, float* pre, float* post, float* comb,
                      float* mixes, void* workspace, size_t workspace_bytes, int64_t n, int32_t hc_, int32_t d,
                      int32_t sinkhorn_iters, float hc_eps, float norm_eps, void* stream, bool gate = true,
                      const NormOut* norm = nullptr) {
    void* h = h_ ? h_ : (norm ? norm->y : nullptr);
    if (hc_ != 4) {
        if (packed) return HC_ERR_UNSUPPORTED;
        const int st = gen_fused(nullptr, R, hc_fn, hc_scale, hc_base, h, pre, post, comb, mixes, workspace,
                                 workspace_bytes, n, hc_, d, sinkhorn_iters, hc_eps, norm_eps, stream);
        if (st || !norm || n == 0) return st;
        return hc::launch_pre_norm(h, nullptr, norm->gamma, nullptr, norm->y, n, 0, d, norm_eps,
                                   (hipStream_t)stream)
                   ? HC_ERR_LAUNCH
                   : HC_OK;
    }
    if (sinkhorn_iters < 1) return HC_ERR_UNSUPPORTED;
    if (!finite_nonneg(hc_eps)) return HC_ERR_VALUE;
    hc::CoopPlan p;
    const void* wsrc = packed ? packed : (const void*)hc_fn;
    int st = coop_common(R, static_cast<const float*>(wsrc), workspace, workspace_bytes, n, hc_, d, norm_eps, p);
    if (st || n == 0) return st;
    const uint64_t K = (uint64_t)4 * d;
    uint64_t wbytes = 24 * K * 4;
    if (packed) {
        wbytes = hc::packed_weights_bytes(d);
        if (wbytes == 0) return HC_ERR_UNSUPPORTED;
        if (packed_bytes < wbytes) return HC_ERR_WORKSPACE;
    }
    if (!hc_scale || !hc_base || !h || !post || !comb) return HC_ERR_NULL;
    if (!al4(hc_scale) || !al4(hc_base) || !al16(h) || !al16(post) || !al16(comb) || (pre && !al16(pre)) ||
        (mixes && !al16(mixes)))
        return HC_ERR_ALIGN;
    const Span ins[] = {span(R, (uint64_t)n * K * 2), span(wsrc, wbytes), span(hc_scale, 12),
                        span(hc_base, 96), span(workspace, p.ws_bytes)};
    Span outs[5];
    int no = 0;
    outs[no++] = span(h, (uint64_t)n * d * 2);
    outs[no++] = span(post, (uint64_t)n * 16);
    outs[no++] = span(comb, (uint64_t)n * 64);
    if (pre) outs[no++] = span(pre, (uint64_t)n * 16);
    if (mixes) outs[no++] = span(mixes, (uint64_t)n * 96);
    for (int i = 0; i < no; ++i) {
        for (const Span& s : ins)
            if (overlap(outs[i], s)) return HC_ERR_ALIAS;
        for (int j = i + 1; j < no; ++j)
            if (overlap(outs[i], outs[j])) return HC_ERR_ALIAS;
    }
    p.gate = gate;
    if (hc::launch_coop(p, R, hc_fn, hc_scale, hc_base, h, pre, post, comb, mixes, workspace, n, d, sinkhorn_iters,
                        hc_eps, norm_eps, true, (hipStream_t)stream, nullptr, packed))
        return HC_ERR_LAUNCH;
    if (norm && hc::launch_pre_norm(h, nullptr, norm->gamma, nullptr, norm->y, n, 0, d, norm_eps,
                                    (hipStream_t)stream))
        return HC_ERR_LAUNCH;
    return HC_OK;
}

extern "C" {

int hc_fused_mix_pre(const void* R, const float* hc_fn, const float* hc_scale, const float* hc_base, void* h,
                     float* pre, float* post, float* comb, float* mixes, void* workspace, size_t workspace_bytes,
                     int64_t n, int32_t hc_, int32_t d, int32_t sinkhorn_iters, float hc_eps, float norm_eps,
                     void* stream) {
    return fused_impl(R, hc_fn, nullptr, 0, hc_scale, hc_base, h, pre, post, comb, mixes, workspace,
                      workspace_bytes, n, hc_, d, sinkhorn_iters, hc_eps, norm_eps, stream);
}

int hc_fused_mix_pre_norm(const void* R, const float* hc_fn, const float* hc_scale, const float* hc_base,
                          const float* gamma, void* h, void* y, float* pre, float* post, float* comb, float* mixes,
                          void* workspace, size_t workspace_bytes, int64_t n, int32_t hc_, int32_t d,
                          int32_t sinkhorn_iters, float hc_eps, float norm_eps, void* stream) {
    int st = check_nd(n, hc_, d);
    if (st) return st;
    if (!finite_nonneg(norm_eps)) return HC_ERR_VALUE;
    if (hc::norm_waves(d) == 0) return HC_ERR_UNSUPPORTED;
    if (n > 0) {
        if (!gamma || !y) return HC_ERR_NULL;
        if (!al16(gamma) || !al16(y)) return HC_ERR_ALIGN;
        const uint64_t K = (uint64_t)hc_ * d, M = (uint64_t)(2 + hc_) * hc_;
        const Span sy = span(y, (uint64_t)n * d * 2), sg = span(gamma, (uint64_t)d * 4);
        // y and gamma against everything else (the rest is checked below,
        // with y standing in for h when h is null)
        const Span others[] = {span(R, (uint64_t)n * K * 2), span(hc_fn, M * K * 4), span(hc_scale, 12),
                               span(hc_base, M * 4), span(workspace, workspace_bytes), span(h, h ? (uint64_t)n * d * 2 : 0),
                               span(post, (uint64_t)n * hc_ * 4), span(comb, (uint64_t)n * hc_ * hc_ * 4),
                               span(pre, pre ? (uint64_t)n * hc_ * 4 : 0), span(mixes, mixes ? (uint64_t)n * M * 4 : 0)};
        if (overlap(sy, sg)) return HC_ERR_ALIAS;
        for (int i = 0; i < 10; ++i) {
            if (overlap(sy, others[i])) return HC_ERR_ALIAS;
            if (i >= 5 && overlap(sg, others[i])) return HC_ERR_ALIAS;     // gamma is an input: outputs only
        }
    }
    const NormOut no{y, gamma};
    return fused_impl(R, hc_fn, nullptr, 0, hc_scale, hc_base, h, pre, post, comb, mixes, workspace,
                      workspace_bytes, n, hc_, d, sinkhorn_iters, hc_eps, norm_eps, stream, true, &no);
}

size_t hc_packed_weights_bytes(int32_t hc_, int32_t d) {
    if (hc_ != 4 || d <= 0) return 0;
    return hc::packed_weights_bytes(d);
}

int hc_pack_weights(const float* hc_fn, void* packed, size_t packed_bytes, int32_t hc_, int32_t d, void* stream) {
    if (d <= 0 || d % 8 != 0) return HC_ERR_SHAPE;
    if (hc_ != 4) return HC_ERR_UNSUPPORTED;
    const size_t pb = hc::packed_weights_bytes(d);
    if (pb == 0) return HC_ERR_UNSUPPORTED;
    if (!hc_fn || !packed) return HC_ERR_NULL;
    if (!al16(hc_fn) || !al16(packed)) return HC_ERR_ALIGN;
    if (packed_bytes < pb) return HC_ERR_WORKSPACE;
    if (overlap(span(packed, pb), span(hc_fn, (uint64_t)24 * 4 * d * 4))) return HC_ERR_ALIAS;
    return hc::launch_pack(hc_fn, packed, d, (hipStream_t)stream) ? HC_ERR_LAUNCH : HC_OK;
}

int hc_fused_mix_pre_packed(const void* R, const void* packed, size_t packed_bytes, const float* hc_scale,
                            const float* hc_base, void* h, float* pre, float* post, float* comb, float* mixes,
                            void* workspace, size_t workspace_bytes, int64_t n, int32_t hc_, int32_t d,
                            int32_t sinkhorn_iters, float hc_eps, float norm_eps, void* stream) {
    if (!packed && n > 0) return HC_ERR_NULL;
    return fused_impl(R, nullptr, packed, packed_bytes, hc_scale, hc_base, h, pre, post, comb, mixes, workspace,
                      workspace_bytes, n, hc_, d, sinkhorn_iters, hc_eps, norm_eps, stream);
}

size_t hc_scratch_bytes(void) { return HC_SCRATCH_BYTES; }

int hc_fused_mix_pre_noalloc(const void* R, const float* hc_fn, const float* hc_scale, const float* hc_base,
                             void* h, float* pre, float* post, float* comb, float* mixes, int64_t n, int32_t hc_,
                             int32_t d, int32_t sinkhorn_iters, float hc_eps, float norm_eps, void* stream) {
    int st = check_nd(n, hc_, d);
    if (st) return st;
    if (n == 0) return HC_OK;
    // the workspace this call needs must fit the static array; unsupported
    // shapes (size 0) are reported by the call itself
    // other stream counts need only the minimum (the weights are then split
    // as they are staged)
    if (check_nd(n, hc_, d) == HC_OK && n > 0 &&
        (hc_ == 4 ? hc_fused_workspace_bytes(n, hc_, d) : hc::gen_ws_min_bytes(n, hc_, d)) > HC_SCRATCH_BYTES)
        return HC_ERR_SCRATCH;
    void* ws = hc::scratch_ptr();
    if (!ws) return HC_ERR_DEVICE;
    // no launch ordering across streams here: that would create an event
    // (calls that overlap on one GPU race on the one array anyway)
    return fused_impl(R, hc_fn, nullptr, 0, hc_scale, hc_base, h, pre, post, comb, mixes, ws, HC_SCRATCH_BYTES, n,
                      hc_, d, sinkhorn_iters, hc_eps, norm_eps, stream, false);
}

int hc_workspace_status(const void* workspace, size_t workspace_bytes, int clear) {
    if (!workspace) return HC_ERR_NULL;
    if ((uintptr_t)workspace & 255u) return HC_ERR_ALIGN;
    if (workspace_bytes < 256) return HC_ERR_WORKSPACE;
    const int r = hc::ws_status(workspace, clear != 0);
    return r < 0 ? HC_ERR_DEVICE : (r ? HC_ERR_TIMEOUT : HC_OK);
}

int hc_noalloc_status(int clear) {
    void* ws = hc::scratch_ptr();
    if (!ws) return HC_ERR_DEVICE;
    const int r = hc::ws_status(ws, clear != 0);
    return r < 0 ? HC_ERR_DEVICE : (r ? HC_ERR_TIMEOUT : HC_OK);
}

int hc_phase_trace(uint64_t* out, size_t count) {
    if (!out && count) return HC_ERR_NULL;
    const int r = hc::phase_trace_copy(out, count);
    return r < 0 ? HC_ERR_UNSUPPORTED : r;
}

int hc_probe_stream(const void* src, void* dst, size_t bytes, int32_t wg_per_cu, void* stream) {
    if (bytes % 16 != 0) return HC_ERR_SHAPE;
    if (wg_per_cu < 0 || wg_per_cu > 32) return HC_ERR_VALUE;
    if (bytes == 0) return HC_OK;
    if (!src) return HC_ERR_NULL;
    if (!al16(src) || (dst && !al16(dst))) return HC_ERR_ALIGN;
    if (dst && overlap(span(src, bytes), span(dst, bytes))) return HC_ERR_ALIAS;
    return hc::launch_probe(src, dst, bytes, wg_per_cu ? wg_per_cu : 2, (hipStream_t)stream) ? HC_ERR_LAUNCH
                                                                                              : HC_OK;
}

int hc_debug_force_timeout(int calls) {
    if (calls < 0) return HC_ERR_VALUE;
    hc::set_force_timeout(calls);
    return HC_OK;
}

int hc_post_backward(const void* x, const void* R, const float* post, const float* comb, const void* gRout,
                     void* gx, float* gpost, float* gcomb, int64_t n, int32_t hc_, int32_t d, void* stream) {
    int st = check_nd(n, hc_, d);
    if (st) return st;
    if (hc_ != 4) return HC_ERR_UNSUPPORTED;
    if (n == 0) return HC_OK;
    if (!x || !R || !post || !comb || !gRout || !gx || !gpost || !gcomb) return HC_ERR_NULL;
    if (!al16(x) || !al16(R) || !al16(post) || !al16(comb) || !al16(gRout) || !al16(gx) || !al16(gpost) ||
        !al16(gcomb))
        return HC_ERR_ALIGN;
    const uint64_t nd = (uint64_t)n * d;
    const Span ins[] = {span(x, nd * 2), span(R, nd * 8), span(post, (uint64_t)n * 16), span(comb, (uint64_t)n * 64),
                        span(gRout, nd * 8)};
    const Span outs[] = {span(gx, nd * 2), span(gpost, (uint64_t)n * 16), span(gcomb, (uint64_t)n * 64)};
    for (int i = 0; i < 3; ++i) {
        for (const Span& in : ins)
            if (overlap(outs[i], in)) return HC_ERR_ALIAS;
        for (int j = i + 1; j < 3; ++j)
            if (overlap(outs[i], outs[j])) return HC_ERR_ALIAS;
    }
    return hc::launch_post_bwd(x, R, post, comb, gRout, gx, gpost, gcomb, n, d, (hipStream_t)stream) ? HC_ERR_LAUNCH
                                                                                                    : HC_OK;
}

size_t hc_backward_workspace_bytes(int64_t n, int32_t hc_, int32_t d) {
    if (check_nd(n, hc_, d) != HC_OK || n == 0 || !hc::bwd_supported(hc_, d, 1)) return 0;
    return hc::bwd_ws_bytes(n, d);
}

int hc_mix_pre_backward(const void* R, const float* hc_fn, const float* hc_scale, const float* hc_base,
                        const float* mixes, const void* gh, const void* gRout, const float* gpost,
                        const float* gcomb, void* gR, float* g_hc_fn, float* g_hc_scale, float* g_hc_base,
                        float* gmixes, void* workspace, size_t workspace_bytes, int64_t n, int32_t hc_, int32_t d,
                        int32_t sinkhorn_iters, float hc_eps, float norm_eps, void* stream) {
    int st = check_nd(n, hc_, d);
    if (st) return st;
    if (!hc::bwd_supported(hc_, d, sinkhorn_iters)) return HC_ERR_UNSUPPORTED;
    if (!finite_nonneg(hc_eps) || !finite_nonneg(norm_eps)) return HC_ERR_VALUE;
    if (n == 0) return HC_OK;
    if (!R || !hc_fn || !hc_scale || !hc_base || !mixes || !gh || !gRout || !gpost || !gcomb || !gR || !g_hc_fn ||
        !g_hc_scale || !g_hc_base)
        return HC_ERR_NULL;
    if (!workspace) return HC_ERR_WORKSPACE;
    const size_t wsb = hc::bwd_ws_bytes(n, d);
    if (workspace_bytes < wsb) return HC_ERR_WORKSPACE;
    if (!al16(R) || !al16(hc_fn) || !al4(hc_scale) || !al4(hc_base) || !al16(mixes) || !al16(gh) || !al16(gRout) ||
        !al16(gpost) || !al16(gcomb) || !al16(gR) || !al16(g_hc_fn) || !al4(g_hc_scale) || !al4(g_hc_base) ||
        (gmixes && !al16(gmixes)) || ((uintptr_t)workspace & 255u))
        return HC_ERR_ALIGN;
    const uint64_t nd = (uint64_t)n * d, K = (uint64_t)4 * d;
    const Span ins[] = {span(R, nd * 8),           span(hc_fn, 24 * K * 4),        span(hc_scale, 12),
                        span(hc_base, 96),         span(mixes, (uint64_t)n * 96), span(gh, nd * 2),
                        span(gRout, nd * 8),       span(gpost, (uint64_t)n * 16), span(gcomb, (uint64_t)n * 64),
                        span(workspace, wsb)};
    Span outs[5];
    int no = 0;
    outs[no++] = span(gR, nd * 8);
    outs[no++] = span(g_hc_fn, 24 * K * 4);
    outs[no++] = span(g_hc_scale, 12);
    outs[no++] = span(g_hc_base, 96);
    if (gmixes) outs[no++] = span(gmixes, (uint64_t)n * 96);
    for (int i = 0; i < no; ++i) {
        for (const Span& in : ins)
            if (overlap(outs[i], in)) return HC_ERR_ALIAS;
        for (int j = i + 1; j < no; ++j)
            if (overlap(outs[i], outs[j])) return HC_ERR_ALIAS;
    }
    return hc::launch_mix_pre_bwd(R, hc_fn, hc_scale, hc_base, mixes, gh, gRout, gpost, gcomb, gR, g_hc_fn,
                                  g_hc_scale, g_hc_base, gmixes, workspace, n, d, sinkhorn_iters, hc_eps, norm_eps,
                                  (hipStream_t)stream)
               ? HC_ERR_LAUNCH
               : HC_OK;
}

int hc_post_mix_pre(const void* x, const void* R, const float* post, const float* comb, void* R_out,
                    const float* hc_fn, const float* hc_scale, const float* hc_base, void* h, float* pre_next,
                    float* post_next, float* comb_next, float* mixes_next, void* workspace, size_t workspace_bytes,
                    int64_t n, int32_t hc_, int32_t d, int32_t sinkhorn_iters, float hc_eps, float norm_eps,
                    void* stream) {
    if (hc_ != 4) {
        const hc::PostIn prev{x, post, comb, R_out};
        return gen_fused(&prev, R, hc_fn, hc_scale, hc_base, h, pre_next, post_next, comb_next, mixes_next,
                         workspace, workspace_bytes, n, hc_, d, sinkhorn_iters, hc_eps, norm_eps, stream);
    }
    if (sinkhorn_iters < 1) return HC_ERR_UNSUPPORTED;
    if (!finite_nonneg(hc_eps)) return HC_ERR_VALUE;
    hc::CoopPlan p;
    int st = coop_common(R, hc_fn, workspace, workspace_bytes, n, hc_, d, norm_eps, p);
    if (st || n == 0) return st;
    if (!x || !post || !comb || !R_out || !hc_scale || !hc_base || !h || !post_next || !comb_next)
        return HC_ERR_NULL;
    if (!al16(x) || !al16(post) || !al16(comb) || !al16(R_out) || !al4(hc_scale) || !al4(hc_base) || !al16(h) ||
        !al16(post_next) || !al16(comb_next) || (pre_next && !al16(pre_next)) || (mixes_next && !al16(mixes_next)))
        return HC_ERR_ALIGN;
    const uint64_t K = (uint64_t)4 * d;
    const Span sR = span(R, (uint64_t)n * K * 2), sRo = span(R_out, (uint64_t)n * K * 2);
    // R_out == R is allowed (the residual updated in place); any other
    // overlap of R_out with R is not
    if (R_out != R && overlap(sRo, sR)) return HC_ERR_ALIAS;
    const Span ins[] = {span(x, (uint64_t)n * d * 2), span(post, (uint64_t)n * 16), span(comb, (uint64_t)n * 64),
                        span(hc_fn, 24 * K * 4), span(hc_scale, 12), span(hc_base, 96),
                        span(workspace, p.ws_bytes)};
    Span outs[6];
    int no = 0;
    outs[no++] = sRo;
    outs[no++] = span(h, (uint64_t)n * d * 2);
    outs[no++] = span(post_next, (uint64_t)n * 16);
    outs[no++] = span(comb_next, (uint64_t)n * 64);
    if (pre_next) outs[no++] = span(pre_next, (uint64_t)n * 16);
    if (mixes_next) outs[no++] = span(mixes_next, (uint64_t)n * 96);
    for (int i = 0; i < no; ++i) {
        for (const Span& s : ins)
            if (overlap(outs[i], s)) return HC_ERR_ALIAS;
        if (i > 0 && overlap(outs[i], sR)) return HC_ERR_ALIAS;
        for (int j = i + 1; j < no; ++j)
            if (overlap(outs[i], outs[j])) return HC_ERR_ALIAS;
    }
    const hc::PostIn prev{x, post, comb, R_out};
    return hc::launch_coop(p, R, hc_fn, hc_scale, hc_base, h, pre_next, post_next, comb_next, mixes_next, workspace,
                           n, d, sinkhorn_iters, hc_eps, norm_eps, true, (hipStream_t)stream, &prev)
               ? HC_ERR_LAUNCH
               : HC_OK;
}

}  // extern "C"
