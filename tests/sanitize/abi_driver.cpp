// Test infrastructure (not part of the library): calls every entry point of
// include/hc.h on its argument-checking paths (null, misaligned, aliased
// and out-of-range arguments, n = 0) and every host-only query, in a build
// of the library's host code with AddressSanitizer and
// UndefinedBehaviorSanitizer.  None of these calls reaches a kernel launch,
// so no GPU is needed.  Exit status 0 when every status is the documented
// one.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "hc.h"

namespace {

int g_bad = 0;

void expect(const char* what, long got, long want) {
    if (got != want) {
        std::fprintf(stderr, "%s: got %ld, want %ld\n", what, got, want);
        g_bad = 1;
    }
}

void* P(uintptr_t a) { return reinterpret_cast<void*>(a); }
float* F(uintptr_t a) { return reinterpret_cast<float*>(a); }

// fake, aligned, far-apart addresses: the checks compare them, never read them
constexpr uintptr_t A = 0x10000, B = 0x20000000, C = 0x40000000, D = 0x60000000, E = 0x70000000,
                    W = 0x7C000000, G = 0x50000000, Y = 0x58000000;
const float NAN_F = std::nanf("");

}  // namespace

int main() {
    // status strings and version
    for (int s = -12; s <= 1; ++s) {
        const char* str = hc_status_str(s);
        if (!str || std::strncmp(str, "HC_", 3) != 0) expect("hc_status_str prefix", s, 1000);
    }
    expect("hc_version dots", std::strchr(hc_version(), '.') != nullptr, 1);

    // host-only size queries over a grid
    for (int hc = 0; hc <= 9; ++hc)
        for (int d : {8, 48, 64, 256, 1000, 5120, 6144, 32768}) {
            for (int64_t n : {0, 1, 64, 2048, 2049, 65536}) {
                (void)hc_fused_workspace_bytes(n, hc, d);
                (void)hc_backward_workspace_bytes(n, hc, d);
            }
            (void)hc_packed_weights_bytes(hc, d);
        }
    expect("hc_fused_workspace_bytes(0)", (long)hc_fused_workspace_bytes(0, 4, 5120), 0);
    expect("hc_scratch_bytes", hc_scratch_bytes() == HC_SCRATCH_BYTES, 1);

    // hc_mixes
    auto mixes = [](uintptr_t R, uintptr_t Wt, uintptr_t out, int64_t n, int hc, int d, float neps, uintptr_t ws,
                    size_t wsb) { return hc_mixes(P(R), F(Wt), F(out), n, hc, d, neps, P(ws), wsb, nullptr); };
    expect("mixes n=0", mixes(A, B, C, 0, 4, 64, 1e-20f, W, 1u << 30), HC_OK);
    expect("mixes null out", mixes(A, B, 0, 4, 4, 64, 1e-20f, W, 1u << 30), HC_ERR_NULL);
    expect("mixes misaligned", mixes(A, B, C + 4, 4, 4, 64, 1e-20f, W, 1u << 30), HC_ERR_ALIGN);
    expect("mixes alias", mixes(A, B, A, 4, 4, 64, 1e-20f, W, 1u << 30), HC_ERR_ALIAS);
    expect("mixes workspace", mixes(A, B, C, 4, 4, 64, 1e-20f, W, 0), HC_ERR_WORKSPACE);
    expect("mixes hc", mixes(A, B, C, 4, 9, 64, 1e-20f, W, 1u << 30), HC_ERR_UNSUPPORTED);
    expect("mixes eps", mixes(A, B, C, 4, 4, 64, NAN_F, W, 1u << 30), HC_ERR_VALUE);

    // hc_split_sinkhorn
    auto split = [](int64_t n, int hc, int it, float eps, uintptr_t pre) {
        return hc_split_sinkhorn(F(A), F(B), F(B + 64), F(pre), F(D), F(E), n, hc, it, eps, nullptr);
    };
    expect("split n=0", split(0, 4, 20, 1e-6f, C), HC_OK);
    expect("split n<0", split(-3, 4, 20, 1e-6f, C), HC_ERR_SHAPE);
    expect("split iters", split(4, 4, 0, 1e-6f, C), HC_ERR_UNSUPPORTED);
    expect("split eps", split(4, 4, 20, -1.0f, C), HC_ERR_VALUE);
    expect("split pre misaligned", split(4, 4, 20, 1e-6f, C + 4), HC_ERR_ALIGN);

    // hc_pre, hc_post, hc_diag_scale
    expect("pre null", hc_pre(P(A), F(B), nullptr, 4, 4, 64, nullptr), HC_ERR_NULL);
    expect("pre alias", hc_pre(P(A), F(B), P(A + 64), 4, 4, 64, nullptr), HC_ERR_ALIAS);
    expect("pre shape", hc_pre(P(A), F(B), P(C), 4, 4, 12, nullptr), HC_ERR_SHAPE);
    expect("pre size bound", hc_pre(P(A), F(B), P(C), (int64_t)1 << 40, 4, 64, nullptr), HC_ERR_SHAPE);
    expect("post alias", hc_post(P(A), P(B), F(C), F(D), P(B + 16), 4, 4, 64, nullptr), HC_ERR_ALIAS);
    expect("post misaligned", hc_post(P(A), P(B + 8), F(C), F(D), P(E), 4, 4, 64, nullptr), HC_ERR_ALIGN);
    expect("post hc", hc_post(P(A), P(B), F(C), F(D), P(E), 4, 0, 64, nullptr), HC_ERR_UNSUPPORTED);
    expect("diag null", hc_diag_scale(P(A), nullptr, P(C), 4, 64, nullptr), HC_ERR_NULL);
    expect("diag n=0", hc_diag_scale(P(A), P(B), P(C), 0, 64, nullptr), HC_OK);

    // the RMSNorm calls
    expect("rmsnorm n=0", hc_rmsnorm(P(A), F(B), P(C), 0, 64, 1e-20f, nullptr), HC_OK);
    expect("rmsnorm wide", hc_rmsnorm(P(A), F(B), P(C), 4, 32776, 1e-20f, nullptr), HC_ERR_UNSUPPORTED);
    expect("rmsnorm eps", hc_rmsnorm(P(A), F(B), P(C), 4, 64, -1.0f, nullptr), HC_ERR_VALUE);
    expect("rmsnorm alias", hc_rmsnorm(P(A), F(B), P(A + 256), 4, 64, 1e-20f, nullptr), HC_ERR_ALIAS);
    expect("pre_norm null", hc_pre_norm(P(A), F(B), nullptr, P(C), P(D), 4, 4, 64, 1e-20f, nullptr), HC_ERR_NULL);
    expect("pre_norm alias", hc_pre_norm(P(A), F(B), F(B + 4096), P(C), P(C + 64), 4, 4, 64, 1e-20f, nullptr),
           HC_ERR_ALIAS);

    // the fused calls
    auto fused = [](uintptr_t h, uintptr_t ws, size_t wsb, int64_t n, int hc, int d, int it) {
        return hc_fused_mix_pre(P(A), F(B), F(C), F(C + 64), P(h), F(E), F(E + 4096), F(E + 8192), nullptr, P(ws),
                                wsb, n, hc, d, it, 1e-6f, 1e-20f, nullptr);
    };
    expect("fused n=0", fused(D, W, 1u << 30, 0, 4, 64, 20), HC_OK);
    expect("fused untileable", fused(D, W, 1u << 30, 4, 4, 48, 20), HC_ERR_UNSUPPORTED);
    expect("fused iters", fused(D, W, 1u << 30, 4, 4, 64, 0), HC_ERR_UNSUPPORTED);
    expect("fused h null", fused(0, W, 1u << 30, 4, 4, 64, 20), HC_ERR_NULL);
    expect("fused ws align", fused(D, W + 128, 1u << 30, 4, 4, 64, 20), HC_ERR_ALIGN);
    expect("fused ws small", fused(D, W, 16, 4, 4, 64, 20), HC_ERR_WORKSPACE);
    expect("fused alias", fused(A, W, 1u << 30, 4, 4, 64, 20), HC_ERR_ALIAS);
    expect("fused hc=2 alias", fused(A, W, 1u << 30, 4, 2, 64, 20), HC_ERR_ALIAS);
    expect("fused_norm gamma null",
           hc_fused_mix_pre_norm(P(A), F(B), F(C), F(C + 64), nullptr, P(D), P(Y), F(E), F(E + 4096), F(E + 8192),
                                 nullptr, P(W), 1u << 30, 4, 4, 64, 20, 1e-6f, 1e-20f, nullptr),
           HC_ERR_NULL);
    expect("fused_norm y alias",
           hc_fused_mix_pre_norm(P(A), F(B), F(C), F(C + 64), F(G), nullptr, P(A + 64), F(E), F(E + 4096),
                                 F(E + 8192), nullptr, P(W), 1u << 30, 4, 4, 64, 20, 1e-6f, 1e-20f, nullptr),
           HC_ERR_ALIAS);
    expect("post_mix_pre alias",
           hc_post_mix_pre(P(A), P(B), F(C), F(C + 64), P(B + 16), F(E), F(E + 0x10000), F(E + 0x10040), P(D),
                           F(D + 0x1000), F(D + 0x2000), F(D + 0x3000), nullptr, P(W), 1u << 30, 4, 4, 64, 20, 1e-6f,
                           1e-20f, nullptr),
           HC_ERR_ALIAS);
    expect("pack small", hc_pack_weights(F(A), P(B), 16, 4, 5120, nullptr), HC_ERR_WORKSPACE);
    expect("pack hc", hc_pack_weights(F(A), P(B), 1u << 30, 3, 5120, nullptr), HC_ERR_UNSUPPORTED);
    expect("packed small",
           hc_fused_mix_pre_packed(P(A), P(B), 16, F(C), F(C + 64), P(D), F(E), F(E + 4096), F(E + 8192), nullptr,
                                   P(W), 1u << 30, 4, 4, 5120, 20, 1e-6f, 1e-20f, nullptr),
           HC_ERR_WORKSPACE);
    expect("noalloc hc", hc_fused_mix_pre_noalloc(P(A), F(B), F(C), F(C + 64), P(D), F(E), F(E + 4096), F(E + 8192),
                                                  nullptr, 4, 9, 64, 20, 1e-6f, 1e-20f, nullptr),
           HC_ERR_UNSUPPORTED);

    // the backward calls
    expect("post_backward null",
           hc_post_backward(P(A), P(B), F(C), F(C + 64), nullptr, P(D), F(E), F(E + 4096), 4, 4, 64, nullptr),
           HC_ERR_NULL);
    expect("post_backward hc",
           hc_post_backward(P(A), P(B), F(C), F(C + 64), P(G), P(D), F(E), F(E + 4096), 4, 3, 64, nullptr),
           HC_ERR_UNSUPPORTED);
    auto mix_b = [](uintptr_t ws, size_t wsb, int hc, int d, int it) {
        return hc_mix_pre_backward(P(A), F(B), F(C), F(C + 64), F(C + 4096), P(D), P(D + 0x100000), F(E),
                                   F(E + 4096), P(G), F(Y), F(Y + 0x100000), F(Y + 0x200000), nullptr, P(ws), wsb, 4,
                                   hc, d, it, 1e-6f, 1e-20f, nullptr);
    };
    expect("mix_pre_backward ws", mix_b(0, 0, 4, 256, 20), HC_ERR_WORKSPACE);
    expect("mix_pre_backward d", mix_b(W, 1u << 24, 4, 64, 20), HC_ERR_UNSUPPORTED);
    expect("mix_pre_backward iters", mix_b(W, 1u << 24, 4, 256, 65), HC_ERR_UNSUPPORTED);
    expect("mix_pre_backward hc", mix_b(W, 1u << 24, 2, 256, 20), HC_ERR_UNSUPPORTED);

    // the bandwidth probe
    expect("probe n=0", hc_probe_stream(P(A), P(B), 0, 0, nullptr), HC_OK);
    expect("probe shape", hc_probe_stream(P(A), P(B), 24, 0, nullptr), HC_ERR_SHAPE);
    expect("probe null", hc_probe_stream(nullptr, P(B), 4096, 0, nullptr), HC_ERR_NULL);
    expect("probe alias", hc_probe_stream(P(A), P(A + 1024), 4096, 0, nullptr), HC_ERR_ALIAS);
    expect("probe wg", hc_probe_stream(P(A), P(B), 4096, 33, nullptr), HC_ERR_VALUE);

    // workspace status and diagnostics
    expect("status null", hc_workspace_status(nullptr, 256, 0), HC_ERR_NULL);
    expect("status align", hc_workspace_status(P(W + 16), 256, 0), HC_ERR_ALIGN);
    expect("status small", hc_workspace_status(P(W), 16, 0), HC_ERR_WORKSPACE);
    (void)hc_noalloc_status(0);
    expect("force_timeout negative", hc_debug_force_timeout(-1), HC_ERR_VALUE);
    uint64_t trace_words[16] = {0};
    expect("phase_trace null", hc_phase_trace(nullptr, 16), HC_ERR_NULL);
    expect("phase_trace untraced build", hc_phase_trace(trace_words, 16), HC_ERR_UNSUPPORTED);

    std::printf(g_bad ? "FAIL\n" : "ok\n");
    return g_bad;
}
