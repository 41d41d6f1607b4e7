// hc_launch.hpp -- internal launch interface between the C-ABI layer and the
// kernel translation units.  Host code only; not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hc {

// Compute units of the current device (cached per device id).
int num_cus();

// Streaming kernels (hc_stream.hip).  Return 0, or -1 if the launch failed.
int launch_pre(const void* R, const float* pre, void* h, int64_t n, int d, hipStream_t s);
int launch_post(const void* x, const void* R, const float* post, const float* comb, void* Rout,
                int64_t n, int d, hipStream_t s);
int launch_diag(const void* h, const void* D, void* x, int64_t n, int d, hipStream_t s);

// Pre-sublayer RMSNorm (hc_norm.hip): hc = 0 normalises h = R itself (pre
// unused, h unused); hc >= 1 forms h = hc_pre(R, pre) first, written to h
// unless it is null.  norm_waves(d) is 0 if d is too wide.
int norm_waves(int d);
int launch_pre_norm(const void* R, const float* pre, const float* gamma, void* h, void* y, int64_t n, int hc,
                    int d, float norm_eps, hipStream_t s);

// Bandwidth probe (hc_probe.hip): copy src -> dst, or read src when dst is
// null, on wg_per_cu workgroups per compute unit.
int launch_probe(const void* src, void* dst, uint64_t bytes, int wg_per_cu, hipStream_t s);
// Phase tables of the wave-specialised kernel (phase-tracing builds only):
// words copied, or -1.
int phase_trace_copy(uint64_t* out, size_t count);

// Standalone split + Sinkhorn (hc_sinkhorn.hip); pre may be NULL (not written).
int launch_split(const float* mixes, const float* scale, const float* base, float* pre, float* post,
                 float* comb, int64_t n, int iters, float eps, hipStream_t s);

// Stream counts other than four (hc_general.hip): 1 <= hc <= kGenMaxHC.
constexpr int kGenMaxHC = 8;
bool gen_hc(int hc);
// Workspace of the fused call: the projection's partial sums, the mixes,
// pre (gen_ws_min_bytes, what a call needs), then the weights split once
// (gen_ws_bytes: with them, for calls long enough to use them).
size_t gen_ws_min_bytes(int64_t n, int hc, int d);
size_t gen_ws_bytes(int64_t n, int hc, int d);
int launch_gen_mixes(const void* R, const float* W, float* mixes, int64_t n, int hc, int d, float norm_eps,
                     hipStream_t s);
int launch_gen_split(const float* mixes, const float* scale, const float* base, float* pre, float* post,
                     float* comb, int64_t n, int hc, int iters, float eps, hipStream_t s);
int launch_gen_pre(const void* R, const float* pre, void* h, int64_t n, int hc, int d, hipStream_t s);
int launch_gen_post(const void* x, const void* R, const float* post, const float* comb, void* Rout, int64_t n,
                    int hc, int d, hipStream_t s);
// mixes, split + Sinkhorn and hc_pre in sequence; mixes and pre may be NULL
// (kept in ws, of gen_ws_bytes).
int launch_gen_fused(const void* R, const float* W, const float* scale, const float* base, void* h, float* pre,
                     float* post, float* comb, float* mixes, void* ws, size_t ws_bytes, int64_t n, int hc, int d,
                     int iters, float eps, float norm_eps, hipStream_t s);

// Work split of the projection kernels (hc_coop.hip): each group of G
// workgroups shares every token; member q owns a 32*KS-feature slice of
// each stream and its 24-column slice of the weights.
struct CoopPlan {
    int KS;          // 8-feature MFMA k-steps per wave (slice = 4 waves * 8 * KS features)
    int G;           // members per group (d / (32 * KS))
    int TM;          // 16-token MFMA tiles per round (T = 16 * TM tokens)
    int NG;          // groups (workgroups launched = G * NG)
    int64_t ntiles;  // ceil(n / T)
    size_t ws_part;  // byte offsets into the workspace: exchange records
    size_t ws_mix;   // mixes of every token when the caller does not keep them
    size_t ws_bytes;
    bool two_pass;   // short run: k_part + k_fin instead of the persistent kernel
    int splits;      // two-pass: column parts of h per block of 4 tokens
    bool gate;       // order persistent launches across streams (off for the no-alloc call)
};
// K-steps per wave for d (0: d cannot be tiled).  Host only, no HIP calls.
int coop_ks(int d);
// Returns false if d cannot be tiled (d % 32 != 0 or no KS in 1..8 gives G <= 32).
bool coop_plan(int64_t n, int d, CoopPlan& p);
// hc_post of the previous sublayer, run ahead of the projection
// (hc_post_mix_pre): R' = hc_post(x, R, post, comb) goes to Rout, and the
// projection, pre and h are those of R'.  R is the argument `R` of
// launch_coop.
struct PostIn {
    const void* x;
    const float* post;
    const float* comb;
    void* Rout;
};
// Wp: the weights already split by launch_pack (widths the wave-specialised
// kernel serves only), or null to split W in each call.
int launch_coop(const CoopPlan& p, const void* R, const float* W, const float* scale, const float* base,
                void* h, float* pre, float* post, float* comb, float* mixes, void* ws, int64_t n, int d,
                int iters, float eps, float norm_eps, bool fused, hipStream_t s, const PostIn* prev = nullptr,
                const void* Wp = nullptr);
// Host status of a workspace's header: 1 if a call on it gave up since the
// last clear (then cleared if `clear`), 0 if not, -1 if the header could not
// be read.  Synchronous (copies the header to the host).
int ws_status(const void* ws, bool clear);
// Diagnostics: the next `calls` persistent-kernel launches of this thread
// give up at their first exchange wait.
void set_force_timeout(int calls);
// Device address of this device's static scratch (hc_api.hip), or null.
void* scratch_ptr();

// Backward pass, four streams (hc_backward.hip).
bool bwd_supported(int hc, int d, int iters);
size_t bwd_ws_bytes(int64_t n, int d);
int launch_post_bwd(const void* x, const void* R, const float* post, const float* comb, const void* gRo, void* gx,
                    float* gpost, float* gcomb, int64_t n, int d, hipStream_t s);
int launch_mix_pre_bwd(const void* R, const float* W, const float* scale, const float* base, const float* mixes,
                       const void* gh, const void* gRo, const float* gpost, const float* gcomb, void* gR, float* gW,
                       float* gscale, float* gbase, float* gmixes, void* ws, int64_t n, int d, int iters, float eps,
                       float norm_eps, hipStream_t s);

// Bytes of packed weights for width d (0: d is not served by the
// wave-specialised kernels), and the packing launch.
size_t packed_weights_bytes(int d);
int launch_pack(const float* W, void* out, int d, hipStream_t s);

}  // namespace hc
