/*
 * hc.h -- libhc: hyper-connection residual-stream mixing on MI355X (gfx950).
 *
 * Every token carries hc = 4 parallel copies ("streams") of a d-wide bf16
 * residual.  For each sublayer the library
 *   1. projects the flattened 4d stream to (2+hc)*hc = 24 mix numbers and
 *      divides them by the stream's root mean square          (hc_mixes),
 *   2. turns the mixes into read weights pre, write weights post and a
 *      4x4 combination matrix comb made nearly doubly stochastic by an
 *      epsilon-Sinkhorn iteration                            (hc_split_sinkhorn),
 *   3. collapses the streams into the sublayer input          (hc_pre),
 *   4. expands the sublayer output back into four streams     (hc_post),
 * and offers steps 1-3 as one fused call (hc_fused_mix_pre).
 *
 * Sources (the pages' titles and the parts of them that define each call):
 *   "DeepSeek V4.1 - Mix projection": the mix formula (RMS over all hc*d
 *     features, eps 1e-20, float32) and the Block.hc_mixes / hc_pre /
 *     hc_post listing;
 *   "DeepSeek V4.1 - Reading weights": the learned-pre formula and the
 *     hc_split_sinkhorn kernel listing and its Python wrapper;
 *   "DeepSeek V4.1 attention": config.json (hc_mult 4, hc_sinkhorn_iters
 *     20, hc_eps 1e-6, norm_eps 1e-20, dim 5120).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers are device pointers on the current HIP device, except where a
 * comment says otherwise.  bf16 tensors are passed as `const void *` / `void *`
 * holding 16-bit bf16 patterns.  All tensors are dense row-major:
 *   R      bf16 [n][hc][d]     residual; element (k, c) of token t at
 *                              (t*hc + k)*d + c (stream-major flattening)
 *   x, h   bf16 [n][d]         sublayer output / sublayer input
 *   hc_fn  fp32 [24][hc*d]     mix projection weights (row j, column k*d + c)
 *   hc_scale fp32 [3]          scales for pre, post, comb (in that order)
 *   hc_base  fp32 [24]         offsets, indexed like the mixes
 *   mixes  fp32 [n][24]        [0,4) pre logits, [4,8) post, [8,24) comb
 *                              logits row-major (j*4 + k)
 *   pre, post fp32 [n][hc];  comb fp32 [n][hc][hc] with comb[j][k] at j*hc + k
 * n = B*T tokens (the caller flattens batch and sequence).
 *
 * Stream counts: hc is 1..8.  The shapes above are those of hc = 4, the
 * model's hc_mult; for another hc there are M = (2+hc)*hc mixes in place of
 * 24 (hc_fn [M][hc*d], hc_base [M], mixes [n][M] with [0,hc) pre logits,
 * [hc,2hc) post logits and [2hc,M) comb logits at 2hc + j*hc + k), as the
 * split + Sinkhorn listing of the "Reading weights" page and the mix
 * formula of the "Mix projection" page are written for any hc.  hc = 4 runs
 * the tuned kernels each entry point describes.  Every other count runs the
 * projection on the matrix cores: tiles of tokens over the whole flattened
 * stream, the fp32 weights split exactly into three bf16 pieces so every
 * product is that of fp32 arithmetic, fp32 sums over 8 fixed segments of
 * the reduction axis added in order (so a token's mixes do not depend on
 * the size of its call); then the split + Sinkhorn with the four-stream
 * arithmetic, then hc_pre / hc_post rounded once as below.
 * There the projection needs only d % 8 == 0, hc_mixes uses no workspace
 * (it may be NULL), and the fused calls' workspace holds the projection's
 * per-segment partial sums and the mixes and pre of every token
 * (hc_fused_workspace_bytes).  The packed-weight calls take hc = 4 only.
 *
 * Ownership: the caller owns every buffer.  The library never allocates,
 * frees or synchronises; each call enqueues its kernels on `stream` (a
 * hipStream_t; NULL is the default stream) and returns.  Errors found by
 * the host-side checks are returned before any HIP call is made; device
 * faults surface at the caller's next synchronisation.  n == 0 returns
 * HC_OK without launching anything.
 *
 * Alignment: every tensor pointer must be 16-byte aligned, except hc_scale
 * and hc_base (4-byte).  Outputs must not overlap inputs or each other,
 * except where an entry point says so.
 *
 * Numerics: mixes, pre, post and comb are computed in float32 (the pages'
 * precision).  Every bf16 output (h, R') is the correctly rounded
 * (nearest-even) value of its defining sum of products of the given fp32
 * coefficients and bf16 inputs: the kernels accumulate in double, where
 * those products are exact, and round once.
 */
#ifndef LIBHC_HC_H
#define LIBHC_HC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum hc_status {
    HC_OK = 0,
    HC_ERR_NULL = -1,        /* a required pointer is NULL */
    HC_ERR_SHAPE = -2,       /* n < 0, d <= 0, d % 8 != 0, or sizes overflow */
    HC_ERR_ALIGN = -3,       /* a pointer is not suitably aligned */
    HC_ERR_UNSUPPORTED = -4, /* hc outside 1..8 (hc != 4 for the packed
                                weights), sinkhorn_iters < 1, or a d the
                                four-stream projection cannot tile */
    HC_ERR_WORKSPACE = -5,   /* workspace missing or too small */
    HC_ERR_ALIAS = -6,       /* an output overlaps an input or another output */
    HC_ERR_VALUE = -7,       /* an epsilon is negative or not finite */
    HC_ERR_LAUNCH = -8,      /* the HIP runtime refused a launch */
    HC_ERR_DEVICE = -9,      /* device query failed (no device, bad id) */
    HC_ERR_TIMEOUT = -10,    /* hc_workspace_status: a call on the workspace
                                stopped early (a bounded wait between
                                workgroups gave up); its outputs are undefined */
    HC_ERR_SCRATCH = -11     /* hc_fused_mix_pre_noalloc: the call needs more
                                workspace than the static scratch holds */
} hc_status;

/* Human-readable name of a status code (static string, never NULL). */
const char *hc_status_str(int status);

/* Library version as "major.minor.patch" (static string). */
const char *hc_version(void);

/*
 * hc_mixes -- "Mix projection" page, the mix formula and Block.hc_mixes:
 *   r_t = 1 / sqrt( sum_i R[t][i]^2 / (hc*d) + norm_eps )
 *   mixes[t][j] = r_t * sum_i R[t][i] * hc_fn[j][i],   i over the hc*d
 *   flattened features, j < 24.
 * The library's hc_mixes stops at the mixes; the pages' Block.hc_mixes
 * also runs the split (call hc_split_sinkhorn, or hc_fused_mix_pre).
 * With hc = 4 it requires d % 32 == 0 and d / (32*k) <= 64 for some k in 1..5 (d = 5120:
 * k = 5, 32 workgroups per token group); otherwise HC_ERR_UNSUPPORTED.
 * hc_fn is used as given, fp32, with no precision reduced: each product is
 * formed exactly from a three-way bf16 split of the weight.
 *
 * Workspace: device memory of at least hc_fused_workspace_bytes(n, hc, d)
 * bytes, 256-byte aligned.  It holds the partial sums the workgroups of a
 * token group exchange, and a small header in its first 256 bytes.  Calls
 * are numbered by a process-wide counter in the library; the number tags
 * every partial sum, so that a record left by an earlier call is never
 * taken for a current one, and the header records which call last
 * prepared the workspace.  Any contents are accepted on first use.  Between
 * calls, leave it alone (or zero its first 256 bytes after using it for
 * something else).  Calls that may run at the same time, on different
 * streams, each need their own workspace.
 *
 * Calls of more than 2,048 tokens (and every call at widths outside the
 * d = 5120 family) run one ordinary launch of at most one workgroup per
 * compute unit, in groups of G workgroups (one XCD's worth at d = 5120)
 * that wait for each other's partial sums; a group starts once all of its
 * members are resident, and no workgroup waits for one outside its group.
 * The library orders these launches across streams: within one process, a
 * launch on another stream than the previous one on the same device first
 * waits (a HIP event) for that one to finish, so two such grids never
 * compete for the compute units (the no-alloc call below is not ordered).
 * Every wait is bounded: a member that is not resident within about two
 * seconds (say, while long-running work of another process holds compute
 * units), or a peer that stops, makes the call stop early; its outputs are
 * then undefined, and hc_workspace_status reports it.  Shorter calls at widths d = 32*k*G with
 * 8 <= G <= 32 (d = 5120 among them) run two ordinary launches with no
 * waits between workgroups: the partial sums go through the workspace.
 * Both give bitwise the same results for a token, so a token's mixes do not
 * depend on how many tokens share its call.
 */
int hc_mixes(const void *R, const float *hc_fn, float *mixes, int64_t n,
             int32_t hc, int32_t d, float norm_eps, void *workspace,
             size_t workspace_bytes, void *stream);

/*
 * hc_split_sinkhorn -- "Reading weights" page, the hc_split_sinkhorn kernel
 * listing (and the learned-pre formula, whose s_1 is hc_scale[0]):
 *   pre[t][j]  = sigmoid(hc_scale[0]*mixes[t][j] + hc_base[j]) + hc_eps
 *   post[t][j] = 2*sigmoid(hc_scale[1]*mixes[t][4+j] + hc_base[4+j])
 *   L[j][k]    = hc_scale[2]*mixes[t][8+4j+k] + hc_base[8+4j+k]
 *   comb = row softmax of L, + hc_eps; comb /= (column sums + hc_eps);
 *   then (sinkhorn_iters - 1) times: comb /= (row sums + hc_eps);
 *   comb /= (column sums + hc_eps).
 * sinkhorn_iters >= 1 (else HC_ERR_UNSUPPORTED); hc_eps finite and >= 0.
 * The pages' wrapper allocates its outputs; here the caller does.
 */
int hc_split_sinkhorn(const float *mixes, const float *hc_scale,
                      const float *hc_base, float *pre, float *post,
                      float *comb, int64_t n, int32_t hc,
                      int32_t sinkhorn_iters, float hc_eps, void *stream);

/*
 * hc_pre -- "Mix projection" page, Block.hc_pre:
 *   h[t][c] = bf16( sum_k pre[t][k] * R[t][k][c] ).
 * d % 8 == 0.  h must not overlap R or pre.
 */
int hc_pre(const void *R, const float *pre, void *h, int64_t n, int32_t hc,
           int32_t d, void *stream);

/*
 * hc_rmsnorm -- the pre-sublayer RMSNorm ("Mix projection" page,
 * Block.__init__ builds RMSNorm(dim, norm_eps); its formula is not printed
 * and is read as the page's mix-formula normalisation over the d features,
 * times a per-feature weight):
 *   y[t][c] = bf16( h[t][c] * r[t] * gamma[c] ),
 *   r[t] = 1 / sqrt( sum_c h[t][c]^2 / d + norm_eps ).
 * h, y: bf16 [n][d]; gamma: fp32 [d].  The sum of squares, r and the
 * products are taken in double and y is rounded once (nearest-even), so y
 * is the correctly rounded result up to the order of the sum of squares.
 * d % 8 == 0 and d <= 32,768 (wider: HC_ERR_UNSUPPORTED); norm_eps finite
 * and >= 0 (HC_ERR_VALUE); y must not overlap h or gamma (HC_ERR_ALIAS).
 * All pointers 16-byte aligned.  Asynchronous on `stream`; no workspace.
 */
int hc_rmsnorm(const void *h, const float *gamma, void *y, int64_t n,
               int32_t d, float norm_eps, void *stream);

/*
 * hc_pre_norm -- hc_pre followed by hc_rmsnorm in one pass over R:
 *   h = hc_pre(R, pre) (bitwise hc_pre's result), y = hc_rmsnorm(h, gamma).
 * h may be NULL (then only y is written: R is read once and y written once,
 * 2 (hc + 1) d bytes per token).  Shapes and rules as hc_pre and
 * hc_rmsnorm; no output may overlap an input or the other output.
 */
int hc_pre_norm(const void *R, const float *pre, const float *gamma, void *h,
                void *y, int64_t n, int32_t hc, int32_t d, float norm_eps,
                void *stream);

/*
 * hc_post -- "Mix projection" page, Block.hc_post:
 *   R_out[t][k][c] = bf16( post[t][k] * x[t][c]
 *                          + sum_j comb[t][j][k] * R[t][j][c] )
 * (column k of comb feeds output stream k).  d % 8 == 0.  R_out == R is
 * allowed (in place); any other overlap of R_out with an input is
 * HC_ERR_ALIAS.
 */
int hc_post(const void *x, const void *R, const float *post,
            const float *comb, void *R_out, int64_t n, int32_t hc, int32_t d,
            void *stream);

/*
 * hc_fused_mix_pre -- hc_mixes, hc_split_sinkhorn and hc_pre in one pass
 * over the residual (the sequence of Block.hc_mixes followed by
 * Block.hc_pre on the "Mix projection" page).  Outputs: h (required),
 * post and comb (required), pre and mixes (each may be NULL; with mixes
 * NULL they are kept in the workspace).  Same constraints on d as
 * hc_mixes; the same workspace rules.  The coefficients are bitwise those
 * of hc_mixes followed by hc_split_sinkhorn, and h is bitwise hc_pre's for
 * those coefficients.  Launches two kernels on `stream`: the projection
 * with pre and h, then the split of post and comb (calls of more than
 * 2,048 tokens), or the partial sums, then their reduction with the split
 * and h (shorter calls); widths outside the d = 5120 family add a workspace
 * header update before the projection.
 */
int hc_fused_mix_pre(const void *R, const float *hc_fn,
                     const float *hc_scale, const float *hc_base, void *h,
                     float *pre, float *post, float *comb, float *mixes,
                     void *workspace, size_t workspace_bytes, int64_t n,
                     int32_t hc, int32_t d, int32_t sinkhorn_iters,
                     float hc_eps, float norm_eps, void *stream);

/*
 * hc_fused_mix_pre_norm -- hc_fused_mix_pre followed by the pre-sublayer
 * RMSNorm of its h (hc_rmsnorm; the norm is a reading of the "Mix
 * projection" page, whose Block.__init__ builds RMSNorm(dim, norm_eps) but
 * prints no formula):  y = bf16(h * r * gamma),
 * r = 1 / sqrt(sum_c h_c^2 / d + norm_eps), per token.
 * Arguments as hc_fused_mix_pre, plus gamma (fp32 [d]) and y (bf16 [n][d],
 * required); h may be NULL (then it is not written).  The coefficients and
 * h are bitwise hc_fused_mix_pre's; y is hc_rmsnorm's result for that h
 * (within one bf16 ulp of the correctly rounded norm: only the order of
 * the double sum of squares is free).  Same workspace
 * (hc_fused_workspace_bytes).  Runs hc_fused_mix_pre's kernels, writing h
 * to h (or, when h is NULL, to y), and then the norm kernel (in place on
 * y when h is NULL).  d <= 32,768 (else HC_ERR_UNSUPPORTED); y must not
 * overlap any input or output, gamma no output.
 */
int hc_fused_mix_pre_norm(const void *R, const float *hc_fn,
                          const float *hc_scale, const float *hc_base,
                          const float *gamma, void *h, void *y, float *pre,
                          float *post, float *comb, float *mixes,
                          void *workspace, size_t workspace_bytes, int64_t n,
                          int32_t hc, int32_t d, int32_t sinkhorn_iters,
                          float hc_eps, float norm_eps, void *stream);

/*
 * hc_post_mix_pre -- one sublayer boundary: hc_post of sublayer l, then
 * hc_fused_mix_pre of sublayer l+1 on its output ("Mix projection" page,
 * Block.hc_post followed by Block.hc_mixes and Block.hc_pre; the coefficients
 * a sublayer computes are used by the next one, as that page's docstring
 * puts it):
 *   R_out = hc_post(x, R, post, comb)                       (sublayer l)
 *   (h, pre_next, post_next, comb_next, mixes_next)
 *         = hc_fused_mix_pre(R_out, hc_fn, hc_scale, hc_base)  (sublayer l+1)
 * x, R, post, comb as for hc_post; hc_fn, hc_scale, hc_base and the outputs
 * as for hc_fused_mix_pre (pre_next and mixes_next may be NULL).  Results
 * are bitwise those of the two calls in sequence.  R_out == R is allowed
 * (the residual updated in place); R_out must not otherwise overlap R, and
 * no output may overlap an input or another output.  Same constraints on d
 * and the same workspace (hc_fused_workspace_bytes) as hc_fused_mix_pre.
 * Calls of more than 2,048 tokens at the widths of the wave-specialised
 * projection (d = 32*k*G, 8 <= G <= 32, d = 5120 among them) run one pass
 * over R: the projection kernel forms R' from each round of R on its way
 * through on-chip memory, writes it to R_out and projects it, so R is read
 * once for hc_post, the mixes and h.  Other calls run hc_post's kernel and
 * then hc_fused_mix_pre's kernels on `stream`.
 */
int hc_post_mix_pre(const void *x, const void *R, const float *post,
                    const float *comb, void *R_out, const float *hc_fn,
                    const float *hc_scale, const float *hc_base, void *h,
                    float *pre_next, float *post_next, float *comb_next,
                    float *mixes_next, void *workspace, size_t workspace_bytes,
                    int64_t n, int32_t hc, int32_t d, int32_t sinkhorn_iters,
                    float hc_eps, float norm_eps, void *stream);

/*
 * Weight packing, for callers that run one weight set many times (a model's
 * layers at inference).  It computes nothing of the method: it re-arranges
 * hc_fn, the projection weights of the "Mix projection" page's mix formula
 * (float32), for the kernels.  The projection uses each fp32 weight as three
 * bf16 pieces (hi + mid + lo, exactly); hc_pack_weights forms those pieces
 * once, in the register layout of the projection kernels, and
 * hc_fused_mix_pre_packed then loads them instead of forming them in every
 * call.  Results are bitwise those of hc_fused_mix_pre with the same hc_fn.
 * Only widths d = 32*k*G with 8 <= G <= 32 (d = 5120 among them) have a
 * packed form; other widths return HC_ERR_UNSUPPORTED.  The packed buffer
 * is owned by the caller, device memory, 16-byte aligned, and must be
 * packed again whenever hc_fn changes.
 *
 * hc_packed_weights_bytes: bytes of the packed form for d (0 if none;
 *   3,276,800 at d = 5120).  Host-only query.
 * hc_pack_weights: packed <- pieces of hc_fn (fp32 [24][hc*d]); enqueued on
 *   `stream`.  HC_ERR_WORKSPACE if packed_bytes is too small.
 * hc_fused_mix_pre_packed: hc_fused_mix_pre with `packed` in place of
 *   hc_fn; all other arguments and rules as there.  HC_ERR_WORKSPACE if
 *   packed_bytes is smaller than hc_packed_weights_bytes(hc, d).
 */
size_t hc_packed_weights_bytes(int32_t hc, int32_t d);

int hc_pack_weights(const float *hc_fn, void *packed, size_t packed_bytes,
                    int32_t hc, int32_t d, void *stream);

int hc_fused_mix_pre_packed(const void *R, const void *packed,
                            size_t packed_bytes, const float *hc_scale,
                            const float *hc_base, void *h, float *pre,
                            float *post, float *comb, float *mixes,
                            void *workspace, size_t workspace_bytes, int64_t n,
                            int32_t hc, int32_t d, int32_t sinkhorn_iters,
                            float hc_eps, float norm_eps, void *stream);

/*
 * Backward pass (training).  The pages give the forward; these return the
 * gradient of a scalar loss L through it, by the chain rule over the
 * forward's steps in reverse order, on the real-valued forward (the bf16
 * roundings of h and R' are storage, not steps).  Four streams only
 * (hc != 4: HC_ERR_UNSUPPORTED).  In a model's backward, a sublayer runs
 * hc_post_backward first (its dL/dx feeds the sublayer's own backward,
 * which yields dL/dh), then hc_mix_pre_backward.
 *
 * hc_post_backward -- the gradient through Block.hc_post ("Mix projection"
 * page), from gRout = dL/dR' (bf16 [n][4][d]):
 *   gx[t][c]       = bf16( sum_k post_k gRout[t][k][c] )  (correctly rounded)
 *   gpost[t][k]    = sum_c x[t][c] gRout[t][k][c]          (fp32 [n][4])
 *   gcomb[t][j][k] = sum_c R[t][j][c] gRout[t][k][c]       (fp32 [n][4][4])
 * The sums over c are accumulated in double and rounded once to float.
 * d % 8 == 0.  No output may overlap an input or another output.
 */
int hc_post_backward(const void *x, const void *R, const float *post,
                     const float *comb, const void *gRout, void *gx,
                     float *gpost, float *gcomb, int64_t n, int32_t hc,
                     int32_t d, void *stream);

/*
 * hc_mix_pre_backward -- the rest of the sublayer's gradient: through
 * Block.hc_pre, the split + epsilon-Sinkhorn ("Reading weights" listing) and
 * the mix formula, plus hc_post's share of dL/dR.  Inputs: the forward's
 * R, hc_fn, hc_scale, hc_base and its mixes (fp32 [n][24], from hc_mixes or
 * hc_fused_mix_pre); gh = dL/dh (bf16 [n][d]); gRout = dL/dR' and gpost,
 * gcomb from hc_post_backward.  Outputs:
 *   gR       bf16 [n][4][d]: dL/dR = sum_k comb[j][k] gRout_k + pre_j gh
 *            + sum_m gdot_m hc_fn[m][j*d + c] + 2 R[j][c] gss, in float,
 *            rounded once; pre and comb are recomputed from the mixes with
 *            the forward's arithmetic (bitwise the forward's), gdot = r dL/dm
 *            and gss = -(r^2 / 2K) sum_m dL/dm_m m_m with r the forward's
 *            RMS normaliser (K = 4d);
 *   g_hc_fn  fp32 [24][4d]: dL/dhc_fn = sum_t gdot[t][m] R[t][i];
 *   g_hc_scale fp32 [3], g_hc_base fp32 [24]: sums over tokens;
 *   gmixes   fp32 [n][24], dL/dmixes (may be NULL).
 * The split + Sinkhorn backward replays the forward's steps in float,
 * keeping every step, and runs them backwards; sums over tokens are added
 * in one fixed order, so results are deterministic.  Requires d % 128 == 0
 * and 1 <= sinkhorn_iters <= 64.  Workspace: hc_backward_workspace_bytes
 * (n, hc, d) bytes, 256-byte aligned (per-token coefficients and partial
 * sums of dL/dhc_fn; about 190 B per token plus up to 32 x 24 x 4d floats).
 * With n == 0 nothing is launched and nothing is written.
 */
int hc_mix_pre_backward(const void *R, const float *hc_fn,
                        const float *hc_scale, const float *hc_base,
                        const float *mixes, const void *gh, const void *gRout,
                        const float *gpost, const float *gcomb, void *gR,
                        float *g_hc_fn, float *g_hc_scale, float *g_hc_base,
                        float *gmixes, void *workspace, size_t workspace_bytes,
                        int64_t n, int32_t hc, int32_t d,
                        int32_t sinkhorn_iters, float hc_eps, float norm_eps,
                        void *stream);

/* Workspace bytes of hc_mix_pre_backward (0 for n == 0 or an unsupported
 * shape).  Host-only query. */
size_t hc_backward_workspace_bytes(int64_t n, int32_t hc, int32_t d);

/*
 * hc_workspace_status -- whether a call on this workspace stopped early.
 * A call that gives up a bounded wait (see hc_mixes) sets a word in the
 * workspace header that stays set until this query clears it.  Call it
 * after synchronising with the calls in question (it copies the header to
 * the host with a synchronous hipMemcpy -- the one call in this library
 * that synchronises).  Returns HC_OK (no call gave up, or the workspace
 * was never used by the calls that wait), HC_ERR_TIMEOUT (some call gave
 * up since the last clear; with clear != 0 the word is reset), or
 * HC_ERR_NULL / HC_ERR_ALIGN / HC_ERR_WORKSPACE (bytes < 256) /
 * HC_ERR_DEVICE (the header could not be read).
 * hc_noalloc_status: the same for this device's static scratch of
 * hc_fused_mix_pre_noalloc.
 */
int hc_workspace_status(const void *workspace, size_t workspace_bytes,
                        int clear);
int hc_noalloc_status(int clear);

/*
 * hc_phase_trace -- diagnostics: where the persistent projection kernel of
 * hc_fused_mix_pre / hc_mixes / hc_post_mix_pre (the wave-specialised
 * kernel, calls of more than 2,048 tokens at d = 5120) spends its time.
 * Only a library built with phase tracing (`python -m
 * hyper_connection_residual_02_amd.build --phase-trace`, libhc_trace.so)
 * records it; every other build returns HC_ERR_UNSUPPORTED.  Copies, after
 * the caller's synchronisation, up to `count` words of the last launch's
 * tables to the host array `out`: per workgroup (block index b, up to
 * 1,024) and per wave (8), 7 words -- the s_memrealtime ticks (100 MHz)
 * spent in phases 0..5, then the number of ticks of the round loop; then,
 * after those 1,024 x 8 x 7 words, 4 words per workgroup -- the clock
 * (s_memrealtime, common to all compute units) at the workgroup's entry, at
 * the end of its start-up protocol, at the start of its round loop (after
 * its weights and first residual loads) and at its end.
 * Phases, MFMA waves 0..3: 0 the tick's barrier, 1 publishing partial
 * sums, 2 issuing the residual loads, 3 products, 4 waiting for the next
 * round's loads, 5 (hc_post_mix_pre) hc_post of the next round; exchange
 * waves 4..7: 0 barrier, 1 exchange (record waits, member sums, pre, the
 * owned token's mixes), 2 h, 3 residual copy, 4 issuing the next record
 * loads, 5 (hc_post_mix_pre) R' stores.  A workgroup's words are those of
 * the last launch that ran it.  Returns the number of words copied, or
 * HC_ERR_NULL (out NULL, count > 0) / HC_ERR_UNSUPPORTED.  Synchronous
 * (hipMemcpyFromSymbol).
 */
int hc_phase_trace(uint64_t *out, size_t count);

/*
 * hc_debug_force_timeout -- diagnostics for tests of the failure path:
 * the next `calls` launches of the waiting kernels (see hc_mixes) made by
 * the calling host thread take every exchanged partial sum for stale and
 * bound their waits to zero time, so each such call gives up at its first
 * exchange, its kernels exit normally, and hc_workspace_status reports
 * HC_ERR_TIMEOUT.  0 cancels.  HC_ERR_VALUE if calls < 0.
 */
int hc_debug_force_timeout(int calls);

/*
 * hc_fused_mix_pre_noalloc -- hc_fused_mix_pre for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, outputs, rules and
 * results (bitwise) as hc_fused_mix_pre, without the workspace arguments:
 * the workspace is a static device array of HC_SCRATCH_BYTES inside the
 * library, one per GPU, held until the process ends.  The call itself
 * allocates nothing and calls no allocating routine; its first call on a
 * device looks up that device's copy of the array (hipGetSymbolAddress).
 *
 * Limit: a call whose workspace (hc_fused_workspace_bytes(n, hc, d)) would
 * exceed HC_SCRATCH_BYTES returns HC_ERR_SCRATCH before any launch
 * (at hc = 4, d = 5120 every call of up to 125,608 tokens fits).  The array
 * keeps the last call's contents, which the
 * workspace header makes harmless to the next call.  Every call on one GPU
 * shares that GPU's array: calls that may overlap in time on one GPU (on
 * different streams, or from different threads) race and must not be made;
 * use hc_fused_mix_pre with a workspace of their own instead.
 */
#define HC_SCRATCH_BYTES ((size_t)16 << 20)

int hc_fused_mix_pre_noalloc(const void *R, const float *hc_fn,
                             const float *hc_scale, const float *hc_base,
                             void *h, float *pre, float *post, float *comb,
                             float *mixes, int64_t n, int32_t hc, int32_t d,
                             int32_t sinkhorn_iters, float hc_eps,
                             float norm_eps, void *stream);

/*
 * hc_probe_stream -- a measurement probe, not a step of the method: a plain
 * HBM stream with the access pattern of the library's streaming kernels
 * (16-byte non-temporal accesses, two in flight per lane) on wg_per_cu
 * workgroups of 256 lanes per compute unit (0: two, as the streaming
 * kernels use on long runs; at most 32, else HC_ERR_VALUE).  dst non-NULL:
 * copies `bytes` from src to dst; dst NULL: reads src only.  It gives the
 * copy and read rates the kernels' roofline fractions are compared with.
 * bytes % 16 == 0 (else HC_ERR_SHAPE); src, dst 16-byte aligned; dst must
 * not overlap src.  Asynchronous on `stream`.
 */
int hc_probe_stream(const void *src, void *dst, size_t bytes,
                    int32_t wg_per_cu, void *stream);

/* HC_SCRATCH_BYTES, the static scratch of hc_fused_mix_pre_noalloc (host only). */
size_t hc_scratch_bytes(void);

/*
 * Bytes of device workspace hc_mixes / hc_fused_mix_pre need for these
 * sizes on the current device (0 for n == 0; 0 with an unsupported shape,
 * in which case the call itself reports the error).  Host-only query.
 */
size_t hc_fused_workspace_bytes(int64_t n, int32_t hc, int32_t d);

/*
 * hc_diag_scale -- the chained-stack workload's stand-in sublayer:
 *   x[t][c] = bf16( h[t][c] * D[c] ),  D bf16 [d].
 * A fixed per-layer diagonal scale between hc_pre and hc_post, so that an
 * 80-sublayer stack can run without trained attention/FFN weights.
 * d % 8 == 0; x must not overlap h or D.
 */
int hc_diag_scale(const void *h, const void *D, void *x, int64_t n,
                  int32_t d, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBHC_HC_H */
