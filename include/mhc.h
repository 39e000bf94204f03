/*
 * mhc.h -- C ABI of libmhc, the MI355X (gfx950) implementation of the
 * Single-Pass mHC residual step: tuned kernels for n = 4 residual streams and
 * a general family (the *_n entry points) for n in {2, 4, 8}.
 *
 * Pages this interface follows (cited by title and section):
 *   [SW] "DeepSeek V4.1 · Stream weights for the feed-forward": the formula list
 *        "All 5 steps", the "Why" paragraph (traffic of the fused single pass)
 *        and the Code excerpts hc_mixes, hc_pre, hc_post and the split/Sinkhorn
 *        kernel with its wrapper.
 *   [RN] "DeepSeek V4.1 · MoE RMSNorm": the RMSNorm formula and the Code
 *        excerpts RMSNorm and Block.forward.
 *
 * Conventions shared by every entry point
 *   - All data pointers are DEVICE pointers, contiguous, row-major, and must be
 *     16-byte aligned. The caller owns all memory and the library allocates
 *     none. Its only state is a per-device cache of two device attributes
 *     (compute-unit count, cooperative-launch support), filled on first use
 *     with atomic stores, so calls from several host threads are safe; the
 *     per-thread detail of mhc_last_error() is the other.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *     and the call returns without synchronising.
 *   - `dtype` (an mhc_dtype value) is the dtype of the stream tensors x, f,
 *     x_out and y_out. Coefficients, mixes and all parameters are float32.
 *   - Layouts: x [T][4][d]; f [T][d]; pre, post [T][4]; comb [T][4][4] indexed
 *     [j][k]; mixes [T][24] with slots 0-3 pre, 4-7 post, 8+4j+k comb; w_mix
 *     float32 [24][4*d] whose column k*d+f multiplies stream k, feature f.
 *   - Errors: argument problems return MHC_ERR_INVALID_ARG and configurations
 *     the kernels do not cover return MHC_ERR_UNSUPPORTED, both before any
 *     launch (the argument checks come before any HIP call; choosing a kernel
 *     family may query the device's attributes, whose failure is
 *     MHC_ERR_HIP). A failing HIP launch returns MHC_ERR_HIP. mhc_last_error() then
 *     describes the failure (per calling thread). tokens == 0 returns MHC_OK
 *     after the scalar checks, without examining pointers and without
 *     launching anything. NaN/Inf in the data propagate; they are not
 *     detected.
 *   - Outputs must not overlap each other or any input, except that x_out may
 *     be exactly x (in-place stream update).
 */
#ifndef MHC_H
#define MHC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MHC_ABI_VERSION 11
#define MHC_N_STREAMS 4
#define MHC_N_MIX 24

typedef enum mhc_status {
  MHC_OK = 0,
  MHC_ERR_INVALID_ARG = 1,
  MHC_ERR_UNSUPPORTED = 2,
  MHC_ERR_HIP = 3
} mhc_status;

typedef enum mhc_dtype { MHC_F32 = 0, MHC_BF16 = 1 } mhc_dtype;

/*
 * Kernel family of mhc_fused_step and mhc_mixes:
 *   MHC_PATH_AUTO   no workspace: the tile kernel. With a workspace: the
 *                   chunked kernels up to 896 tokens (2048 with
 *                   MHC_PATH_COOPERATIVE) where they apply, else the
 *                   feature-split kernel where it applies, else the tile
 *                   kernel.
 *   MHC_PATH_TILE   the tile kernel (one workgroup per 16 tokens, no
 *                   workspace; the workspace argument is ignored).
 *   MHC_PATH_SPLIT  the feature-split kernel (needs a workspace;
 *                   MHC_ERR_UNSUPPORTED where it does not apply).
 *   MHC_PATH_CHUNK  the chunked kernels (needs a workspace;
 *                   MHC_ERR_UNSUPPORTED where they do not apply).
 * MHC_PATH_COOPERATIVE is a flag that may be OR-ed into any of them. It
 * changes how the feature-split kernel is launched and nothing else. That
 * kernel runs one workgroup per compute unit (at most the device's count) in
 * groups of ns workgroups that wait for one another. By default it is an
 * ordinary launch: each workgroup takes its place in start order from a
 * counter in the workspace, and groups are filled in that order, so only the
 * one group still being filled can be waiting; every other group runs to its
 * end and frees its compute units. The call therefore completes whenever the
 * device can eventually hold one group (ns compute units, 20 at d = 5120) of
 * it at once: kernels running alongside only delay it, and two calls in
 * flight on two streams both finish. It cannot complete if other work holds
 * all but fewer than ns compute units for good (a CU mask on the stream that
 * leaves fewer than ns, a kernel elsewhere that waits for this call, or more
 * than (compute units)/(ns - 1) such calls in flight at once); then a wait
 * gives up after 2^20 polls, the workspace status word is set and the outputs
 * are invalid, as after any given-up wait. With MHC_PATH_COOPERATIVE the
 * kernel is launched cooperatively instead: the runtime runs it alone on the
 * device with all workgroups resident, and the device idles for about 11 us
 * before and after it (about 19 us per call issued back to back). With
 * MHC_PATH_AUTO the flag also raises the switch from the chunked kernels to
 * the feature-split kernel from 896 to 2048 tokens, since the split route's
 * fixed cost is then larger. mhc_fused_step_route reports that choice. The
 * n-family's switch is 2048 tokens either way. MHC_PATH_PLAIN_LAUNCH (the
 * ordinary launch, the default since ABI 11) is still accepted and changes
 * nothing; it may not be combined with MHC_PATH_COOPERATIVE.
 */
typedef enum mhc_path {
  MHC_PATH_AUTO = 0,
  MHC_PATH_TILE = 1,
  MHC_PATH_SPLIT = 2,
  MHC_PATH_CHUNK = 3,
  MHC_PATH_PLAIN_LAUNCH = 16,
  MHC_PATH_COOPERATIVE = 32
} mhc_path;

typedef void* mhc_stream_t;

/* Version of this ABI (MHC_ABI_VERSION). */
int32_t mhc_abi_version(void);

/* Static name of a status code; "unknown status" for other values. */
const char* mhc_status_string(int32_t status);

/* Detail of the last non-OK status returned to the calling thread ("" if none).
 * The string belongs to the library and stays valid until the next call. */
const char* mhc_last_error(void);

/* d must be a positive multiple of this many features (32). */
int32_t mhc_d_granule(void);

/* Bytes of the packed projection for width d and stream dtype, or -1 for a bad
 * d or dtype. */
int64_t mhc_wmix_packed_bytes(int32_t d, int32_t dtype);

/*
 * mhc_pack_wmix -- lay the float32 mix projection W [24][4*d] ([SW] Code,
 * hc_mixes: the weight of F.linear; "All 5 steps": W_mix) out in the operand
 * order of the gfx950 matrix instructions the step kernels use.
 *   - MHC_BF16: every weight is split into three bfloat16 terms hi + mid + lo
 *     whose sum is the float32 weight exactly; the 72 terms per column are
 *     padded to 80 rows.
 *   - MHC_F32: float32 copy, rows padded to 32.
 * The packed buffer depends only on (W, d, dtype): pack once per weight and
 * reuse it for every call of mhc_fused_step / mhc_mixes with that dtype.
 * w_packed must hold mhc_wmix_packed_bytes(d, dtype) bytes (packed_bytes is
 * the caller's buffer size, checked).
 */
mhc_status mhc_pack_wmix(const float* w_mix, int32_t d, int32_t dtype, void* w_packed,
                         int64_t packed_bytes, mhc_stream_t stream);

/*
 * mhc_fused_step_workspace_bytes -- bytes of device workspace that
 * mhc_fused_step and mhc_mixes need to run either of their workspace kernel
 * families for these arguments on the current device (the larger of the two
 * needs; 0 when neither applies, and then only the tile kernel runs), -1 for
 * bad arguments or a failing HIP query (see mhc_last_error).
 *   - Feature-split kernel: MHC_BF16 streams whose width splits into ns
 *     slices of S features, ns in {32, 40, 48, 64} and S in {64, 96, 128, 160}
 *     (d = 2048 ... 10240), or S = 256 and 16 <= ns <= 24 (d a multiple of
 *     256 from 4096 to 6144; e.g. 5120 = 20 x 256, the geometry of large
 *     calls there), on a device with at least ns compute units and
 *     cooperative launch support. About 17 MB for d = 5120 on 256 CUs, plus
 *     96 bytes per token for the mixes rows. The 256-feature slices take
 *     the hi + mid terms of the packed projection (|w - hi - mid| <=
 *     2^-16 |w|), the others all three; a call with sinkhorn_iters == 1
 *     takes a three-term geometry where d has one (after a single round the
 *     comb's row sums are not normalised and would carry the two-term error).
 *   - Chunked kernels: at most 8192 tokens; MHC_BF16 streams with d a
 *     multiple of 64 up to 5120, or MHC_F32 streams. The 16,384-byte header
 *     plus 128 bytes per token and chunk, a chunk being 512 features (bf16)
 *     or 256 (f32): 1,280 or 2,560 bytes per token at d = 5120. On bf16
 *     streams they take the hi + mid terms of the packed projection when
 *     sinkhorn_iters >= 2 and all three for a single round.
 */
int64_t mhc_fused_step_workspace_bytes(int64_t tokens, int32_t d, int32_t dtype);

/*
 * mhc_fused_step_route -- the kernel family (MHC_PATH_TILE, MHC_PATH_SPLIT or
 * MHC_PATH_CHUNK) that mhc_fused_step and mhc_mixes run for `path`, these
 * arguments and a workspace given (with_workspace != 0) or not, on the current
 * device; -1 (see mhc_last_error) for bad arguments, a path that cannot run
 * them, or a failing HIP query.
 */
int32_t mhc_fused_step_route(int32_t path, int64_t tokens, int32_t d, int32_t dtype,
                             int32_t with_workspace);

/*
 * mhc_fused_step -- one Single-Pass mHC step at the boundary between sublayer
 * i and sublayer i+1, in one pass over the streams ([SW] "Why": the fused form
 * moves (2n+2)*d elements per token instead of (4n+4)*d; [RN] Code,
 * Block.forward: hc_post, then hc_mixes on the new streams, hc_pre with the
 * read weights of the previous sublayer, then the norm).
 *
 * Per token t, with S the stream dtype and every sum in float32:
 *   x_out[k] = S( sum_j comb_in[j][k] * x[j] + post_in[k] * f )      ([SW] Code, hc_post)
 *   r        = 1 / sqrt( mean over all 4*d of x_out^2 + norm_eps )
 *   mix      = r * (W . flatten(x_out))                              ([SW] Code, hc_mixes)
 *   pre_out, post_out, comb_out = split + Sinkhorn of mix            (as mhc_sinkhorn4)
 *   h        = S( sum_k pre_in[k] * x_out[k] )                       ([SW] Code, hc_pre)
 *   y_out    = S( gamma * (h / sqrt(mean(h^2) + norm_eps)) )         ([RN] RMSNorm)
 *
 * Inputs:  x [T][4][d] (streams entering sublayer i), f [T][d] (sublayer i
 *          output), pre_in/post_in/comb_in (coefficients sublayer i computed
 *          from x), w_packed (mhc_pack_wmix of sublayer i+1's W, same dtype),
 *          base [24], scale [3] (sublayer i+1), gamma [d] (sublayer i+1's
 *          RMSNorm gain), sinkhorn_iters >= 1, norm_eps >= 0, hc_eps >= 0.
 * Outputs: x_out [T][4][d] (may be x), y_out [T][d], pre_out/post_out
 *          [T][4], comb_out [T][4][4], mix_out [T][24] (optional, NULL to skip).
 * path:    mhc_path, the kernel family (MHC_PATH_AUTO picks by size),
 *          optionally with MHC_PATH_COOPERATIVE OR-ed in.
 * Workspace (optional): NULL, or device memory of workspace_bytes bytes,
 *          256-byte aligned, overlapping no other argument, used by:
 *          - the feature-split kernel: each compute unit keeps one slice of
 *            the features and of W on chip; workgroups exchange per-token
 *            partial sums through the workspace. One workgroup per compute
 *            unit, launched as an ordinary kernel, or cooperatively with
 *            MHC_PATH_COOPERATIVE (MHC_ERR_HIP when that launch is refused);
 *            see mhc_path for when it completes.
 *          - the chunked kernels: workgroups of 16 tokens x 512 features write
 *            per-token partial sums to the workspace, and a second kernel
 *            finishes each token (two plain launches; for small calls).
 *          workspace_bytes below the chosen route's need is
 *          MHC_ERR_INVALID_ARG. Calls that share a workspace must be ordered
 *          (same stream or synchronised).
 *          The first 16,384 bytes are a header that must be ZERO-FILLED
 *          before the workspace is first used (e.g. hipMemset once after
 *          allocating it); every call leaves the header as it found it, so
 *          no clearing is needed between calls. The 32-bit word at offset 0
 *          is the status word: the feature-split kernel sets it to 1 when a
 *          cross-workgroup wait gave up after its bounded number of polls,
 *          in which case that call's outputs are invalid. The library never
 *          clears it: it reports every such call since the caller last wrote
 *          0 there.
 */
mhc_status mhc_fused_step(const void* x, const void* f, int32_t dtype, int64_t tokens,
                          int32_t d, const float* pre_in, const float* post_in,
                          const float* comb_in, const void* w_packed, const float* base,
                          const float* scale, const float* gamma, int32_t sinkhorn_iters,
                          float norm_eps, float hc_eps, void* x_out, void* y_out,
                          float* pre_out, float* post_out, float* comb_out, float* mix_out,
                          int32_t path, void* workspace, int64_t workspace_bytes,
                          mhc_stream_t stream);

/*
 * mhc_fused_step_noalloc -- mhc_fused_step for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops and
 * harnesses that forbid allocation. Same arguments and rules as
 * mhc_fused_step without the workspace pair; the library's own scratch
 * serves as the workspace, and the call allocates nothing.
 *   - Scratch: a static 32 MiB device array, one per GPU the library runs
 *     on, held until the process ends. A call whose route needs more
 *     (mhc_fused_step_workspace_bytes: on the feature-split route about
 *     16.2 MB plus 96 bytes per token at d = 5120, i.e. up to about 180,000
 *     tokens) returns MHC_ERR_INVALID_ARG before launching; MHC_PATH_TILE
 *     needs none.
 *   - Every call on a GPU shares that GPU's scratch: calls that overlap on
 *     one GPU (different streams, or host threads without ordering) race on
 *     it and must not be issued.
 *   - The scratch's header starts zeroed and every call leaves it so (the
 *     first call on a device also enqueues one small kernel that zeroes it).
 *     Its status word is not reported: a feature-split wait that gave up
 *     leaves that call's outputs invalid without an error code; callers that
 *     must check it use mhc_fused_step with their own workspace.
 */
mhc_status mhc_fused_step_noalloc(const void* x, const void* f, int32_t dtype, int64_t tokens,
                                  int32_t d, const float* pre_in, const float* post_in,
                                  const float* comb_in, const void* w_packed, const float* base,
                                  const float* scale, const float* gamma, int32_t sinkhorn_iters,
                                  float norm_eps, float hc_eps, void* x_out, void* y_out,
                                  float* pre_out, float* post_out, float* comb_out,
                                  float* mix_out, int32_t path, mhc_stream_t stream);

/*
 * mhc_mixes -- hc_mixes alone ([SW] Code, hc_mixes and "All 5 steps"): one RMS
 * statistic over the flattened 4*d streams, the 24-wide projection, then the
 * split and Sinkhorn of mhc_sinkhorn4. Reads x [T][4][d]; writes pre_out,
 * post_out [T][4], comb_out [T][4][4] and, if not NULL, mix_out [T][24].
 * w_packed as for mhc_fused_step. path, workspace and workspace_bytes as for
 * mhc_fused_step (same size, mhc_fused_step_workspace_bytes): the
 * feature-split and chunked kernels run in their mixes-only modes.
 */
mhc_status mhc_mixes(const void* x, int32_t dtype, int64_t tokens, int32_t d,
                     const void* w_packed, const float* base, const float* scale,
                     int32_t sinkhorn_iters, float norm_eps, float hc_eps, float* pre_out,
                     float* post_out, float* comb_out, float* mix_out, int32_t path,
                     void* workspace, int64_t workspace_bytes, mhc_stream_t stream);

/*
 * The step as separate kernels, in the order of [RN] Code, Block.forward:
 * mhc_hc_post, mhc_mixes, mhc_hc_pre, mhc_rmsnorm. Each reads its inputs from
 * memory and writes its outputs back, so the streams move (4n+4)*d elements
 * per token against the fused step's (2n+2)*d ([SW] "Why"); the per-element
 * arithmetic and rounding points are those of mhc_fused_step. Same argument
 * rules as mhc_fused_step; d a multiple of mhc_d_granule().
 *
 * mhc_hc_post -- [SW] Code, hc_post: x_out[t][k] = S(sum_j comb_in[t][j][k] *
 *   x[t][j] + post_in[t][k] * f[t]). x_out may be exactly x.
 */
mhc_status mhc_hc_post(const void* x, const void* f, int32_t dtype, int64_t tokens, int32_t d,
                       const float* post_in, const float* comb_in, void* x_out,
                       mhc_stream_t stream);

/* mhc_hc_pre -- [SW] Code, hc_pre: h_out[t] = S(sum_k pre_in[t][k] * x[t][k]);
 * x [T][4][d], h_out [T][d]. */
mhc_status mhc_hc_pre(const void* x, int32_t dtype, int64_t tokens, int32_t d,
                      const float* pre_in, void* h_out, mhc_stream_t stream);

/* mhc_rmsnorm -- [RN] RMSNorm: y_out[t] = S(gamma * (h[t] / sqrt(mean(h[t]^2) +
 * norm_eps))); h, y_out [T][d] (y_out may be exactly h), gamma [d] float32. */
mhc_status mhc_rmsnorm(const void* h, int32_t dtype, int64_t tokens, int32_t d,
                       const float* gamma, float norm_eps, void* y_out, mhc_stream_t stream);

/*
 * mhc_sinkhorn4 -- split float32 mixes [T][24] into the three coefficient sets
 * ([SW] Code, the split/Sinkhorn kernel; "All 5 steps", the formulas for p,
 * u and C):
 *   pre[j]  = sigmoid(scale[0]*m[j] + base[j]) + hc_eps
 *   post[k] = 2*sigmoid(scale[1]*m[4+k] + base[4+k])
 *   comb    = row-softmax(scale[2]*m[8+4j+k] + base[8+4j+k]) + hc_eps, divided
 *             by (column sum + hc_eps); then sinkhorn_iters-1 rounds of
 *             division by (row sum + hc_eps) and by (column sum + hc_eps).
 */
mhc_status mhc_sinkhorn4(const float* mixes, int64_t tokens, const float* base,
                         const float* scale, int32_t sinkhorn_iters, float hc_eps,
                         float* pre_out, float* post_out, float* comb_out,
                         mhc_stream_t stream);

/*
 * Any stream count n in {2, 4, 8} ([SW] Code: the Block constructor sizes the
 * projection as (2+n)*n rows over n*d columns -- mixes slots 0..n-1 pre,
 * n..2n-1 post, 2n+n*j+k comb -- and hc_pre, hc_post and the split kernel take
 * hc_mult as a parameter). Same conventions as above with 4 replaced by n:
 * x [T][n][d], pre/post [T][n], comb [T][n][n], mixes [T][(2+n)n], w_mix
 * float32 [(2+n)n][n*d], base [(2+n)n]. n outside {2, 4, 8} is
 * MHC_ERR_UNSUPPORTED. The packed projection of this family has its own
 * layout (each of the three bf16 terms padded to whole 16-column tiles) and
 * is not interchangeable with mhc_pack_wmix's.
 */

/* Bytes of the packed projection for n streams, width d and stream dtype, or
 * -1 for a bad argument. */
int64_t mhc_wmix_packed_bytes_n(int32_t n, int32_t d, int32_t dtype);

/* Pack w_mix [(2+n)n][n*d] (float32) for mhc_fused_step_n / mhc_mixes_n; same
 * rules as mhc_pack_wmix. */
mhc_status mhc_pack_wmix_n(int32_t n, const float* w_mix, int32_t d, int32_t dtype,
                           void* w_packed, int64_t packed_bytes, mhc_stream_t stream);

/*
 * Workspace bytes that cover every workspace route of mhc_fused_step_n and
 * mhc_mixes_n for (n, tokens, d, dtype) on the current device (the larger of
 * the two below); 0 when neither applies; -1 for a bad argument.
 *   - the feature-split kernel: n in {2, 4} with bf16 streams, d = ns * S with
 *     S a multiple of 64 of at most 256 (n = 2) or 128 (n = 4) features and
 *     16 <= ns <= 64 slices, at most one per compute unit, on a device with
 *     cooperative launch support;
 *   - the chunked block kernel: tokens <= 8192, any n and dtype; the
 *     16,384-byte header plus 4 * R bytes per token and chunk, R = (2+n)n
 *     + 2 rounded up to a multiple of 4, with up to 80 chunks of whole units
 *     (64 features for bf16 at n <= 4, else 32) across d.
 */
int64_t mhc_fused_step_n_workspace_bytes(int32_t n, int64_t tokens, int32_t d, int32_t dtype);

/*
 * mhc_fused_step_route_n -- the kernel family that mhc_fused_step_n and
 * mhc_mixes_n run for `path` and these arguments: MHC_PATH_TILE (standing for
 * the token-block kernel), MHC_PATH_SPLIT or MHC_PATH_CHUNK; -1 (see
 * mhc_last_error) as for mhc_fused_step_route.
 */
int32_t mhc_fused_step_route_n(int32_t n, int32_t path, int64_t tokens, int32_t d, int32_t dtype,
                               int32_t with_workspace);

/*
 * mhc_fused_step_n -- mhc_fused_step for n streams: the same six formulas with
 * sums over n streams and the RMS statistic over n*d values. Two kernels: one
 * pass over the streams (hc_post, RMS statistic, projection, hc_pre, RMSNorm)
 * that writes the mixes to mix_out, then the split/Sinkhorn of
 * mhc_sinkhorn_n reading them back. mix_out [T][(2+n)n] is therefore
 * REQUIRED (NULL is MHC_ERR_INVALID_ARG).
 * path: mhc_path, the kernel family of the pass over the streams:
 *   MHC_PATH_TILE   the token-block kernel (one workgroup per 128 tokens, no
 *                   workspace; the workspace argument is ignored);
 *   MHC_PATH_SPLIT  the feature-split kernel (each compute unit keeps a slice
 *                   of the features and of W; one workgroup per compute
 *                   unit, launched as for mhc_fused_step; the same status
 *                   word at offset 0 and ordering rules);
 *   MHC_PATH_CHUNK  the block kernel in chunks of the features (a workgroup
 *                   per 128-token block and chunk writes partial sums to the
 *                   workspace, h parked in y_out; a finishing kernel adds the
 *                   chunks in order, writes the mixes and the RMSNorm);
 *   MHC_PATH_AUTO   no workspace: the block kernel; with one: the chunks up to
 *                   2048 tokens, else the feature-split kernel where it
 *                   applies, else the chunks where they apply (up to 8192
 *                   tokens), else the block kernel.
 * SPLIT and CHUNK need a workspace and are MHC_ERR_UNSUPPORTED where they do
 * not apply. MHC_PATH_COOPERATIVE may be OR-ed in, as for mhc_fused_step.
 * Workspace: NULL / 0 bytes, or device memory of at least the chosen route's
 * bytes (mhc_fused_step_n_workspace_bytes() covers both), 256-byte aligned,
 * overlapping no other argument; a smaller one is MHC_ERR_INVALID_ARG. Its
 * 16,384-byte header must be zero-filled before first use and keeps the
 * status word, as for mhc_fused_step.
 */
mhc_status mhc_fused_step_n(int32_t n, const void* x, const void* f, int32_t dtype,
                            int64_t tokens, int32_t d, const float* pre_in,
                            const float* post_in, const float* comb_in, const void* w_packed,
                            const float* base, const float* scale, const float* gamma,
                            int32_t sinkhorn_iters, float norm_eps, float hc_eps, void* x_out,
                            void* y_out, float* pre_out, float* post_out, float* comb_out,
                            float* mix_out, int32_t path, void* workspace,
                            int64_t workspace_bytes, mhc_stream_t stream);

/* mhc_mixes_n -- mhc_mixes for n streams; mix_out is required; path and
 * workspace as above (same sizes). */
mhc_status mhc_mixes_n(int32_t n, const void* x, int32_t dtype, int64_t tokens, int32_t d,
                       const void* w_packed, const float* base, const float* scale,
                       int32_t sinkhorn_iters, float norm_eps, float hc_eps, float* pre_out,
                       float* post_out, float* comb_out, float* mix_out, int32_t path,
                       void* workspace, int64_t workspace_bytes, mhc_stream_t stream);

/*
 * mhc_sinkhorn_n -- mhc_sinkhorn4 for n streams: mixes [T][(2+n)n] to pre,
 * post [T][n] and comb [T][n][n], with m[n+k] for post and m[2n+n*j+k] for the
 * comb logits. Each division by (sum + hc_eps) is a multiplication by the
 * correctly rounded reciprocal.
 */
mhc_status mhc_sinkhorn_n(int32_t n, const float* mixes, int64_t tokens, const float* base,
                          const float* scale, int32_t sinkhorn_iters, float hc_eps,
                          float* pre_out, float* post_out, float* comb_out,
                          mhc_stream_t stream);

/*
 * Backward of the fused step, n in {2, 4} (n = 8 is MHC_ERR_UNSUPPORTED). The
 * pages give the forward only; the gradient follows from its definitions
 * ([SW] "All 5 steps" and Code; [RN] formula and Code) by the chain rule, with
 * the casts to the stream dtype passing gradients through unchanged (as
 * automatic differentiation treats a dtype conversion).
 *
 * Inputs: the forward's inputs x, f, pre_in, post_in, comb_in; its saved
 *   outputs x_out [T][n][d] (the new streams) and mix [T][(2+n)n] (the mixes
 *   it wrote to mix_out); the float32 parameters w_mix [(2+n)n][n*d]
 *   (unpacked), base, scale, gamma; sinkhorn_iters, norm_eps, hc_eps as in the
 *   forward; the upstream gradients d_x_out [T][n][d] and d_y [T][d] (stream
 *   dtype) and d_pre, d_post [T][n], d_comb [T][n][n] (float32).
 * Outputs: d_x [T][n][d], d_f [T][d] (stream dtype, rounded to nearest even);
 *   d_pre_in, d_post_in [T][n], d_comb_in [T][n][n], d_w_mix [(2+n)n][n*d],
 *   d_base [(2+n)n], d_scale [3], d_gamma [d] (float32, overwritten, not
 *   accumulated). Sums over tokens are taken in a fixed order: repeated calls
 *   give identical results.
 * Workspace: REQUIRED, mhc_fused_step_backward_workspace_bytes_n() bytes,
 *   256-byte aligned, overlapping no other argument; calls sharing one must be
 *   ordered. The backward leaves the first 16,384 bytes (the forward kernels'
 *   header) untouched, so one workspace can serve forward and backward calls;
 *   the rest needs no initialisation.
 * Same conventions as above otherwise (no output may overlap an input).
 */
int64_t mhc_fused_step_backward_workspace_bytes_n(int32_t n, int64_t tokens, int32_t d);

mhc_status mhc_fused_step_backward_n(
    int32_t n, const void* x, const void* f, int32_t dtype, int64_t tokens, int32_t d,
    const float* pre_in, const float* post_in, const float* comb_in, const void* x_out,
    const float* mix, const float* w_mix, const float* base, const float* scale,
    const float* gamma, int32_t sinkhorn_iters, float norm_eps, float hc_eps, const void* d_x_out,
    const void* d_y, const float* d_pre, const float* d_post, const float* d_comb, void* d_x,
    void* d_f, float* d_pre_in, float* d_post_in, float* d_comb_in, float* d_w_mix,
    float* d_base, float* d_scale, float* d_gamma, void* workspace, int64_t workspace_bytes,
    mhc_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MHC_H */
