/*
 * sdm.h: C ABI of the Sparse Delta Memory (SDM) recurrent core for AMD
 * Instinct MI355X (gfx950).
 *
 * The core, per sequence b, head h and token t, in the pages' notation:
 *
 *   select  The pre-PKM key k'_t and query q'_t (length 2*sqrtN each) are
 *           split into halves; slot n = i*sqrtN + j has the outer-sum score
 *           x_1[i] + x_2[j].  The W slots with the highest scores form the
 *           write set I^w_t (from k'), the R highest the read set I^r_t
 *           (from q'), found with the product-key identity
 *           top_k(s1 (+) s2) = top_k(top_k(s1) (+) top_k(s2))
 *           [explainer "Sparse Delta Memory：通过稀疏性扩展线性 RNN 的状态容量"
 *           (papers.ananclaw.com), §3.1 step 1; "Technical Summary: Sparse
 *           Delta Memory (SDM)" (gist.science), Methodology / Core Mechanism 2].
 *           Order, ties and weights are readings of this library (the pages
 *           leave them open): scores are compared as exact real numbers, ties
 *           go to the lower flat index n, lists are returned in that order,
 *           and the weights k^(i), q^(i) are the softmax of the selected
 *           scores.
 *   write   For i in I^w_t:  m = alpha_t * M[i];  M[i] = m + beta_t * k^(i) *
 *           (v_t - m); every other row is left as it is
 *           [explainer §3.1 step 2; Technical Summary, Core Mechanism 3].
 *   read    y_t = sum over i in I^r_t of q^(i) * M[i], on the state after the
 *           same token's write [explainer §3.1 step 3; Technical Summary,
 *           Core Mechanism 4].
 *   M starts from the shared initial state M_0 of the head [explainer §3.1,
 *   learned initial state; Technical Summary, Learned Initial State].
 *
 * Conventions
 *   - Every tensor pointer is a DEVICE pointer (HIP global memory) owned by
 *     the caller; the library never allocates, frees or retains them, except
 *     that a handle borrows M_0 until sdm_destroy.  All tensors are dense,
 *     row-major, and must be 16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is
 *     enqueued asynchronously on it; no call synchronises the host.
 *   - Shapes: B sequences, T tokens, H heads, N = sqrtN^2 slots per head,
 *     d_v columns per slot.  "ht" below is the head-token index
 *     (b*T + t)*H + h.
 *   - Arguments are validated before any HIP call.  On failure the call
 *     returns a non-zero sdm_status, enqueues nothing, and
 *     sdm_last_error() describes the reason (thread-local).  No C++
 *     exception crosses this interface.
 *   - Inputs must be finite; alpha in (0, 1] and beta in [0, 1] are the
 *     intended ranges (not checked).
 *   - Different handles and streams may be used concurrently.  Calls that
 *     share an output or workspace buffer must be ordered by the caller.
 *
 * Limits: 1 <= sqrtN <= 1024, 1 <= W, R <= min(sqrtN, 64), 1 <= d_v, H, B,
 * 1 <= T, B*T*H < 2^31.
 */
#ifndef SDM_H
#define SDM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct sdm_ctx *sdm_handle;

typedef enum {
    SDM_OK = 0,
    SDM_ERR_ARG = 1,         /* invalid argument (null, size, alignment) */
    SDM_ERR_UNSUPPORTED = 2, /* valid but outside the supported limits  */
    SDM_ERR_WORKSPACE = 3,   /* workspace smaller than sdm_workspace_size */
    SDM_ERR_HIP = 4          /* a HIP call failed; see sdm_last_error()  */
} sdm_status;

/* Element type of k', q' and v (SDM_F32 or SDM_BF16), and of the state M
 * (sdm_create_ex, sdm_create_fp8).  alpha, beta, M_0 and y are float32. */
typedef enum { SDM_F32 = 0, SDM_BF16 = 1, SDM_FP8_E4M3 = 2 } sdm_dtype;

/*
 * Write/read schedule used by sdm_forward.  Both produce the same result up
 * to float32 rounding order.
 *   SERIAL   token-serial per (sequence, head, column slice), rows gathered
 *            and scattered in HBM with cross-token prefetch; where those
 *            units are fewer than four per compute unit, the slots of each
 *            token are split over the four waves of a workgroup.
 *   TIMEPAR  time-parallel: (slot, t) events sorted per chunk of tokens and
 *            a per-slot scan of the affine map M <- a*M + c*v.
 *   AUTO     the library's choice for the shape.
 * With one token per sequence (T == 1: a decode step) there is no order
 * across tokens to schedule, and TIMEPAR runs a single kernel instead of the
 * sort and scan: the token's writes, then its reads of the updated rows.
 * With a bfloat16 or E4M3 state, TIMEPAR applies the chunks either in one
 * launch (chunks of at most 256 tokens, and enough (sequence, head,
 * 64-column slice) units to fill the GPU) or as a read and a write launch
 * per chunk; both give the same bits.  The environment variable
 * SDM_TP_FUSED=0 or SDM_TP_FUSED=1, read at each call, forces the per-chunk
 * or the one-launch form where it applies (for tests and measurements).
 */
typedef enum {
    SDM_VARIANT_AUTO = 0,
    SDM_VARIANT_SERIAL = 1,
    SDM_VARIANT_TIMEPAR = 2
} sdm_variant;

/* sdm_forward flags */
#define SDM_FLAG_CONTINUE 1u /* start from the state already in M (no M <- M_0) */

/*
 * Create a handle for one SDM layer shape: H heads, each with N = sqrtN^2
 * slots of d_v columns, W write slots and R read slots per token
 * [explainer "Sparse Delta Memory：通过稀疏性扩展线性 RNN 的状态容量", §3.1 and
 * §3.3 Eq. (6); "Technical Summary: Sparse Delta Memory (SDM)", Methodology].
 *   M0     device [H][N][d_v] float32, the shared initial state (explainer
 *          §3.1, learned initial state); borrowed: it must stay valid and
 *          unchanged until sdm_destroy.
 *   H, sqrtN, d_v, W, R  as above.
 *   out    receives the handle.
 * Makes no HIP call.  Errors: SDM_ERR_ARG (null, size), SDM_ERR_UNSUPPORTED
 * (outside the limits).
 */
sdm_status sdm_create(const float *M0, int H, int sqrtN, int d_v, int W, int R,
                      sdm_handle *out);

/*
 * As sdm_create, with the element type of the state M that the calls below
 * read and write:
 *   SDM_F32   float32 (what sdm_create gives);
 *   SDM_BF16  bfloat16, a reduced-precision state (the explainer "Sparse
 *             Delta Memory：通过稀疏性扩展线性 RNN 的状态容量" suggests a narrower
 *             state type to fit larger N in its engineering notes; the pages
 *             fix no rounding rule).  M_0 stays float32 and is rounded to
 *             bfloat16 (nearest, ties to even) when M is initialised; every
 *             write computes a*row + c*v in float32 from the stored row and
 *             stores it rounded the same way; reads use the stored rows and
 *             accumulate y in float32.  Halves the row traffic.  Needs the
 *             time-parallel schedule (d_v % 4 == 0): SDM_VARIANT_SERIAL
 *             returns SDM_ERR_UNSUPPORTED.  Every read sees the row as the
 *             state holds it after the writes at tokens <= its own, rounded
 *             after each of them, so y does not depend on how the tokens are
 *             split into calls.
 * Errors as sdm_create, plus SDM_ERR_ARG for another state_dtype
 * (SDM_FP8_E4M3 included: it takes a scale, see sdm_create_fp8).
 */
sdm_status sdm_create_ex(const float *M0, int H, int sqrtN, int d_v, int W, int R,
                         sdm_dtype state_dtype, sdm_handle *out);

/*
 * As sdm_create, with an 8-bit state: M holds OCP FP8 E4M3 codes (sign, 4
 * exponent bits with bias 7, 3 mantissa bits, largest magnitude 448, no
 * infinities) of the state scaled by 2^-scale_log2, i.e. a code c stands for
 * the value c * 2^scale_log2.  The explainer "Sparse Delta Memory：通过稀疏性
 * 扩展线性 RNN 的状态容量" names 8-bit states to fit N ~ 10^7 slots on one card
 * (engineering notes); the pages fix no format or scale, so this is a
 * reading: one power-of-two scale per layer (so scaling is exact), values
 * rounded to the nearest code, ties to even, magnitudes beyond 448 *
 * 2^scale_log2 saturated.  M_0 stays float32 and is rounded that way when M
 * is initialised; every write computes a*row + c*v in float32 from the
 * stored row and stores it rounded; reads use the stored rows and
 * accumulate y in float32.  A quarter of the float32 row traffic.  Needs the
 * time-parallel schedule (d_v % 4 == 0); no backward.  Choose the scale so
 * that the state's magnitudes stay below 448 * 2^scale_log2 (e.g. -4 for
 * values up to 28 with spacing 2^-11 near 2^-5).
 * Errors as sdm_create, plus SDM_ERR_ARG for scale_log2 outside [-64, 64].
 */
sdm_status sdm_create_fp8(const float *M0, int H, int sqrtN, int d_v, int W, int R,
                          int scale_log2, sdm_handle *out);

/*
 * Release a handle (M_0 is not touched).  Makes no HIP call.  NULL is
 * accepted.
 */
sdm_status sdm_destroy(sdm_handle h);

/*
 * Bytes of device workspace sdm_forward needs for B sequences of T tokens
 * with the given input dtype and variant (a pure function of its
 * arguments; makes no HIP call).
 */
sdm_status sdm_workspace_size(sdm_handle h, int B, int64_t T, sdm_dtype dtype,
                              sdm_variant variant, size_t *bytes);

/*
 * Selection only (the first step of the core, standalone): the top-W slots of
 * k' and the top-R slots of q' under the outer-sum scores, by the
 * product-key identity, with softmax weights [explainer §3.1 step 1;
 * Technical Summary, Core Mechanism 2].
 *   kp, qp  device [B][T][H][2*sqrtN], element type `dtype`.
 *   Iw, kw  device [B][T][H][W]: write slots (int32, canonical order) and
 *           their softmax weights (float32).
 *   Ir, qw  device [B][T][H][R]: read slots and weights.
 * Outputs must not alias inputs.
 */
sdm_status sdm_select(sdm_handle h, int B, int64_t T, const void *kp, const void *qp,
                      sdm_dtype dtype, int32_t *Iw, float *kw, int32_t *Ir, float *qw,
                      void *stream);

/*
 * The whole core: select, then the gated delta write and the sparse read for
 * every token in order [explainer §3.1 steps 1-3; Technical Summary, Core
 * Mechanism 2-4].
 *   kp, qp     device [B][T][H][2*sqrtN], element type `dtype`.
 *   v          device [B][T][H][d_v], element type `dtype`.
 *   alpha,beta device [B][T][H] float32, the gates of each head-token.
 *   workspace  device scratch of ws_bytes >= sdm_workspace_size(...) bytes,
 *              16-byte aligned; its contents are undefined afterwards.
 *   y          device [B][T][H][d_v] float32, output.
 *   M          device [B][H][N][d_v], float32, bfloat16 or E4M3 codes as the
 *              handle's state type (sdm_create_ex, sdm_create_fp8): the
 *              final state on return.
 *              Unless SDM_FLAG_CONTINUE is set it is first overwritten with
 *              M_0 (so a failed call can simply be retried); with the flag it
 *              must hold the state to continue from.
 * Outputs must not alias inputs or each other.
 * Everything runs on `stream`, with the results of sdm_prepare(...) then
 * sdm_apply(...) with the same arguments, bit for bit.  For one token per
 * sequence (T = 1) with the time-parallel variant the whole step is one
 * kernel launch (after the copy of M_0 unless SDM_FLAG_CONTINUE is set) and
 * the workspace is not touched.
 */
sdm_status sdm_forward(sdm_handle h, int B, int64_t T, const void *kp, const void *qp,
                       const void *v, const float *alpha, const float *beta,
                       sdm_dtype dtype, sdm_variant variant, unsigned flags,
                       void *workspace, size_t ws_bytes, float *y, void *M,
                       void *stream);

/*
 * sdm_forward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops such as
 * one-token decode steps, harnesses that forbid allocation).  The scratch is
 * a static device array of SDM_NOALLOC_MAX_BYTES that the library holds on
 * each GPU it runs on until the process ends; the call allocates nothing.
 * Arguments, results and errors as sdm_forward, plus SDM_ERR_UNSUPPORTED
 * when sdm_workspace_size(...) for the call exceeds SDM_NOALLOC_MAX_BYTES
 * (a one-token step of every layer shape within the limits above fits; so
 * do a few hundred tokens of the shapes with sqrtN <= 128).  The first call
 * on a device looks up that device's scratch address (a HIP call; the
 * stream's device is made current for it and restored).  Every call on one
 * GPU uses the same scratch: calls that overlap on one GPU (other streams,
 * other threads) race and must be ordered by the caller.  Nothing in the
 * scratch needs to start at zero.
 */
#define SDM_NOALLOC_MAX_BYTES (64u << 20)

sdm_status sdm_forward_noalloc(sdm_handle h, int B, int64_t T, const void *kp, const void *qp,
                               const void *v, const float *alpha, const float *beta,
                               sdm_dtype dtype, sdm_variant variant, unsigned flags, float *y,
                               void *M, void *stream);

/*
 * The two halves of sdm_forward, for callers that time or pipeline them.
 * sdm_forward(...) is sdm_prepare(...) followed by sdm_apply(...) with the
 * same handle, shapes, dtype, variant and workspace.
 *
 * sdm_prepare: unless SDM_FLAG_CONTINUE is set, M <- M_0; then the selection
 *   of every head-token is written into the workspace (with the write
 *   coefficients alpha*(1 - beta*k) and beta*k, and the forwarding plan the
 *   token-serial schedule needs).  Arguments as for sdm_forward.
 * sdm_apply: the gated delta write and sparse read of every token, in order,
 *   from the prepared workspace: reads v and M, writes y and M.  The
 *   workspace must hold the result of sdm_prepare for the same call shape
 *   (stream order is enough; nothing else may write it in between).
 */
sdm_status sdm_prepare(sdm_handle h, int B, int64_t T, const void *kp, const void *qp,
                       const float *alpha, const float *beta, sdm_dtype dtype,
                       sdm_variant variant, unsigned flags, void *workspace,
                       size_t ws_bytes, void *M, void *stream);

sdm_status sdm_apply(sdm_handle h, int B, int64_t T, const void *v, sdm_dtype dtype,
                     sdm_variant variant, void *workspace, size_t ws_bytes, float *y,
                     void *M, void *stream);

/*
 * Write-slot utilisation (an addressing-collapse monitor; the explainer's
 * limitations and engineering notes suggest tracking how often each slot is
 * updated).  Runs the write-set selection of every head-token and adds, for
 * head h and slot n, the number of head-tokens (b, t) whose write set
 * contains n:  counts[h][n] += #{(b, t) : n in I^w_(b,t,h)}.
 *   kp      device [B][T][H][2*sqrtN], element type `dtype`.
 *   counts  device [H][N] uint32, accumulated into (zero it for a fresh
 *           count; integer atomics, so the result does not depend on order).
 */
sdm_status sdm_write_histogram(sdm_handle h, int B, int64_t T, const void *kp,
                               sdm_dtype dtype, uint32_t *counts, void *stream);

/*
 * Backward of the core: gradients of a loss L(y, M_T) given dL/dy and
 * dL/dM_T, with the selected slot sets held fixed (they are piecewise
 * constant in k', q'; the gradient reaches k' and q' through the softmax
 * weights).  The explainer "Sparse Delta Memory：通过稀疏性扩展线性 RNN 的状态容量"
 * (§3.1; its training discussion needs a memory-efficient backward and the
 * gradient of the learned initial state) fixes the forward; the derivatives
 * follow from it by the chain rule.
 *
 * The call recomputes the forward (selection, then the writes, recording
 * the epoch-start row of every slot an epoch writes) and runs the tokens in
 * reverse on the time-parallel schedule; it needs a float32 state
 * (sdm_create) and d_v % 4 == 0 (else SDM_ERR_UNSUPPORTED).  Memory stays
 * bounded for long sequences: the tokens are taken in chunks of whole epochs,
 * the recorded rows cover one chunk, and the state at each chunk start is
 * kept (a first forward pass computes those states, then each chunk's
 * forward runs again from its start state and is reversed).  The call uses
 * the fewest chunks that ws_bytes allows; every chunk count gives the same
 * gradients bit for bit.
 *   kp, qp, v, alpha, beta, dtype   the forward's inputs (as sdm_forward)
 *   Minit      device [B][H][N][d_v] float32: the state the forward started
 *              from (as with SDM_FLAG_CONTINUE), or NULL for M_0
 *   dy         device [B][T][H][d_v] float32, dL/dy
 *   dMT        device [B][H][N][d_v] float32, dL/dM_T, or NULL for zero
 *   workspace  >= sdm_backward_workspace_size(...) bytes, 16-byte aligned:
 *              the least memory the call can run in.  A larger workspace
 *              (sdm_backward_workspace_size_ex with fewer chunks) saves
 *              forward recomputation.
 * Outputs (device, float32, overwritten):
 *   dkp, dqp   [B][T][H][2*sqrtN]   dL/dk', dL/dq'
 *   dv         [B][T][H][d_v]       dL/dv
 *   dalpha, dbeta [B][T][H]
 *   dMinit     [B][H][N][d_v]       dL/d(initial state of each sequence)
 *   dM0        [H][N][d_v]          sum over b of dMinit, or NULL to skip
 * Results are deterministic (fixed reduction orders).
 */
sdm_status sdm_backward_workspace_size(sdm_handle h, int B, int64_t T, sdm_dtype dtype,
                                       size_t *bytes);

/*
 * Workspace for the backward run in `chunks` chunks of whole epochs (1: the
 * whole sequence in one chunk, the fastest; 0: the count that needs the least
 * memory, which is what sdm_backward_workspace_size reports).  Counts beyond
 * the number of epochs act as that number.  A pure function of its
 * arguments; no HIP call.  Errors as sdm_backward_workspace_size, plus
 * SDM_ERR_ARG for chunks < 0.
 */
sdm_status sdm_backward_workspace_size_ex(sdm_handle h, int B, int64_t T, sdm_dtype dtype,
                                          int chunks, size_t *bytes);

sdm_status sdm_backward(sdm_handle h, int B, int64_t T, const void *kp, const void *qp,
                        const void *v, const float *alpha, const float *beta, sdm_dtype dtype,
                        const float *Minit, const float *dy, const float *dMT, void *workspace,
                        size_t ws_bytes, float *dkp, float *dqp, float *dv, float *dalpha,
                        float *dbeta, float *dMinit, float *dM0, void *stream);

/* Static description of a status code. */
const char *sdm_status_string(sdm_status s);

/* Thread-local description of the last failure on this thread ("" if none). */
const char *sdm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SDM_H */
