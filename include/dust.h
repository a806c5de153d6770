/*
 * dust.h -- C ABI of libdust, the MI355X (gfx950) implementation of the Dust
 * virtual-population gradient estimator.
 *
 * The method ("Dust: Pretraining Transformers Without Backpropagation",
 * Q Labs), as the pages about it describe it:
 *   - HN-mirror digest of the paper, section 2.1 (activation-space
 *     perturbation) and section 2.2 (credit assignment): a linear layer's
 *     output y_t = W x_t is jittered to y_t + sigma a_t, independently for every
 *     token; token s scores a draw by its centred loss decrease c_s; the reward
 *     is r_t = sum_{s>=t} gamma^(s-t) c_s (gamma = 0: the token's own c); over K
 *     draws the output-error estimate is g_t = -(1/(K sigma)) sum_i r_t^(i) a_t^(i)
 *     and the weight gradient is G_W = sum_t g_t x_t^T.
 *   - laoyaoba analysis, mechanism section, and linlog explainer, section "the
 *     core of Dust: virtual population": a_t ~ N(0, I); the LM head is perturbed
 *     directly on the cached logits and only the cross-entropy is recomputed.
 *
 * Conventions shared by every call
 *   - Pointers named as device pointers are HIP device memory owned by the
 *     caller.  The library allocates nothing and keeps no state between calls,
 *     so calls on different streams may run concurrently (they must not share
 *     output or workspace buffers).  The exceptions are
 *     dust_embedding_grad_noalloc, whose scratch is a fixed array per GPU, and
 *     dust_check_targets with a NULL flag, which uses one int32 per GPU.
 *   - Calls enqueue kernels on the caller's stream `s` and return without
 *     waiting, except dust_check_targets, which waits for its own result.
 *     Outputs are overwritten, never accumulated.
 *   - All argument checks run on the host before any HIP call; a rejected call
 *     has no effect.  Launch failures are reported as DUST_ERR_HIP.  Nothing is
 *     thrown across this interface.
 *   - Layouts are row-major; [A,B] means A rows of B contiguous elements.
 *   - T tokens (T % seq_len == 0, sequences of seq_len consecutive tokens),
 *     N = layer output width (N = V for the LM head, N % 4 == 0), d = layer
 *     input width, K draws.
 *   - Size limits (DUST_ERR_UNSUPPORTED beyond them): the calls that form G_W
 *     take T <= 2^22 and N, d <= 2^20, with at most 2^24 - 1 workgroups in the
 *     outer-product grid: ceil(N/256) x ceil(d/256) tiles of G_W times the
 *     token splits (the splits x row tiles rounded up to a multiple of 8),
 *     where one split holds at most about 2^30 / (max(N, d) + 256) tokens;
 *     the per-token stages (dust_head_losses, dust_centre, dust_error_estimate,
 *     dust_perturbed_linear, dust_ce_grad) take T < 2^24; element counts of
 *     every array stay <= 2^40.
 *   - G_W precision (every call that forms G_W): the product runs on the fp16
 *     matrix cores with fp32 accumulation, over copies of each token's g_t and
 *     x_t rescaled by 2^-s_t and 2^s_t (exact; s_t from the two rows' maxima)
 *     and rounded to fp16.  Each product g x then errs by at most 2^-11 of
 *     itself (2^-10 with fp32 X), except elements that fall below fp16's normal
 *     range after scaling (below 2^-14: from 2^-3 of their row's maximum when
 *     the two maxima's exponents sum to -22, the lowest admitted, to 2^-27 at
 *     the highest, 26), which keep an absolute error of 2^-25.  Tokens whose
 *     maxima fit no power of two, or with a non-finite value, are added in
 *     fp32 from the original rows.  Results are deterministic.
 *   - Support calls are this library's own conventions, not steps of the
 *     method, and cite no passage: dust_status_string, dust_version, the
 *     *_workspace_size and dust_embedding_noalloc_bytes size queries,
 *     dust_philox4x32_10 (the raw generator behind the noise convention
 *     below, for checking it) and dust_check_targets (an opt-in input check).
 *
 * Noise convention (the pages fix only that the noise is standard normal and
 * independent per token; this is this library's counter-based stream, which
 * dust_noise reproduces):  a^(i)_t[n] for draw i, token t, column n comes from the
 * Philox4x32-10 block (Salmon et al., SC'11) with key (seed mod 2^32,
 * seed >> 32) and counter words (t, n / 4, i, stream), output words x0..x3.
 * With m(x) = x >> 9 (the top 23 bits), the even words give the radius from
 * u = (m + 1/2) * 2^-23 in (0,1) and the odd words the angle from
 * v = m * 2^-23 in [0,1) revolutions: Box-Muller maps (x0,x1) to columns 4j,
 * 4j+1 (radius sqrt(-2 ln u0), angle 2 pi v1, cosine first) and (x2,x3) to
 * columns 4j+2, 4j+3.  Draw indices and token indices are 0-based within the
 * call.
 */
#ifndef DUST_H
#define DUST_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DUST_OK = 0,
    DUST_ERR_INVALID_ARG = 1, /* null pointer, bad size or parameter            */
    DUST_ERR_WORKSPACE = 2,   /* workspace pointer null or smaller than needed    */
    DUST_ERR_HIP = 3,         /* a HIP launch or runtime call failed              */
    DUST_ERR_UNSUPPORTED = 4, /* valid request beyond the library's size limits   */
    DUST_ERR_TARGETS = 5      /* dust_check_targets found a target out of range   */
} dust_status;

typedef enum { DUST_F32 = 0, DUST_BF16 = 1 } dust_dtype;

/* Opaque stream and event handles: a hipStream_t / hipEvent_t cast to void*.
 * A null stream is HIP's default stream. */
typedef void* dust_stream_t;
typedef void* dust_event_t;

/* Largest accepted sigma.  The LM-head kernels take the exponentials relative
 * to the clean row maximum; |sigma a| <= 8 * 5.77 keeps every term of the
 * perturbed sum inside fp32 range. */
#define DUST_SIGMA_MAX 8.0f
/* Largest accepted vocabulary / layer width N. */
#define DUST_N_MAX 65536
/* Number of stage events dust_head_estimate / dust_linear_estimate record
 * when `stage_events` is non-null (see below). */
#define DUST_STAGE_EVENTS 4

/* Human-readable name of a status code (static string, never null). */
const char* dust_status_string(dust_status st);

/* Library version string, e.g. "libdust 1.0 gfx950". */
const char* dust_version(void);

/* ------------------------------------------------------------------------ */
/* Composed estimators                                                       */
/* ------------------------------------------------------------------------ */

/* LM head (laoyaoba analysis, mechanism section; linlog explainer, "the core
 * of Dust"; paper digest, sections 2.2-2.3): noise on the cached logits, the
 * per-token cross-entropy recomputed for every draw, then centring, the
 * gamma scan, the error estimate and the outer product of the paper digest,
 * section 2.2.
 *   logits  device [T,V], dtype logits_dt (DUST_F32 or DUST_BF16), read only
 *   targets device [T] int32, 0 <= targets[t] < V (not checked here: see
 *           dust_check_targets; an out-of-range target gives undefined values,
 *           never an out-of-bounds access)
 *   X       device [T,d], dtype x_dt, the head's input activations
 *   sigma   noise scale, 0 < sigma <= DUST_SIGMA_MAX
 *   K       draws, 1 <= K < 2^31 (K = 1 gives g_hat = 0: centring zeroes c)
 *   gamma   discount, 0 <= gamma <= 1; the scan restarts at every sequence
 *   seed, stream   noise key and fourth counter word
 *   g_hat   device [T,V] fp32 out: the output-error estimate g_t
 *   G_W     device [V,d] fp32 out: sum_t g_t x_t^T (a sum over tokens)
 *   losses_opt  device [K,T] fp32 out (per-draw perturbed losses) or NULL
 *   workspace   device scratch of at least dust_head_workspace_size(...) bytes
 *   stage_events  NULL, or DUST_STAGE_EVENTS events recorded on s: [0] before
 *           the first kernel, [1] after the per-draw loss / fused estimate
 *           stage, [2] after the error-estimate stage, [3] after the outer
 *           product.  Stages a call skips record back to back.  A NULL entry
 *           is not recorded (each record puts a few microseconds of marker
 *           between the kernels, so a timing loop can drop the ones it does
 *           not need, e.g. [0] when the previous call's [3] marks the start).
 * Requires V % 4 == 0, V <= DUST_N_MAX, T % seq_len == 0. */
dust_status dust_head_estimate(const void* logits, dust_dtype logits_dt,
                               const int32_t* targets,
                               const void* X, dust_dtype x_dt,
                               int64_t T, int64_t V, int64_t d, int64_t seq_len,
                               float sigma, int64_t K, float gamma,
                               uint64_t seed, uint32_t stream,
                               float* g_hat, float* G_W, float* losses_opt,
                               void* workspace, size_t workspace_bytes,
                               dust_stream_t s, const dust_event_t* stage_events);

/* Bytes of workspace dust_head_estimate needs (0 is never returned; for sizes
 * the call rejects, invalid or beyond the size limits, the minimum of 256).
 * The other *_workspace_size queries answer the same way. */
size_t dust_head_workspace_size(int64_t T, int64_t V, int64_t d, int64_t K, float gamma);

/* Hidden linear layer y = W x (paper digest, section 2.2): the caller ran its
 * perturbed forwards with noise from dust_noise(seed, stream, draw0, K, T, N)
 * and measured c[i,t], the centred loss decrease of token t under draw
 * draw0 + i.  c is used as given (the library does not centre it).
 *   X      device [T,d_in], dtype x_dt
 *   c      device [K,T] fp32: draws draw0 .. draw0 + K - 1
 *   draw0, K_total  this call's draws are draw0 .. draw0 + K - 1 of a
 *          population of K_total draws, the K of the estimate's 1/(K sigma):
 *          g_t = -(1/(K_total sigma)) sum_{i<K} r^(i)_t a^(draw0+i)_t.  The
 *          estimate of a population therefore splits into draw ranges whose
 *          results add up (restart, or several calls over one population);
 *          draw0 = 0, K_total = K is the whole estimate.  Requires draw0 >= 0,
 *          K_total >= 1, draw0 + K <= 2^32 (the draw is a 32-bit counter word).
 *   g_hat  device [T,N] fp32 out;  G_W device [N,d_in] fp32 out
 * Same rules as above for sigma, K, gamma, seq_len, N % 4, workspace and
 * stage_events ([1] after the gamma scan). */
dust_status dust_linear_estimate(const void* X, dust_dtype x_dt, const float* c,
                                 int64_t T, int64_t d_in, int64_t N, int64_t seq_len,
                                 float sigma, int64_t K, float gamma,
                                 uint64_t seed, uint32_t stream, int64_t draw0, int64_t K_total,
                                 float* g_hat, float* G_W,
                                 void* workspace, size_t workspace_bytes,
                                 dust_stream_t s, const dust_event_t* stage_events);

size_t dust_linear_workspace_size(int64_t T, int64_t d_in, int64_t N, int64_t K, float gamma);

/* ------------------------------------------------------------------------ */
/* Stages (each is one step of the estimator and can be called on its own)   */
/* ------------------------------------------------------------------------ */

/* Noise (laoyaoba analysis, mechanism section; paper digest, section 2.1):
 * out[k,t,n] = a^(draw0+k)_t[n] for k < ndraw, t < T, n < N (N % 4 == 0).
 * For a caller's perturbed forward y + sigma a and for tests.
 *   out device [ndraw,T,N] fp32. */
dust_status dust_noise(uint64_t seed, uint32_t stream, int64_t draw0, int64_t ndraw,
                       int64_t T, int64_t N, float* out, dust_stream_t s);

/* Raw Philox4x32-10 blocks: out[b] = Philox(key = seed, counter = ctr[b]).
 *   ctr, out device [n,4] uint32.  n may be 0. */
dust_status dust_philox4x32_10(uint64_t seed, const uint32_t* ctr, uint32_t* out, int64_t n,
                               dust_stream_t s);

/* Per-draw LM-head losses (laoyaoba analysis, mechanism section; linlog
 * explainer): losses[i,t] = CE(logits_t + sigma a^(i)_t, targets[t]) in nats.
 *   losses device [K,T] fp32 out. */
dust_status dust_head_losses(const void* logits, dust_dtype logits_dt, const int32_t* targets,
                             int64_t T, int64_t V, float sigma, int64_t K,
                             uint64_t seed, uint32_t stream, float* losses, dust_stream_t s);

/* Centring (paper digest, section 2.2: the centred loss decrease):
 * c[i,t] = mean_j x[j,t] - x[i,t] for per-draw losses x [K,T]; this is the
 * loss decrease d_i = l0 - l_i minus its mean over the draws, whatever the
 * clean loss l0.  x and c device [K,T] fp32; c may equal x (in place). */
dust_status dust_centre(const float* x, int64_t K, int64_t T, float* c, dust_stream_t s);

/* Discounted reward (paper digest, section 2.2):
 * r[i,t] = c[i,t] + gamma r[i,t+1] inside each sequence of seq_len tokens,
 * r = c at a sequence's last token.  c, r device [K,T] fp32; r may equal c. */
dust_status dust_reward_scan(const float* c, int64_t K, int64_t T, int64_t seq_len,
                             float gamma, float* r, dust_stream_t s);

/* Error estimate (paper digest, section 2.2):
 * g_hat[t,n] = -(1/(K_total sigma)) sum_{i<K} r[i,t] a^(draw0+i)_t[n], the
 * noise regenerated from (seed, stream); draw0 and K_total as for
 * dust_linear_estimate (draw0 = 0, K_total = K: the whole estimate).
 *   r device [K,T] fp32; g_hat device [T,N] fp32 out. */
dust_status dust_error_estimate(const float* r, int64_t K, int64_t T, int64_t N,
                                float sigma, uint64_t seed, uint32_t stream,
                                int64_t draw0, int64_t K_total,
                                float* g_hat, dust_stream_t s);

/* Weight gradient (paper digest, section 2.2): G_W[n,k] = sum_t g_hat[t,n] X[t,k].
 *   g_hat device [T,N] fp32; X device [T,d], dtype x_dt; G_W device [N,d] fp32
 *   out; workspace of at least dust_outer_sum_workspace_size(T,N,d) bytes.
 * N need not be a multiple of 4 here. */
dust_status dust_outer_sum(const float* g_hat, const void* X, dust_dtype x_dt,
                           int64_t T, int64_t N, int64_t d, float* G_W,
                           void* workspace, size_t workspace_bytes, dust_stream_t s);

size_t dust_outer_sum_workspace_size(int64_t T, int64_t N, int64_t d);

/* Perturbed forward of a hidden linear layer y = W x (paper digest, sections 2
 * and 2.1; laoyaoba analysis, mechanism section): for k < ndraw,
 *   Y[k,t,n] = sum_j X[t,j] W[n,j] + sigma a^(draw0+k)_t[n],
 * the noise from the same (seed, stream) counters that dust_linear_estimate
 * regenerates, so a caller's perturbed forwards and its estimate agree.
 *   X device [T,d] and W device [N,d] (PyTorch Linear layout), both of dtype dt
 *   (bf16 operands multiply exactly; fp32 operands are split into bf16 hi + lo)
 *   Y device [ndraw,T,N] fp32 out
 * Requires N % 4 == 0, d % 8 == 0, 0 < sigma <= DUST_SIGMA_MAX (sigma = 0 is
 * rejected: use a plain GEMM), T < 2^24, N, d <= 2^20 and fewer than 2^24
 * output tiles of 128 x 128 (DUST_ERR_UNSUPPORTED otherwise). */
dust_status dust_perturbed_linear(const void* X, const void* W, dust_dtype dt, int64_t T,
                                  int64_t d, int64_t N, float sigma, uint64_t seed,
                                  uint32_t stream, int64_t draw0, int64_t ndraw, float* Y,
                                  dust_stream_t s);

/* Embedding layer (paper digest, section 2.2: a one-hot input turns the outer
 * product into a scatter-add): G_E[v,:] = sum over tokens t with ids[t] = v of
 * g_hat[t,:], the rows taken in increasing t (in blocks of 32 of the id-sorted
 * order; deterministic: no float atomics, and the sort's integer counts do not
 * depend on the order of their adds; rows of unused ids are 0; ids outside
 * [0, vocab) are skipped).
 *   ids device [T] int32; g_hat device [T,N] fp32 (N % 4 == 0);
 *   G_E device [vocab,N] fp32 out;
 *   workspace >= dust_embedding_workspace_size(T, N, vocab) bytes (about
 *   T/512 * vocab * 4 + T/32 * N * 8 + 12 T + 8 vocab).
 * Requires T <= 2^22, N <= 2^20, vocab <= 2^24 and ceil(T/512) * vocab <= 2^31
 * (DUST_ERR_UNSUPPORTED otherwise). */
dust_status dust_embedding_grad(const int32_t* ids, const float* g_hat, int64_t T, int64_t N,
                                int64_t vocab, float* G_E, void* workspace,
                                size_t workspace_bytes, dust_stream_t s);
size_t dust_embedding_workspace_size(int64_t T, int64_t N, int64_t vocab);

/* dust_embedding_grad without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, kernels and results (bitwise) as
 * dust_embedding_grad; the scratch is the library's own fixed device array of
 * DUST_EMBEDDING_NOALLOC_BYTES per GPU, held until the process ends, and the
 * call allocates nothing.  Sizes whose scratch (dust_embedding_noalloc_bytes)
 * exceeds it return DUST_ERR_UNSUPPORTED before any HIP call; the pages'
 * embedding shape (16384 tokens, width 512, vocabulary 4096) needs about 2.7
 * MiB.  Call with the stream's device current.  All calls on one GPU share its
 * array: calls that overlap in time on one GPU (different streams, or
 * different host threads) race and give undefined results; calls ordered on
 * one stream are safe, since each call writes every scratch byte it reads. */
#define DUST_EMBEDDING_NOALLOC_BYTES ((size_t)16 << 20)
dust_status dust_embedding_grad_noalloc(const int32_t* ids, const float* g_hat, int64_t T,
                                        int64_t N, int64_t vocab, float* G_E, dust_stream_t s);
/* Scratch bytes dust_embedding_grad_noalloc needs for a size (0 for invalid
 * sizes and sizes beyond dust_embedding_grad's limits). */
size_t dust_embedding_noalloc_bytes(int64_t T, int64_t N, int64_t vocab);

/* Optimiser steps on a weight gradient (linlog explainer, experiment setup:
 * SGD with momentum; paper digest, section 3.3: Adam).  All arrays device fp32
 * [n], updated in place; G_W approximates +dL/dW, so W moves against it.
 *   SGD:  m = momentum m + (G + wd W);  W -= lr m   (PyTorch SGD, dampening 0)
 *   Adam: g = G + wd W; m = b1 m + (1-b1) g; v = b2 v + (1-b2) g^2;
 *         W -= lr/(1-b1^step) m / (sqrt(v)/sqrt(1-b2^step) + eps)  (step >= 1)
 * n <= 2^40 (DUST_ERR_UNSUPPORTED beyond). */
dust_status dust_sgd_momentum(float* W, const float* G, float* m, int64_t n, float lr,
                              float momentum, float weight_decay, dust_stream_t s);
dust_status dust_adam(float* W, const float* G, float* m, float* v, int64_t n, float lr,
                      float beta1, float beta2, float eps, float weight_decay, int64_t step,
                      dust_stream_t s);

/* Closed-form LM-head gradient dCE/dz = softmax(z_t) - onehot(y_t) (paper
 * digest, section 4.2: the backprop gradient the estimate is compared with).
 *   logits device [T,V] (dtype dt), targets device [T] int32, out device [T,V] fp32. */
dust_status dust_ce_grad(const void* logits, dust_dtype dt, const int32_t* targets, int64_t T,
                         int64_t V, float* out, dust_stream_t s);

/* Checks 0 <= targets[t] < V for all t; waits on s for the answer.
 * Returns DUST_OK or DUST_ERR_TARGETS.  `flag` is a device int32 the call
 * overwrites (caller-owned scratch), or NULL for the library's own flag, one
 * per GPU: calls with NULL that overlap on one GPU race. */
dust_status dust_check_targets(const int32_t* targets, int64_t T, int64_t V, int32_t* flag,
                               dust_stream_t s);

#ifdef __cplusplus
}
#endif

#endif /* DUST_H */
