/*
 * dust_oracle.c -- plain, slow, fp64 CPU oracle of the Dust virtual-population
 * gradient estimator.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library.  The GPU library
 * (libdust) shares no code, header, table or helper with it, and neither side
 * includes or links the other.
 *
 * Sources (the pages about "Dust: Pretraining Transformers Without
 * Backpropagation", Q Labs):
 *   [P1] laoyaoba news analysis, section "mechanism: how the virtual population
 *        bypasses backprop" -- per-token, per-layer Gaussian noise on linear
 *        outputs; LM head perturbed on cached logits, only CE recomputed.
 *   [P2] HN-mirror digest of the paper, section 2.1 (activation-space
 *        perturbation) and section 2.2 (credit assignment): y_t = W x_t is
 *        jittered to y_t + sigma a_t; c_s is token s's centred loss decrease;
 *        r_t = sum_{s>=t} gamma^(s-t) c_s (gamma = 0: the token's own c);
 *        g_t = -(1/(K sigma)) sum_i r_t^(i) a_t^(i); G_W = sum_t g_t x_t^T.
 *   [P3] linlog.top explainer, section "the core of Dust: virtual population"
 *        -- a ~ N(0, I) per token; LM head: perturb cached logits, recompute CE.
 *
 * Readings taken where the pages are silent:
 *   - "centred" = subtract the per-token mean over the K draws.
 *   - noise stream = Philox4x32-10 (Salmon et al., SC'11) keyed by the 64-bit
 *     seed, counter (token, column/4, draw, stream), then Box-Muller (1958):
 *     the radius from a uniform in (0,1) and the angle from a fraction of a
 *     revolution in [0,1), both made from the top 23 bits of a word.
 *   - the gamma scan restarts at every sequence boundary (seq_len tokens).
 *   - G_W sums over tokens (no mean); no bias term.
 *
 * Every step below follows the pages' order: noise, per-draw loss, loss
 * decrease, centring, discounted reward, error estimate, outer product.
 * Everything is double precision with libm; loops are plain.  OpenMP only
 * splits independent tokens (or independent output rows) across threads and
 * does not change any result.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------- */
/* Philox4x32-10: Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as   */
/* easy as 1, 2, 3", SC'11.  Round function: two 32x32->64 products of      */
/* counter words 0 and 2 with the multipliers, the high halves xor-ed with   */
/* the other counter words and the key; the key is bumped by the Weyl        */
/* constants between rounds.                                                 */
/* ------------------------------------------------------------------------- */
#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

void oracle_philox4x32_10(uint64_t seed, const uint32_t ctr_in[4], uint32_t out[4])
{
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = (uint32_t)(seed & 0xFFFFFFFFu);
    uint32_t k1 = (uint32_t)(seed >> 32);
    for (int round = 0; round < 10; ++round) {
        uint64_t p0 = (uint64_t)PHILOX_M0 * (uint64_t)c0;
        uint64_t p1 = (uint64_t)PHILOX_M1 * (uint64_t)c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += PHILOX_W0;
        k1 += PHILOX_W1;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Uniform in (0,1): the top 23 bits of a Philox word as an integer m, then
 * u = (m + 1/2) / 2^23.  Exact in fp32 and fp64; never 0 or 1. */
double oracle_uniform(uint32_t x)
{
    double m = (double)(x >> 9);
    return m * 0x1p-23 + 0x1p-24;
}

/* Angle of Box-Muller as a fraction of a revolution, in [0,1): the top 23
 * bits of a Philox word as an integer m, v = m / 2^23.  Exact in fp32 and
 * fp64.  (The angle needs no offset: 0 is a valid angle, and v and v + 1 give
 * the same point of the circle.) */
double oracle_angle(uint32_t x)
{
    return (double)(x >> 9) * 0x1p-23;
}

/* Four standard normals of one Philox block: Box-Muller on the pairs of words
 * (0,1) and (2,3); radius sqrt(-2 ln u) from the even word's uniform u, angle
 * 2 pi v from the odd word's fraction v. */
void oracle_normal4(uint64_t seed, uint32_t j, uint32_t t, uint32_t i, uint32_t stream,
                    double a[4])
{
    const double two_pi = 6.283185307179586476925286766559;
    uint32_t ctr[4] = { t, j, i, stream };
    uint32_t x[4];
    oracle_philox4x32_10(seed, ctr, x);
    double u0 = oracle_uniform(x[0]), v1 = oracle_angle(x[1]);
    double u2 = oracle_uniform(x[2]), v3 = oracle_angle(x[3]);
    double rho0 = sqrt(-2.0 * log(u0));
    double rho1 = sqrt(-2.0 * log(u2));
    a[0] = rho0 * cos(two_pi * v1);
    a[1] = rho0 * sin(two_pi * v1);
    a[2] = rho1 * cos(two_pi * v3);
    a[3] = rho1 * sin(two_pi * v3);
}

/* Batch forms for the tests: n independent blocks / uniforms. */
void oracle_philox_batch(uint64_t seed, const uint32_t* ctr, uint32_t* out, int64_t n)
{
    for (int64_t b = 0; b < n; ++b) oracle_philox4x32_10(seed, ctr + 4 * b, out + 4 * b);
}

void oracle_uniform_batch(const uint32_t* x, double* u, int64_t n)
{
    for (int64_t b = 0; b < n; ++b) u[b] = oracle_uniform(x[b]);
}

void oracle_angle_batch(const uint32_t* x, double* v, int64_t n)
{
    for (int64_t b = 0; b < n; ++b) v[b] = oracle_angle(x[b]);
}

/* The noise row a^(i)_t of width N (N a multiple of 4). */
static void noise_row(uint64_t seed, uint32_t stream, int64_t i, int64_t t, int64_t N,
                      double* row)
{
    for (int64_t j = 0; j < N / 4; ++j)
        oracle_normal4(seed, (uint32_t)j, (uint32_t)t, (uint32_t)i, stream, row + 4 * j);
}

/* out[k, t, n] = a^(draw0 + k)_t[n] for k < ndraw. */
void oracle_noise(uint64_t seed, uint32_t stream, int64_t draw0, int64_t ndraw,
                  int64_t T, int64_t N, double* out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t kt = 0; kt < ndraw * T; ++kt) {
        int64_t k = kt / T, t = kt % T;
        noise_row(seed, stream, draw0 + k, t, N, out + (k * T + t) * N);
    }
}

/* ------------------------------------------------------------------------- */
/* Per-token cross-entropy (next-token loss in nats) of a logit row z:      */
/* CE = log sum_v exp(z_v) - z_y, with the row maximum taken out first.      */
/* ------------------------------------------------------------------------- */
static double cross_entropy(const double* z, int64_t V, int32_t y)
{
    double m = z[0];
    for (int64_t v = 1; v < V; ++v) if (z[v] > m) m = z[v];
    double s = 0.0;
    for (int64_t v = 0; v < V; ++v) s += exp(z[v] - m);
    return log(s) + m - z[y];
}

/* LM-head draws of one token t ([P1], [P3]: noise on the cached logits, only
 * the CE recomputed).  ell0 = clean loss; ell[i] = loss under draw i. */
static void head_token_losses(const double* z, int32_t y, int64_t V, double sigma, int64_t K,
                              uint64_t seed, uint32_t stream, int64_t t,
                              double* ell0, double* ell, double* a_scratch,
                              double* zp_scratch)
{
    *ell0 = cross_entropy(z, V, y);
    for (int64_t i = 0; i < K; ++i) {
        noise_row(seed, stream, i, t, V, a_scratch);
        for (int64_t v = 0; v < V; ++v) zp_scratch[v] = z[v] + sigma * a_scratch[v];
        ell[i] = cross_entropy(zp_scratch, V, y);
    }
}

/* Centred loss decrease of one token over its K draws:
 * d_i = ell0 - ell_i, c_i = d_i - mean_j d_j. */
static void centre_token(double ell0, const double* ell, int64_t K, int64_t stride,
                         double* c)
{
    double mean = 0.0;
    for (int64_t i = 0; i < K; ++i) mean += (ell0 - ell[i * stride]);
    mean /= (double)K;
    for (int64_t i = 0; i < K; ++i) c[i * stride] = (ell0 - ell[i * stride]) - mean;
}

/* Discounted reward inside each sequence of L tokens ([P2] section 2.2):
 * r_t = c_t + gamma * r_{t+1}, with r = c at a sequence's last token.
 * c and r are [K, T]. */
void oracle_reward_scan(const double* c, int64_t K, int64_t T, int64_t L, double gamma,
                        double* r)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < K; ++i) {
        for (int64_t s0 = 0; s0 < T; s0 += L) {
            double carry = 0.0;
            for (int64_t t = s0 + L - 1; t >= s0; --t) {
                carry = c[i * T + t] + gamma * carry;
                r[i * T + t] = carry;
            }
        }
    }
}

/* Error estimate of token t ([P2] section 2.2):
 * g_t = -(1/(K sigma)) sum_i r^(i)_t a^(i)_t, a regenerated from its counters.
 * r^(i)_t is read at r[i * r_stride + r_col]; t keys the noise.
 * s_row (NULL to skip) receives the scale that a rounding error of the sum is
 * measured against; it does not enter g.  It is the magnitude of the sum's
 * terms plus the same with every reward replaced by the token's largest,
 * (1/(K sigma)) sum_i (|r^(i)_t| + max_j |r^(j)_t|) |a^(i)_t|: a reward computed
 * in single precision (a loss change formed from a ratio of exp sums, or a
 * discounted scan) errs by a fraction of the token's largest reward, whatever
 * the size of the reward itself. */
static void error_estimate_token(const double* r, int64_t K, int64_t r_stride, int64_t r_col,
                                 int64_t t, int64_t N, double sigma, uint64_t seed,
                                 uint32_t stream, double* g_row, double* a_scratch,
                                 double* s_row)
{
    for (int64_t n = 0; n < N; ++n) g_row[n] = 0.0;
    if (s_row) for (int64_t n = 0; n < N; ++n) s_row[n] = 0.0;
    double rmax = 0.0;
    if (s_row)
        for (int64_t i = 0; i < K; ++i) rmax = fmax(rmax, fabs(r[i * r_stride + r_col]));
    for (int64_t i = 0; i < K; ++i) {
        double rit = r[i * r_stride + r_col];
        noise_row(seed, stream, i, t, N, a_scratch);
        for (int64_t n = 0; n < N; ++n) g_row[n] += rit * a_scratch[n];
        if (s_row)
            for (int64_t n = 0; n < N; ++n) s_row[n] += (fabs(rit) + rmax) * fabs(a_scratch[n]);
    }
    double scale = -1.0 / ((double)K * sigma);
    for (int64_t n = 0; n < N; ++n) g_row[n] *= scale;
    if (s_row) for (int64_t n = 0; n < N; ++n) s_row[n] *= -scale;
}

/* Weight gradient ([P2] section 2.2): G_W[n][k] = sum_t g[t][n] * X[t][k]. */
void oracle_outer_sum(const double* g, const double* X, int64_t T, int64_t N, int64_t d,
                      double* G)
{
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < d; ++k) {
            double s = 0.0;
            for (int64_t t = 0; t < T; ++t) s += g[t * N + n] * X[t * d + k];
            G[n * d + k] = s;
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Full LM-head estimator.                                                   */
/*   logits [T,V], targets [T], X [T,d] -> g_hat [T,V], G_W [V,d].           */
/* Optional diagnostics (NULL to skip): ell [K,T], c [K,T], r [K,T],         */
/* ell0 [T].                                                                 */
/* Returns 0, or -1 on bad arguments / allocation failure.                   */
/* ------------------------------------------------------------------------- */
int oracle_head_estimate(const double* logits, const int32_t* targets, const double* X,
                         int64_t T, int64_t V, int64_t d, int64_t L,
                         double sigma, int64_t K, double gamma,
                         uint64_t seed, uint32_t stream,
                         double* g_hat, double* G_W,
                         double* ell_out, double* c_out, double* r_out, double* ell0_out,
                         double* g_scale_out)
{
    if (T <= 0 || V <= 0 || V % 4 != 0 || d <= 0 || K <= 0 || L <= 0 || T % L != 0)
        return -1;
    double* ell = (double*)malloc(sizeof(double) * (size_t)(K * T));
    double* ell0 = (double*)malloc(sizeof(double) * (size_t)T);
    double* c = (double*)malloc(sizeof(double) * (size_t)(K * T));
    double* r = (double*)malloc(sizeof(double) * (size_t)(K * T));
    if (!ell || !ell0 || !c || !r) { free(ell); free(ell0); free(c); free(r); return -1; }

    /* per-draw losses */
    #pragma omp parallel
    {
        double* a = (double*)malloc(sizeof(double) * (size_t)V);
        double* zp = (double*)malloc(sizeof(double) * (size_t)V);
        double* el = (double*)malloc(sizeof(double) * (size_t)K);
        #pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < T; ++t) {
            head_token_losses(logits + t * V, targets[t], V, sigma, K, seed, stream, t,
                              &ell0[t], el, a, zp);
            for (int64_t i = 0; i < K; ++i) ell[i * T + t] = el[i];
        }
        free(a); free(zp); free(el);
    }
    /* centred loss decrease */
    for (int64_t t = 0; t < T; ++t) centre_token(ell0[t], ell + t, K, T, c + t);
    /* discounted reward */
    oracle_reward_scan(c, K, T, L, gamma, r);
    /* error estimate */
    #pragma omp parallel
    {
        double* a = (double*)malloc(sizeof(double) * (size_t)V);
        #pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < T; ++t)
            error_estimate_token(r, K, T, t, t, V, sigma, seed, stream, g_hat + t * V, a,
                                 g_scale_out ? g_scale_out + t * V : NULL);
        free(a);
    }
    /* weight gradient */
    oracle_outer_sum(g_hat, X, T, V, d, G_W);

    if (ell_out) memcpy(ell_out, ell, sizeof(double) * (size_t)(K * T));
    if (c_out) memcpy(c_out, c, sizeof(double) * (size_t)(K * T));
    if (r_out) memcpy(r_out, r, sizeof(double) * (size_t)(K * T));
    if (ell0_out) memcpy(ell0_out, ell0, sizeof(double) * (size_t)T);
    free(ell); free(ell0); free(c); free(r);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* LM-head error-estimate rows for a subset of tokens (for full-size checks).*/
/* Token t's row needs the losses of tokens t .. end of its sequence when    */
/* gamma > 0 (and of token t alone when gamma = 0); only those are computed. */
/* rows [n_tok, V]; ell_rows [K, n_tok] and scale_rows [n_tok, V] (term      */
/* magnitudes, see error_estimate_token) may be NULL.                        */
/* ------------------------------------------------------------------------- */
int oracle_head_rows(const double* logits, const int32_t* targets,
                     int64_t T, int64_t V, int64_t L,
                     double sigma, int64_t K, double gamma, uint64_t seed, uint32_t stream,
                     const int64_t* tokens, int64_t n_tok,
                     double* rows, double* ell_rows, double* scale_rows)
{
    if (T <= 0 || V <= 0 || V % 4 != 0 || K <= 0 || L <= 0 || T % L != 0) return -1;
    for (int64_t q = 0; q < n_tok; ++q)
        if (tokens[q] < 0 || tokens[q] >= T) return -1;
    int fail = 0;
    #pragma omp parallel
    {
        double* a = (double*)malloc(sizeof(double) * (size_t)V);
        double* zp = (double*)malloc(sizeof(double) * (size_t)V);
        int64_t span_max = (gamma == 0.0) ? 1 : L;
        double* ell = (double*)malloc(sizeof(double) * (size_t)(K * span_max));
        double* c = (double*)malloc(sizeof(double) * (size_t)(K * span_max));
        double* r = (double*)malloc(sizeof(double) * (size_t)(K * span_max));
        if (!a || !zp || !ell || !c || !r) {
            #pragma omp atomic write
            fail = 1;
        } else {
            #pragma omp for schedule(dynamic, 1)
            for (int64_t q = 0; q < n_tok; ++q) {
                int64_t t = tokens[q];
                int64_t seg_end = (t / L + 1) * L;
                int64_t span = (gamma == 0.0) ? 1 : (seg_end - t);
                /* losses and centring for tokens t .. t+span-1 (draw-major, width span) */
                for (int64_t s = 0; s < span; ++s) {
                    double e0;
                    double* el = (double*)malloc(sizeof(double) * (size_t)K);
                    head_token_losses(logits + (t + s) * V, targets[t + s], V, sigma, K, seed,
                                      stream, t + s, &e0, el, a, zp);
                    for (int64_t i = 0; i < K; ++i) ell[i * span + s] = el[i];
                    centre_token(e0, ell + s, K, span, c + s);
                    if (ell_rows && s == 0)
                        for (int64_t i = 0; i < K; ++i) ell_rows[i * n_tok + q] = el[i];
                    free(el);
                }
                /* the suffix t .. seg_end-1 is one (truncated) sequence */
                oracle_reward_scan(c, K, span, span, gamma, r);
                /* r of token t is column 0 of the [K, span] array */
                error_estimate_token(r, K, span, 0, t, V, sigma, seed, stream, rows + q * V, a,
                                     scale_rows ? scale_rows + q * V : NULL);
            }
        }
        free(a); free(zp); free(ell); free(c); free(r);
    }
    return fail ? -1 : 0;
}

/* ------------------------------------------------------------------------- */
/* Hidden linear layer y = W x ([P2] section 2.2): the caller measured the    */
/* centred loss decreases c [K,T] with noise from (seed, stream, draws        */
/* 0..K-1); c is used as given (not re-centred).                              */
/*   X [T,d_in], c [K,T] -> g_hat [T,N], G_W [N,d_in]; r [K,T] optional.      */
/* ------------------------------------------------------------------------- */
int oracle_linear_estimate(const double* X, const double* c,
                           int64_t T, int64_t d_in, int64_t N, int64_t L,
                           double sigma, int64_t K, double gamma,
                           uint64_t seed, uint32_t stream,
                           double* g_hat, double* G_W, double* r_out, double* g_scale_out)
{
    if (T <= 0 || N <= 0 || N % 4 != 0 || d_in <= 0 || K <= 0 || L <= 0 || T % L != 0)
        return -1;
    double* r = (double*)malloc(sizeof(double) * (size_t)(K * T));
    if (!r) return -1;
    oracle_reward_scan(c, K, T, L, gamma, r);
    #pragma omp parallel
    {
        double* a = (double*)malloc(sizeof(double) * (size_t)N);
        #pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < T; ++t)
            error_estimate_token(r, K, T, t, t, N, sigma, seed, stream, g_hat + t * N, a,
                                 g_scale_out ? g_scale_out + t * N : NULL);
        free(a);
    }
    oracle_outer_sum(g_hat, X, T, N, d_in, G_W);
    if (r_out) memcpy(r_out, r, sizeof(double) * (size_t)(K * T));
    free(r);
    return 0;
}

/* Linear-layer error-estimate rows for a subset of tokens; r is scanned
 * from the caller's c over the whole [K,T] array first. rows [n_tok, N];
 * scale_rows [n_tok, N] (term magnitudes) may be NULL. */
int oracle_linear_rows(const double* c, int64_t T, int64_t N, int64_t L,
                       double sigma, int64_t K, double gamma, uint64_t seed, uint32_t stream,
                       const int64_t* tokens, int64_t n_tok, double* rows, double* scale_rows)
{
    if (T <= 0 || N <= 0 || N % 4 != 0 || K <= 0 || L <= 0 || T % L != 0) return -1;
    for (int64_t q = 0; q < n_tok; ++q)
        if (tokens[q] < 0 || tokens[q] >= T) return -1;
    double* r = (double*)malloc(sizeof(double) * (size_t)(K * T));
    if (!r) return -1;
    oracle_reward_scan(c, K, T, L, gamma, r);
    #pragma omp parallel
    {
        double* a = (double*)malloc(sizeof(double) * (size_t)N);
        #pragma omp for schedule(dynamic, 1)
        for (int64_t q = 0; q < n_tok; ++q)
            error_estimate_token(r, K, T, tokens[q], tokens[q], N, sigma, seed, stream,
                                 rows + q * N, a, scale_rows ? scale_rows + q * N : NULL);
        free(a);
    }
    free(r);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Perturbed forward of a hidden linear layer ([P2] sections 2 and 2.1: the   */
/* layer's output y_t = W x_t is jittered to y_t + sigma a_t per token):      */
/*   Y[k][t][n] = sum_j X[t][j] W[n][j] + sigma a^(draw0+k)_t[n].              */
/* X [T,d], W [N,d]; Y [ndraw,T,N].                                           */
/* ------------------------------------------------------------------------- */
int oracle_perturbed_linear(const double* X, const double* W, int64_t T, int64_t d, int64_t N,
                            double sigma, uint64_t seed, uint32_t stream, int64_t draw0,
                            int64_t ndraw, double* Y)
{
    if (T <= 0 || d <= 0 || N <= 0 || N % 4 != 0 || ndraw < 0) return -1;
    #pragma omp parallel
    {
        double* a = (double*)malloc(sizeof(double) * (size_t)N);
        #pragma omp for schedule(static)
        for (int64_t kt = 0; kt < ndraw * T; ++kt) {
            int64_t k = kt / T, t = kt % T;
            noise_row(seed, stream, draw0 + k, t, N, a);
            for (int64_t n = 0; n < N; ++n) {
                double y = 0.0;
                for (int64_t j = 0; j < d; ++j) y += X[t * d + j] * W[n * d + j];
                Y[(k * T + t) * N + n] = y + sigma * a[n];
            }
        }
        free(a);
    }
    return 0;
}

/* Embedding layer ([P2] section 2.2: one-hot input, so the outer product is a
 * scatter-add): G_E[v] = sum_{t: ids[t] = v} g[t]; ids outside [0, vocab)
 * contribute nothing. */
int oracle_embedding_grad(const int32_t* ids, const double* g, int64_t T, int64_t N,
                          int64_t vocab, double* GE)
{
    if (T < 0 || N <= 0 || vocab <= 0) return -1;
    for (int64_t e = 0; e < vocab * N; ++e) GE[e] = 0.0;
    for (int64_t t = 0; t < T; ++t) {
        int32_t v = ids[t];
        if (v < 0 || v >= vocab) continue;
        for (int64_t n = 0; n < N; ++n) GE[v * N + n] += g[t * N + n];
    }
    return 0;
}

/* SGD with momentum (linlog explainer, setup): m = mu m + (G + wd W); W -= lr m. */
void oracle_sgd_momentum(double* W, const double* G, double* m, int64_t n, double lr, double mu,
                         double wd)
{
    for (int64_t i = 0; i < n; ++i) {
        double g = G[i] + wd * W[i];
        m[i] = mu * m[i] + g;
        W[i] -= lr * m[i];
    }
}

/* Adam (paper digest, section 3.3), bias-corrected at step k >= 1. */
void oracle_adam(double* W, const double* G, double* m, double* v, int64_t n, double lr,
                 double b1, double b2, double eps, double wd, int64_t k)
{
    double bc1 = 1.0 - pow(b1, (double)k), bc2 = 1.0 - pow(b2, (double)k);
    for (int64_t i = 0; i < n; ++i) {
        double g = G[i] + wd * W[i];
        m[i] = b1 * m[i] + (1.0 - b1) * g;
        v[i] = b2 * v[i] + (1.0 - b2) * g * g;
        W[i] -= (lr / bc1) * m[i] / (sqrt(v[i]) / sqrt(bc2) + eps);
    }
}

/* Closed-form LM-head gradient: softmax(z_t) - onehot(y_t). */
void oracle_ce_grad(const double* z, const int32_t* y, int64_t T, int64_t V, double* out)
{
    for (int64_t t = 0; t < T; ++t) {
        const double* zr = z + t * V;
        double m = zr[0];
        for (int64_t v = 1; v < V; ++v) if (zr[v] > m) m = zr[v];
        double s = 0.0;
        for (int64_t v = 0; v < V; ++v) s += exp(zr[v] - m);
        for (int64_t v = 0; v < V; ++v)
            out[t * V + v] = exp(zr[v] - m) / s - (v == y[t] ? 1.0 : 0.0);
    }
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
