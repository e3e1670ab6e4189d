/*
 * gdn_oracle.c -- CPU reference (the oracle) for the gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the GPU product path may link, load
 * or call this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code with the HIP library.
 *
 * What it computes: the sequential per-token gated delta rule as the
 * Qwen3.5-9B-npu model page states it ("How it works", paragraph
 * "Gated DeltaNet on the NPU", the four-line per-token update that the
 * exported Loop applies):
 *
 *     S   <- S * exp(g_t)                 (decay the whole state first)
 *     kv  <- S^T k_t                      (read with the decayed state)
 *     S   <- S + k_t (outer) ((v_t - kv) * beta_t)
 *     o_t <- S^T q_t                      (read after the write)
 *
 * S is dk x dv, row index over the key dimension and column index over the
 * value dimension (kv = S^T k has dv entries).  Everything is IEEE fp64 with
 * plain loops: no BLAS, no SIMD intrinsics, no fast-math, no reordering of the
 * four steps.  The chunkwise-parallel prompt form and the one-token matrix form
 * on the same page reach this same result up to rounding order; the oracle is
 * deliberately the plain definition, not either faster form.
 *
 * Parallelism: independent (sequence, head) units are handed to a pthread pool
 * through an atomic counter.  Each unit is computed start to finish by one
 * thread, so the result does not depend on the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* One token of the recurrence on a dk x dv state (row-major, S[i*dv + j]).
 * kv is caller scratch of dv doubles. */
static void gdn_token(double *S, int64_t dk, int64_t dv,
                      const double *q, const double *k, const double *v,
                      double g, double beta, double *o, double *kv)
{
    const double decay = exp(g);
    for (int64_t i = 0; i < dk; ++i)            /* S <- S * exp(g_t) */
        for (int64_t j = 0; j < dv; ++j)
            S[i * dv + j] *= decay;

    for (int64_t j = 0; j < dv; ++j) {          /* kv <- S^T k_t */
        double acc = 0.0;
        for (int64_t i = 0; i < dk; ++i)
            acc += S[i * dv + j] * k[i];
        kv[j] = acc;
    }

    for (int64_t i = 0; i < dk; ++i)            /* S <- S + k_t (x) ((v_t - kv) beta_t) */
        for (int64_t j = 0; j < dv; ++j)
            S[i * dv + j] += k[i] * ((v[j] - kv[j]) * beta);

    for (int64_t j = 0; j < dv; ++j) {          /* o_t <- S^T q_t */
        double acc = 0.0;
        for (int64_t i = 0; i < dk; ++i)
            acc += S[i * dv + j] * q[i];
        o[j] = acc;
    }
}

/* A unit is one (sequence, head): a run of ntok tokens read with fixed strides
 * (in elements) between consecutive tokens, and the state it carries. */
typedef struct {
    const double *q, *k, *v, *g, *beta;
    double *o;
    int64_t ntok;
    int64_t s_qk, s_v, s_gb;   /* token strides for q/k, v/o, g/beta */
    const double *S_in;        /* NULL: zero initial state */
    double *S_out;             /* dk x dv; may equal S_in */
    double *S_tok;             /* NULL, or the state after each token ... */
    int64_t s_st;              /* ... with this stride (elements) between tokens */
} unit_t;

typedef struct {
    unit_t *units;
    int64_t nunits, dk, dv;
    int64_t next;              /* atomic work counter */
    int failed;
} pool_t;

static void run_unit(const unit_t *u, int64_t dk, int64_t dv, double *S, double *kv)
{
    if (u->S_in)
        memcpy(S, u->S_in, (size_t)(dk * dv) * sizeof(double));
    else
        memset(S, 0, (size_t)(dk * dv) * sizeof(double));
    for (int64_t t = 0; t < u->ntok; ++t) {
        gdn_token(S, dk, dv, u->q + t * u->s_qk, u->k + t * u->s_qk,
                  u->v + t * u->s_v, u->g[t * u->s_gb], u->beta[t * u->s_gb],
                  u->o + t * u->s_v, kv);
        if (u->S_tok)
            memcpy(u->S_tok + t * u->s_st, S, (size_t)(dk * dv) * sizeof(double));
    }
    memcpy(u->S_out, S, (size_t)(dk * dv) * sizeof(double));
}

static void *worker(void *arg)
{
    pool_t *p = (pool_t *)arg;
    double *S = (double *)malloc((size_t)(p->dk * p->dv) * sizeof(double));
    double *kv = (double *)malloc((size_t)p->dv * sizeof(double));
    if (!S || !kv) {
        __atomic_store_n(&p->failed, 1, __ATOMIC_SEQ_CST);
        free(S);
        free(kv);
        return NULL;
    }
    for (;;) {
        int64_t u = __atomic_fetch_add(&p->next, 1, __ATOMIC_SEQ_CST);
        if (u >= p->nunits)
            break;
        run_unit(&p->units[u], p->dk, p->dv, S, kv);
    }
    free(S);
    free(kv);
    return NULL;
}

static int run_pool(unit_t *units, int64_t nunits, int64_t dk, int64_t dv, int nthreads)
{
    pool_t p = {units, nunits, dk, dv, 0, 0};
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > nunits)
        nthreads = nunits > 0 ? (int)nunits : 1;
    pthread_t *th = (pthread_t *)malloc((size_t)nthreads * sizeof(pthread_t));
    if (!th)
        return -2;
    int started = 0;
    for (int i = 0; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, worker, &p) != 0)
            break;
        ++started;
    }
    if (started == 0)
        worker(&p);    /* no threads available: run inline */
    for (int i = 0; i < started; ++i)
        pthread_join(th[i], NULL);
    free(th);
    return p.failed ? -2 : 0;
}

/*
 * Whole-sequence run (the prompt case).
 *   q, k : [B, T, H, dk]      v, O : [B, T, H, dv]      g, beta : [B, T, H]
 *   S0   : [N, H, dk, dv] or NULL (zero state)           S_T : [N, H, dk, dv]
 * Without cu_seqlens there are N = B sequences of T tokens each.  With
 * cu_seqlens ([N+1] offsets, non-decreasing, cu_seqlens[N] = T) the tokens are
 * one packed batch (B = 1) and sequence n owns tokens cu_seqlens[n] ..
 * cu_seqlens[n+1]-1; each sequence starts from its own S0 slice.
 * S_T may equal S0 (in-place update).  Returns 0, -1 for bad arguments, -2 for
 * an allocation failure.
 */
static int prefill_units(const double *q, const double *k, const double *v,
                         const double *g, const double *beta, const double *S0,
                         const int64_t *cu_seqlens, int64_t N, int64_t T,
                         int64_t H, int64_t dk, int64_t dv, double *O,
                         double *S_T, double *S_tok, int nthreads)
{
    if (N < 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0 || !S_T)
        return -1;
    if (cu_seqlens) {
        if (cu_seqlens[0] != 0 || cu_seqlens[N] != T)
            return -1;
        for (int64_t n = 0; n < N; ++n)
            if (cu_seqlens[n + 1] < cu_seqlens[n])
                return -1;
    }
    const int64_t nunits = N * H;
    unit_t *units = (unit_t *)calloc((size_t)(nunits > 0 ? nunits : 1), sizeof(unit_t));
    if (!units)
        return -2;
    for (int64_t n = 0; n < N; ++n) {
        /* first token of the sequence, counted in rows of H heads */
        const int64_t start = cu_seqlens ? cu_seqlens[n] : n * T;
        const int64_t len = cu_seqlens ? cu_seqlens[n + 1] - cu_seqlens[n] : T;
        for (int64_t h = 0; h < H; ++h) {
            unit_t *u = &units[n * H + h];
            u->q = q + (start * H + h) * dk;
            u->k = k + (start * H + h) * dk;
            u->v = v + (start * H + h) * dv;
            u->o = O + (start * H + h) * dv;
            u->g = g + start * H + h;
            u->beta = beta + start * H + h;
            u->ntok = len;
            u->s_qk = H * dk;
            u->s_v = H * dv;
            u->s_gb = H;
            u->S_in = S0 ? S0 + (n * H + h) * dk * dv : NULL;
            u->S_out = S_T + (n * H + h) * dk * dv;
            u->S_tok = S_tok ? S_tok + (start * H + h) * dk * dv : NULL;
            u->s_st = H * dk * dv;
        }
    }
    int rc = run_pool(units, nunits, dk, dv, nthreads);
    free(units);
    return rc;
}

int gdn_oracle_prefill(const double *q, const double *k, const double *v,
                       const double *g, const double *beta, const double *S0,
                       const int64_t *cu_seqlens, int64_t N, int64_t T,
                       int64_t H, int64_t dk, int64_t dv, double *O,
                       double *S_T, int nthreads)
{
    return prefill_units(q, k, v, g, beta, S0, cu_seqlens, N, T, H, dk, dv, O, S_T,
                         NULL, nthreads);
}

/*
 * The same run, also keeping the state after every token (what a caller needs
 * to roll back a verify pass to any accepted prefix without a snapshot):
 *   S_tok : [B, T, H, dk, dv] (packed: [1, T, H, dk, dv]); S_tok at token row r
 *           of head h is the state after that token, within its sequence.
 */
int gdn_oracle_prefill_states(const double *q, const double *k, const double *v,
                              const double *g, const double *beta, const double *S0,
                              const int64_t *cu_seqlens, int64_t N, int64_t T,
                              int64_t H, int64_t dk, int64_t dv, double *O,
                              double *S_T, double *S_tok, int nthreads)
{
    if (!S_tok)
        return -1;
    return prefill_units(q, k, v, g, beta, S0, cu_seqlens, N, T, H, dk, dv, O, S_T,
                         S_tok, nthreads);
}

/*
 * Consecutive one-token steps on a batch of states (the decode case).
 *   q, k : [steps, B, H, dk]   v, o : [steps, B, H, dv]   g, beta : [steps, B, H]
 *   S    : [B, H, dk, dv], updated in place across all steps.
 * Step s of unit (b, h) reads token s of that unit; this is the same update as
 * above applied once per call.
 */
int gdn_oracle_decode(const double *q, const double *k, const double *v,
                      const double *g, const double *beta, double *S,
                      int64_t steps, int64_t B, int64_t H, int64_t dk,
                      int64_t dv, double *o, int nthreads)
{
    if (steps < 0 || B < 0 || H <= 0 || dk <= 0 || dv <= 0 || !S)
        return -1;
    const int64_t nunits = B * H;
    unit_t *units = (unit_t *)calloc((size_t)(nunits > 0 ? nunits : 1), sizeof(unit_t));
    if (!units)
        return -2;
    for (int64_t u = 0; u < nunits; ++u) {
        units[u].q = q + u * dk;
        units[u].k = k + u * dk;
        units[u].v = v + u * dv;
        units[u].o = o + u * dv;
        units[u].g = g + u;
        units[u].beta = beta + u;
        units[u].ntok = steps;
        units[u].s_qk = nunits * dk;
        units[u].s_v = nunits * dv;
        units[u].s_gb = nunits;
        units[u].S_in = S + u * dk * dv;
        units[u].S_out = S + u * dk * dv;
    }
    int rc = run_pool(units, nunits, dk, dv, nthreads);
    free(units);
    return rc;
}

/*
 * Gated RMS norm of output rows -- the norm that follows the recurrence inside
 * a Gated DeltaNet block (Qwen3.5-4B -- Hexagon NPU (QHexRT) -- v81 page, the
 * opening description of the text decoder, which lists a short convolution
 * window carried between calls, the recurrent state and a gated RMS norm; the Qwen3.5-9B-npu model page, "How it works" ->
 * "fp16 precision of the DeltaNet output", relies on that norm being
 * scale-invariant with eps scaled by the square of the factor).  Per row of dv
 * values:
 *
 *     r   = 1 / sqrt(mean_j(o_j^2) + eps)
 *     y_j = w_j * (o_j * r) * silu(z_j),     silu(x) = x / (1 + exp(-x))
 *
 *   o, z, y : [rows, dv]     w : [dv] (one weight vector shared by every row)
 */
int gdn_oracle_gated_rmsnorm(const double *o, const double *z, const double *w,
                             int64_t rows, int64_t dv, double eps, double *y)
{
    if (rows < 0 || dv <= 0 || !(eps >= 0.0))
        return -1;
    for (int64_t r = 0; r < rows; ++r) {
        const double *orow = o + r * dv, *zrow = z + r * dv;
        double ss = 0.0;
        for (int64_t j = 0; j < dv; ++j)
            ss += orow[j] * orow[j];
        const double inv = 1.0 / sqrt(ss / (double)dv + eps);
        for (int64_t j = 0; j < dv; ++j) {
            const double silu = zrow[j] / (1.0 + exp(-zrow[j]));
            y[r * dv + j] = w[j] * (orow[j] * inv) * silu;
        }
    }
    return 0;
}

/*
 * Pre-operations of a Gated DeltaNet block, from the per-token projections to
 * the recurrence's inputs (Qwen3.5-4B -- Hexagon NPU (QHexRT) -- v81 page, the
 * opening description of the text decoder: a causal convolution over a short
 * window carried between calls comes before the recurrent state; the QCS6490
 * page's port notes name Softplus among the gate's operations; the gate and
 * write strength enter the recurrence as g <= 0 and beta in (0, 1)).  For every
 * sequence n, head h and each of the three streams x in {q, k, v}, channel c:
 *
 *     conv_t[c] = sum_{j=0}^{K-1} w[c][j] * x_{t-K+1+j}[c]
 *                 (rows before the sequence's first token are the carried FIFO
 *                  state: the K-1 rows that preceded it, oldest first)
 *     y_t[c]    = silu(conv_t[c]),                 silu(u) = u / (1 + exp(-u))
 *     q_t       = y_t / sqrt(sum_c y_t[c]^2 + eps)  (and likewise k_t; v_t = y_t)
 *     g_t       = -softplus(a_t),                  softplus(u) = log(1 + exp(u))
 *     beta_t    = sigmoid(b_t)                     = 1 / (1 + exp(-b_t))
 *
 * and the FIFO state after the call holds the last K-1 raw rows of the
 * concatenation [state_in; x rows of the sequence].
 *
 *   xq, xk : [rows, H, dk]   xv : [rows, H, dv]      (raw projections)
 *   a, b   : [rows, H]
 *   conv_w : [3, H, dmax, K]  (stream s = 0, 1, 2 for q, k, v; dmax = max(dk, dv);
 *                              only the first dk or dv channels are used)
 *   state  : [N, 3, H, K-1, dmax] in, state_out the same shape out (may alias)
 *   cu     : N+1 row offsets (rows = cu[N]); NULL for N sequences of T rows
 *   outputs q, k : [rows, H, dk]  v : [rows, H, dv]  g, beta : [rows, H]
 */
int gdn_oracle_preop(const double *xq, const double *xk, const double *xv,
                     const double *a, const double *b, const double *conv_w,
                     const double *state_in, const int64_t *cu, int64_t N, int64_t T,
                     int64_t H, int64_t dk, int64_t dv, int64_t K, double eps,
                     double *q, double *k, double *v, double *g, double *beta,
                     double *state_out)
{
    if (N < 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0 || K < 1 || !(eps >= 0.0))
        return -1;
    const int64_t dmax = dk > dv ? dk : dv, W = K - 1;
    const double *xs[3] = {xq, xk, xv};
    double *ys[3] = {q, k, v};
    const int64_t ds[3] = {dk, dk, dv};
    double *sout = (double *)malloc((size_t)(N * 3 * H * (W > 0 ? W : 1) * dmax) * sizeof(double));
    double *win = (double *)malloc((size_t)(K * dmax) * sizeof(double));
    double *row = (double *)malloc((size_t)dmax * sizeof(double));
    if (!sout || !win || !row) {
        free(sout); free(win); free(row);
        return -2;
    }
    for (int64_t n = 0; n < N; ++n) {
        const int64_t start = cu ? cu[n] : n * T, len = cu ? cu[n + 1] - cu[n] : T;
        for (int64_t h = 0; h < H; ++h) {
            for (int64_t t = 0; t < len; ++t) {      /* the gates */
                const int64_t i = (start + t) * H + h;
                g[i] = -log1p(exp(a[i]));
                beta[i] = 1.0 / (1.0 + exp(-b[i]));
            }
            for (int s = 0; s < 3; ++s) {
                const int64_t d = ds[s];
                const double *st = state_in + ((n * 3 + s) * H + h) * W * dmax;
                const double *wc = conv_w + (s * H + h) * dmax * K;
                for (int64_t t = 0; t < len; ++t) {
                    /* window rows t-K+1 .. t: from the state before the start */
                    for (int64_t j = 0; j < K; ++j) {
                        const int64_t r = t - (K - 1) + j;      /* row within the sequence */
                        for (int64_t c = 0; c < d; ++c)
                            win[j * dmax + c] = r >= 0 ? xs[s][((start + r) * H + h) * d + c]
                                                       : st[(W + r) * dmax + c];
                    }
                    double ss = 0.0;
                    for (int64_t c = 0; c < d; ++c) {
                        double acc = 0.0;
                        for (int64_t j = 0; j < K; ++j)
                            acc += wc[c * K + j] * win[j * dmax + c];
                        row[c] = acc / (1.0 + exp(-acc));
                        ss += row[c] * row[c];
                    }
                    const double scale = s < 2 ? 1.0 / sqrt(ss + eps) : 1.0;
                    for (int64_t c = 0; c < d; ++c)
                        ys[s][((start + t) * H + h) * d + c] = row[c] * scale;
                }
                /* the FIFO after the call: the last W rows of [state; x rows] */
                double *so = sout + ((n * 3 + s) * H + h) * W * dmax;
                for (int64_t j = 0; j < W; ++j) {
                    const int64_t r = len - W + j;              /* row within the sequence */
                    for (int64_t c = 0; c < dmax; ++c)
                        so[j * dmax + c] = c >= d ? 0.0
                                         : r >= 0 ? xs[s][((start + r) * H + h) * d + c]
                                                  : st[(W + r) * dmax + c];
                }
            }
        }
    }
    memcpy(state_out, sout, (size_t)(N * 3 * H * W * dmax) * sizeof(double));
    free(sout); free(win); free(row);
    return 0;
}
