/*
 * kda_oracle.c -- plain, slow CPU oracle for the Kimi Delta Attention (KDA)
 * operator.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  The HIP product path never
 * links, calls or imports it, and it shares no code, header, table or constant
 * generator with that path.
 *
 * All arithmetic is float64 (one float32 twin of the recurrence exists only to
 * show the float32 noise floor).  Inputs are float32 arrays: bf16 inputs are
 * widened exactly, so both sides see identical values.
 *
 * Pages this follows (cited by title and section):
 *  [K3]  "Kimi K3 architecture" (molayo1419.me), section on the sequence
 *        bottleneck (hybrid KDA and Gated MLA): the lower-bounded log-decay
 *        g = g_min * Sigmoid(e^{A_h} z_t^h), g_min = -5, alpha = exp(g); the
 *        16-token tiles that keep cumulative log-decay inside (-80, 0).
 *  [KL]  "Kimi Linear: An Expressive, Efficient Attention Architecture"
 *        summary (greeksharifa.github.io):
 *          2.1  notation: d_k x d_v memory, length-C chunks, stacked chunk
 *               variables, Tril / StrictTril masks, cumulative decay;
 *          2.2  delta rule as online gradient descent on 1/2||S^T k - v||^2;
 *               Gated DeltaNet with one scalar forget gate per head;
 *          3    the recurrence S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1}
 *               + b_t k_t v_t^T, o_t = S_t^T q_t, decay first, then the
 *               delta correction;
 *          3.1  chunkwise algorithm: WY representation, UT transform,
 *               lower-triangular inverse by forward substitution, output =
 *               incoming-state term + causally masked intra-chunk term;
 *          6.2  the transition as the constrained DPLR matrix
 *               Diag(a_t) - b_t k_t k_t^T Diag(a_t);
 *          6.3  prefill uses the chunk form, generation the recurrent update;
 *          App. B / C  the chunkwise derivation and chunk_kda(q, k, v, g,
 *               beta, initial_state, chunk_size=64) (bodies not printed).
 *
 * Readings where the pages are silent (each is a documented design reading):
 *   - no query scale: o_t = S_t^T q_t;
 *   - the erase uses the decayed state; o_t uses the post-update state;
 *   - A is one scalar per head, z is per (token, head, key channel);
 *   - beta arrives final (already squashed into (0,1));
 *   - NULL initial state means zeros;
 *   - each packed sequence is independent, its chunk grid starts at its own
 *     first token, and the last chunk may be partial.
 *
 * Layouts: q, k, z: [T_total, H, dk]; v: [T_total, H, dv]; beta: [T_total, H];
 * A: [H]; states: [N, H, dk, dv] (row = key channel); o: [T_total, H, dv].
 * cu: host int64 [N+1] sequence offsets into the packed token axis.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define KDA_GMIN (-5.0) /* [K3]: g_min = -5 */

/* ---------------------------------------------------------------- gate -- */

/* [K3] g = g_min * Sigmoid(e^{A_h} * z).  The logistic function is written in
 * its two-branch form so that z = +inf gives exactly g_min and z = -inf gives
 * exactly 0 (alpha = 1); NaN propagates. */
static double gate_one(double expA, double z)
{
    double x = expA * z;
    double s;
    if (x >= 0.0) {
        s = 1.0 / (1.0 + exp(-x));
    } else {
        double e = exp(x);
        s = e / (1.0 + e);
    }
    return KDA_GMIN * s;
}

/* g for n values of z belonging to a head with parameter A. */
void kdao_gate(const float *z, int64_t n, float A, double *g)
{
    double expA = exp((double)A);
    for (int64_t i = 0; i < n; ++i) g[i] = gate_one(expA, (double)z[i]);
}

/* ------------------------------------------------------ thread helpers -- */

typedef struct {
    int64_t ntasks;
    int64_t next; /* atomic task counter */
    void *ctx;
    void (*fn)(void *ctx, int64_t task);
} pool_t;

static void *pool_worker(void *arg)
{
    pool_t *p = (pool_t *)arg;
    for (;;) {
        int64_t t = __atomic_fetch_add(&p->next, 1, __ATOMIC_RELAXED);
        if (t >= p->ntasks) break;
        p->fn(p->ctx, t);
    }
    return NULL;
}

/* Runs fn(ctx, 0..ntasks-1) on up to nthreads threads (<= 0: all online CPUs).
 * Returns the number of threads used. */
static int run_pool(int64_t ntasks, int nthreads, void *ctx, void (*fn)(void *, int64_t))
{
    if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (nthreads < 1) nthreads = 1;
    if ((int64_t)nthreads > ntasks) nthreads = (int)(ntasks > 0 ? ntasks : 1);
    pool_t p = {ntasks, 0, ctx, fn};
    if (nthreads == 1) {
        pool_worker(&p);
        return 1;
    }
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    int started = 0;
    for (int i = 0; i < nthreads; ++i)
        if (pthread_create(&th[i], NULL, pool_worker, &p) == 0) ++started;
    if (started == 0) pool_worker(&p);
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    free(th);
    return started > 0 ? started : 1;
}

/* --------------------------------------------- token recurrence (fp64) -- */

typedef struct {
    const float *q, *k, *v, *z, *beta, *A;
    const double *S0;
    const int64_t *cu;
    int N, H, dk, dv;
    double *o, *S_final;
    const double *g; /* non-NULL: log-decays given directly ([T, H, dk]), z and A unused */
} rec_args;

/* [KL 3] one (sequence, head): for every token, in order,
 *   1. S <- Diag(alpha_t) S                (decay first)
 *   2. p = S^T k_t
 *   3. delta = beta_t (v_t - p)
 *   4. S <- S + k_t delta^T               (the delta-rule correction)
 *   5. o_t = S^T q_t                       (read-out from the updated state)
 */
static void rec_task_f64(void *vctx, int64_t task)
{
    const rec_args *a = (const rec_args *)vctx;
    const int n = (int)(task / a->H), h = (int)(task % a->H);
    const int dk = a->dk, dv = a->dv, H = a->H;
    double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
    double *alpha = (double *)malloc(sizeof(double) * (size_t)dk);
    double *p = (double *)malloc(sizeof(double) * (size_t)dv);
    double *d = (double *)malloc(sizeof(double) * (size_t)dv);
    const size_t sidx = ((size_t)n * H + h) * (size_t)dk * dv;
    if (a->S0)
        memcpy(S, a->S0 + sidx, sizeof(double) * (size_t)dk * dv);
    else
        memset(S, 0, sizeof(double) * (size_t)dk * dv);
    const double expA = a->A ? exp((double)a->A[h]) : 0.0;

    for (int64_t t = a->cu[n]; t < a->cu[n + 1]; ++t) {
        const float *qt = a->q + ((size_t)t * H + h) * dk;
        const float *kt = a->k + ((size_t)t * H + h) * dk;
        const float *zt = a->z ? a->z + ((size_t)t * H + h) * dk : NULL;
        const float *vt = a->v + ((size_t)t * H + h) * dv;
        const double bt = (double)a->beta[(size_t)t * H + h];
        double *ot = a->o + ((size_t)t * H + h) * dv;

        if (a->g) {
            const double *gt = a->g + ((size_t)t * H + h) * dk;
            for (int i = 0; i < dk; ++i) alpha[i] = exp(gt[i]);
        } else {
            for (int i = 0; i < dk; ++i) alpha[i] = exp(gate_one(expA, (double)zt[i]));
        }
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= alpha[i];
        for (int j = 0; j < dv; ++j) p[j] = 0.0;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) p[j] += (double)kt[i] * S[(size_t)i * dv + j];
        for (int j = 0; j < dv; ++j) d[j] = bt * ((double)vt[j] - p[j]);
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += (double)kt[i] * d[j];
        for (int j = 0; j < dv; ++j) ot[j] = 0.0;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) ot[j] += (double)qt[i] * S[(size_t)i * dv + j];
    }
    if (a->S_final) memcpy(a->S_final + sidx, S, sizeof(double) * (size_t)dk * dv);
    free(S);
    free(alpha);
    free(p);
    free(d);
}

/* The reference for all parity.  S0 may be NULL (zeros) and may alias S_final.
 * Returns the number of threads used. */
int kdao_recurrent(const float *q, const float *k, const float *v, const float *z,
                   const float *beta, const float *A, const double *S0, const int64_t *cu,
                   int N, int H, int dk, int dv, double *o, double *S_final, int nthreads)
{
    rec_args a = {q, k, v, z, beta, A, S0, cu, N, H, dk, dv, o, S_final, NULL};
    return run_pool((int64_t)N * H, nthreads, &a, rec_task_f64);
}

/* The same recurrence with the log-decays g given directly (any decay
 * parameterisation: alpha = e^g).  Returns the number of threads used. */
int kdao_recurrent_g(const float *q, const float *k, const float *v, const double *g, const float *beta,
                     const double *S0, const int64_t *cu, int N, int H, int dk, int dv, double *o,
                     double *S_final, int nthreads)
{
    rec_args a = {q, k, v, NULL, beta, NULL, S0, cu, N, H, dk, dv, o, S_final, g};
    return run_pool((int64_t)N * H, nthreads, &a, rec_task_f64);
}

/* ------------------------------------- token recurrence, float32 twin -- */

typedef struct {
    const float *q, *k, *v, *z, *beta, *A;
    const float *S0;
    const int64_t *cu;
    int N, H, dk, dv;
    float *o, *S_final;
} rec32_args;

/* The same five steps in float32 arithmetic (noise-floor reference only). */
static void rec_task_f32(void *vctx, int64_t task)
{
    const rec32_args *a = (const rec32_args *)vctx;
    const int n = (int)(task / a->H), h = (int)(task % a->H);
    const int dk = a->dk, dv = a->dv, H = a->H;
    float *S = (float *)malloc(sizeof(float) * (size_t)dk * dv);
    float *alpha = (float *)malloc(sizeof(float) * (size_t)dk);
    float *p = (float *)malloc(sizeof(float) * (size_t)dv);
    float *d = (float *)malloc(sizeof(float) * (size_t)dv);
    const size_t sidx = ((size_t)n * H + h) * (size_t)dk * dv;
    if (a->S0)
        memcpy(S, a->S0 + sidx, sizeof(float) * (size_t)dk * dv);
    else
        memset(S, 0, sizeof(float) * (size_t)dk * dv);
    const float expA = expf(a->A[h]);
    for (int64_t t = a->cu[n]; t < a->cu[n + 1]; ++t) {
        const float *qt = a->q + ((size_t)t * H + h) * dk;
        const float *kt = a->k + ((size_t)t * H + h) * dk;
        const float *zt = a->z + ((size_t)t * H + h) * dk;
        const float *vt = a->v + ((size_t)t * H + h) * dv;
        const float bt = a->beta[(size_t)t * H + h];
        float *ot = a->o + ((size_t)t * H + h) * dv;
        for (int i = 0; i < dk; ++i) {
            float x = expA * zt[i], s;
            if (x >= 0.0f) {
                s = 1.0f / (1.0f + expf(-x));
            } else {
                float e = expf(x);
                s = e / (1.0f + e);
            }
            alpha[i] = expf((float)KDA_GMIN * s);
        }
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= alpha[i];
        for (int j = 0; j < dv; ++j) p[j] = 0.0f;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) p[j] += kt[i] * S[(size_t)i * dv + j];
        for (int j = 0; j < dv; ++j) d[j] = bt * (vt[j] - p[j]);
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += kt[i] * d[j];
        for (int j = 0; j < dv; ++j) ot[j] = 0.0f;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) ot[j] += qt[i] * S[(size_t)i * dv + j];
    }
    if (a->S_final) memcpy(a->S_final + sidx, S, sizeof(float) * (size_t)dk * dv);
    free(S);
    free(alpha);
    free(p);
    free(d);
}

int kdao_recurrent_f32(const float *q, const float *k, const float *v, const float *z,
                       const float *beta, const float *A, const float *S0, const int64_t *cu,
                       int N, int H, int dk, int dv, float *o, float *S_final, int nthreads)
{
    rec32_args a = {q, k, v, z, beta, A, S0, cu, N, H, dk, dv, o, S_final};
    return run_pool((int64_t)N * H, nthreads, &a, rec_task_f32);
}

/* ------------------------------------------------- chunk form (fp64) -- */

/*
 * One chunk of n (<= C) tokens of one head, following [KL 2.1, 3.1, App. B/C]
 * as derived from the recurrence.  Let G_r = sum_{s<=r} g_s (per key channel,
 * inclusive, restarting at each chunk) and Gam_r = e^{G_r}.  Unrolling the
 * recurrence inside the chunk from the incoming state S gives
 *     S_r = Diag(Gam_r) S + sum_{c<=r} Diag(Gam_r / Gam_c) k_c delta_c^T,
 * with delta_r = beta_r (v_r - (Diag(alpha_r) S_{r-1})^T k_r).  Hence
 *     delta_r + sum_{c<r} Akk[r,c] delta_c = beta_r v_r - beta_r (k_r*Gam_r)^T S
 * where Akk[r,c] = beta_r sum_j k_rj k_cj e^{G_rj - G_cj} (StrictTril).  The
 * UT transform T = (I + Akk)^{-1} (forward substitution, row by row) yields
 * the WY vectors W = T diag(beta) (K*Gam), U = T diag(beta) V and
 *     Delta = U - W S,
 *     O     = (Q*Gam) S + (Aqk * Tril) Delta,
 *            Aqk[r,c] = sum_j q_rj k_cj e^{G_rj - G_cj},
 *     S'    = Diag(Gam_{n-1}) S + (K * e^{G_{n-1} - G})^T Delta.
 *
 * shaped != 0 evaluates every e^{G_r - G_c} as e^{G_r - R_i} * e^{R_i - G_c}
 * with R_i = G just before the first token of the sub-chunk of row r
 * (0 for the first sub-chunk) [K3 16-token tiles]; shaped == 0 evaluates the
 * difference directly.  Both are exact in real arithmetic.
 *
 * Inputs are row pointers with row stride rs (elements between consecutive
 * tokens of the same head).  S (dk x dv) is updated in place; o receives the
 * chunk's n output rows with row stride os.  Every *_out argument may be NULL;
 * otherwise it receives the intermediate (G n x dk, Akk / T / Aqk n x n,
 * W n x dk, U / Delta n x dv), densely packed.
 */
void kdao_chunk_step(const float *q, const float *k, const float *v, const float *z,
                     const float *beta, int64_t rs, int64_t bs, float A, int n, int dk, int dv,
                     int sub, int shaped, double *S, double *o, int64_t os, double *G_out,
                     double *Akk_out, double *T_out, double *W_out, double *U_out,
                     double *Aqk_out, double *Delta_out)
{
    const double expA = exp((double)A);
    double *G = (double *)calloc((size_t)n * dk, sizeof(double));
    double *Akk = (double *)calloc((size_t)n * n, sizeof(double));
    double *Aqk = (double *)calloc((size_t)n * n, sizeof(double));
    double *T = (double *)calloc((size_t)n * n, sizeof(double));
    double *W = (double *)calloc((size_t)n * dk, sizeof(double));
    double *U = (double *)calloc((size_t)n * dv, sizeof(double));
    double *Dl = (double *)calloc((size_t)n * dv, sizeof(double));
    double *Snew = (double *)calloc((size_t)dk * dv, sizeof(double));
#define Q_(r, j) ((double)q[(size_t)(r) * rs + (j)])
#define K_(r, j) ((double)k[(size_t)(r) * rs + (j)])
#define V_(r, j) ((double)v[(size_t)(r) * rs + (j)])
#define B_(r) ((double)beta[(size_t)(r) * bs])

    /* cumulative log-decay inside the chunk (inclusive) */
    for (int r = 0; r < n; ++r)
        for (int j = 0; j < dk; ++j) {
            double g = gate_one(expA, (double)z[(size_t)r * rs + j]);
            G[(size_t)r * dk + j] = (r ? G[(size_t)(r - 1) * dk + j] : 0.0) + g;
        }

    /* decay factor between positions c <= r for channel j */
#define DECAY(r, c, j)                                                                    \
    (shaped ? exp(G[(size_t)(r) * dk + (j)] - REF(r, j)) * exp(REF(r, j) - G[(size_t)(c) * dk + (j)]) \
            : exp(G[(size_t)(r) * dk + (j)] - G[(size_t)(c) * dk + (j)]))
#define REF(r, j) (((r) / sub) * sub == 0 ? 0.0 : G[(size_t)(((r) / sub) * sub - 1) * dk + (j)])

    /* the two decay-scaled Gram matrices */
    for (int r = 0; r < n; ++r)
        for (int c = 0; c <= r; ++c) {
            double skk = 0.0, sqk = 0.0;
            for (int j = 0; j < dk; ++j) {
                double e = DECAY(r, c, j);
                skk += K_(r, j) * K_(c, j) * e;
                sqk += Q_(r, j) * K_(c, j) * e;
            }
            if (c < r) Akk[(size_t)r * n + c] = B_(r) * skk;
            Aqk[(size_t)r * n + c] = sqk;
        }

    /* T = (I + Akk)^{-1} by forward substitution: T[r,:] = e_r - sum_{c<r} Akk[r,c] T[c,:] */
    for (int r = 0; r < n; ++r) {
        for (int m = 0; m < n; ++m) T[(size_t)r * n + m] = (m == r) ? 1.0 : 0.0;
        for (int c = 0; c < r; ++c) {
            double a = Akk[(size_t)r * n + c];
            for (int m = 0; m <= c; ++m) T[(size_t)r * n + m] -= a * T[(size_t)c * n + m];
        }
    }

    /* WY vectors: W = T diag(beta) (K * Gam), U = T diag(beta) V */
    for (int r = 0; r < n; ++r) {
        for (int c = 0; c <= r; ++c) {
            double tb = T[(size_t)r * n + c] * B_(c);
            for (int j = 0; j < dk; ++j) W[(size_t)r * dk + j] += tb * K_(c, j) * exp(G[(size_t)c * dk + j]);
            for (int j = 0; j < dv; ++j) U[(size_t)r * dv + j] += tb * V_(c, j);
        }
    }

    /* Delta = U - W S */
    for (int r = 0; r < n; ++r)
        for (int j = 0; j < dv; ++j) {
            double s = U[(size_t)r * dv + j];
            for (int i = 0; i < dk; ++i) s -= W[(size_t)r * dk + i] * S[(size_t)i * dv + j];
            Dl[(size_t)r * dv + j] = s;
        }

    /* O = (Q * Gam) S + (Aqk * Tril) Delta */
    for (int r = 0; r < n; ++r)
        for (int j = 0; j < dv; ++j) {
            double s = 0.0;
            for (int i = 0; i < dk; ++i) s += Q_(r, i) * exp(G[(size_t)r * dk + i]) * S[(size_t)i * dv + j];
            for (int c = 0; c <= r; ++c) s += Aqk[(size_t)r * n + c] * Dl[(size_t)c * dv + j];
            o[(size_t)r * os + j] = s;
        }

    /* S' = Diag(Gam_last) S + (K * e^{G_last - G})^T Delta */
    for (int i = 0; i < dk; ++i) {
        double gl = G[(size_t)(n - 1) * dk + i];
        for (int j = 0; j < dv; ++j) {
            double s = exp(gl) * S[(size_t)i * dv + j];
            for (int c = 0; c < n; ++c)
                s += K_(c, i) * exp(gl - G[(size_t)c * dk + i]) * Dl[(size_t)c * dv + j];
            Snew[(size_t)i * dv + j] = s;
        }
    }
    memcpy(S, Snew, sizeof(double) * (size_t)dk * dv);

    if (G_out) memcpy(G_out, G, sizeof(double) * (size_t)n * dk);
    if (Akk_out) memcpy(Akk_out, Akk, sizeof(double) * (size_t)n * n);
    if (T_out) memcpy(T_out, T, sizeof(double) * (size_t)n * n);
    if (W_out) memcpy(W_out, W, sizeof(double) * (size_t)n * dk);
    if (U_out) memcpy(U_out, U, sizeof(double) * (size_t)n * dv);
    if (Aqk_out) memcpy(Aqk_out, Aqk, sizeof(double) * (size_t)n * n);
    if (Delta_out) memcpy(Delta_out, Dl, sizeof(double) * (size_t)n * dv);
#undef Q_
#undef K_
#undef V_
#undef B_
#undef DECAY
#undef REF
    free(G);
    free(Akk);
    free(Aqk);
    free(T);
    free(W);
    free(U);
    free(Dl);
    free(Snew);
}

typedef struct {
    const float *q, *k, *v, *z, *beta, *A;
    const double *S0;
    const int64_t *cu;
    int N, H, dk, dv, C, sub, shaped;
    double *o, *S_final;
} chunk_args;

/* [KL 2.1] each chunk starts from the previous chunk's final state; the chunk
 * grid of a sequence starts at its first token and its last chunk may be
 * partial. */
static void chunk_task(void *vctx, int64_t task)
{
    const chunk_args *a = (const chunk_args *)vctx;
    const int n = (int)(task / a->H), h = (int)(task % a->H);
    const int H = a->H, dk = a->dk, dv = a->dv;
    const size_t sidx = ((size_t)n * H + h) * (size_t)dk * dv;
    double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
    if (a->S0)
        memcpy(S, a->S0 + sidx, sizeof(double) * (size_t)dk * dv);
    else
        memset(S, 0, sizeof(double) * (size_t)dk * dv);
    for (int64_t c0 = a->cu[n]; c0 < a->cu[n + 1]; c0 += a->C) {
        int len = (int)((a->cu[n + 1] - c0) < a->C ? (a->cu[n + 1] - c0) : a->C);
        size_t off = ((size_t)c0 * H + h);
        kdao_chunk_step(a->q + off * dk, a->k + off * dk, a->v + off * dv, a->z + off * dk,
                        a->beta + off, (int64_t)H * dk, H, a->A[h], len, dk, dv, a->sub, a->shaped,
                        S, a->o + off * dv, (int64_t)H * dv, NULL, NULL, NULL, NULL, NULL, NULL, NULL);
    }
    if (a->S_final) memcpy(a->S_final + sidx, S, sizeof(double) * (size_t)dk * dv);
    free(S);
}

/* Chunk form over a packed batch (requires dk == dv for the strided views
 * above to share one row stride; the KDA head has dk = dv = 128). */
int kdao_chunk(const float *q, const float *k, const float *v, const float *z, const float *beta,
               const float *A, const double *S0, const int64_t *cu, int N, int H, int dk, int dv,
               int C, int sub, int shaped, double *o, double *S_final, int nthreads)
{
    if (dk != dv || C < 1 || sub < 1) return -1;
    chunk_args a = {q, k, v, z, beta, A, S0, cu, N, H, dk, dv, C, sub, shaped, o, S_final};
    return run_pool((int64_t)N * H, nthreads, &a, chunk_task);
}

/* ------------------------------------------- brute force (dense DPLR) -- */

/*
 * [KL 6.2] the transition written as the dense d_k x d_k matrix
 *     M_t = Diag(alpha_t) - beta_t k_t k_t^T Diag(alpha_t),
 * so S_t = M_t S_{t-1} + beta_t k_t v_t^T.  With the explicit products
 * P_{t,s} = M_t ... M_{s+1} (P_{t,t} = I):
 *     o_t = (P_{t,0} S0)^T q_t + sum_{s<=t} (q_t^T P_{t,s} k_s) beta_s v_s,
 *     S_T = P_{T,0} S0 + sum_s P_{T,s} k_s beta_s v_s^T.
 * One head, one sequence of T tokens; q, k, z: [T, dk]; v: [T, dv]; beta: [T];
 * S0: [dk, dv] or NULL.  No rank-1 shortcut, no chunking.
 */
int kdao_bruteforce(const float *q, const float *k, const float *v, const float *z,
                    const float *beta, float A, const double *S0, int T, int dk, int dv,
                    double *o, double *S_final)
{
    if (T < 0 || T > 64) return -1;
    const double expA = exp((double)A);
    const size_t mm = (size_t)dk * dk;
    double *M = (double *)malloc(sizeof(double) * mm * (size_t)(T + 1));  /* M[t], t = 1..T */
    double *P = (double *)malloc(sizeof(double) * mm * (size_t)(T + 1) * (T + 1));
    double *tmp = (double *)malloc(sizeof(double) * mm);
    double *PS = (double *)malloc(sizeof(double) * (size_t)dk * dv);
#define PM(t, s) (P + ((size_t)(t) * (T + 1) + (s)) * mm)
    for (int t = 1; t <= T; ++t) {
        const float *kt = k + (size_t)(t - 1) * dk;
        const double bt = (double)beta[t - 1];
        double *Mt = M + (size_t)t * mm;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dk; ++j) {
                double al = exp(gate_one(expA, (double)z[(size_t)(t - 1) * dk + j]));
                Mt[(size_t)i * dk + j] = ((i == j) ? al : 0.0) - bt * (double)kt[i] * (double)kt[j] * al;
            }
    }
    for (int t = 0; t <= T; ++t) {
        double *Ptt = PM(t, t);
        for (size_t e = 0; e < mm; ++e) Ptt[e] = 0.0;
        for (int i = 0; i < dk; ++i) Ptt[(size_t)i * dk + i] = 1.0;
        for (int s = 0; s < t; ++s) { /* P_{t,s} = M_t P_{t-1,s} */
            const double *Mt = M + (size_t)t * mm, *Pp = PM(t - 1, s);
            double *Pts = PM(t, s);
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dk; ++j) {
                    double acc = 0.0;
                    for (int l = 0; l < dk; ++l) acc += Mt[(size_t)i * dk + l] * Pp[(size_t)l * dk + j];
                    Pts[(size_t)i * dk + j] = acc;
                }
        }
    }
    for (int t = 1; t <= T; ++t) {
        const float *qt = q + (size_t)(t - 1) * dk;
        double *ot = o + (size_t)(t - 1) * dv;
        for (int j = 0; j < dv; ++j) ot[j] = 0.0;
        if (S0) { /* (P_{t,0} S0)^T q_t */
            const double *P0 = PM(t, 0);
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) {
                    double acc = 0.0;
                    for (int l = 0; l < dk; ++l) acc += P0[(size_t)i * dk + l] * S0[(size_t)l * dv + j];
                    PS[(size_t)i * dv + j] = acc;
                }
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) ot[j] += (double)qt[i] * PS[(size_t)i * dv + j];
        }
        for (int s = 1; s <= t; ++s) {
            const double *Pts = PM(t, s);
            const float *ks = k + (size_t)(s - 1) * dk;
            const float *vs = v + (size_t)(s - 1) * dv;
            double w = 0.0; /* q_t^T P_{t,s} k_s */
            for (int i = 0; i < dk; ++i)
                for (int l = 0; l < dk; ++l) w += (double)qt[i] * Pts[(size_t)i * dk + l] * (double)ks[l];
            w *= (double)beta[s - 1];
            for (int j = 0; j < dv; ++j) ot[j] += w * (double)vs[j];
        }
    }
    if (S_final) {
        const double *P0 = PM(T, 0);
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) {
                double acc = 0.0;
                if (S0)
                    for (int l = 0; l < dk; ++l) acc += P0[(size_t)i * dk + l] * S0[(size_t)l * dv + j];
                S_final[(size_t)i * dv + j] = acc;
            }
        for (int s = 1; s <= T; ++s) {
            const double *Pts = PM(T, s);
            const float *ks = k + (size_t)(s - 1) * dk;
            const float *vs = v + (size_t)(s - 1) * dv;
            for (int i = 0; i < dk; ++i) {
                double pk = 0.0;
                for (int l = 0; l < dk; ++l) pk += Pts[(size_t)i * dk + l] * (double)ks[l];
                pk *= (double)beta[s - 1];
                for (int j = 0; j < dv; ++j) S_final[(size_t)i * dv + j] += pk * (double)vs[j];
            }
        }
    }
#undef PM
    free(M);
    free(P);
    free(tmp);
    free(PS);
    return 0;
}

/* ------------------------------------------- Gated DeltaNet (scalar) -- */

/*
 * [KL 2.2] Gated DeltaNet: one scalar forget gate alpha_t per head.  Written
 * independently of the KDA recurrence (erase on the undecayed state, then
 * decay, which is the same map when alpha is a scalar):
 *     S <- alpha_t (S - beta_t k_t (k_t^T S)) + beta_t k_t v_t^T,  o_t = S^T q_t.
 * One head, one sequence; alpha: [T].
 */
void kdao_gdn(const float *q, const float *k, const float *v, const double *alpha,
              const float *beta, const double *S0, int T, int dk, int dv, double *o,
              double *S_final)
{
    double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
    double *kS = (double *)malloc(sizeof(double) * (size_t)dv);
    if (S0)
        memcpy(S, S0, sizeof(double) * (size_t)dk * dv);
    else
        memset(S, 0, sizeof(double) * (size_t)dk * dv);
    for (int t = 0; t < T; ++t) {
        const float *qt = q + (size_t)t * dk, *kt = k + (size_t)t * dk, *vt = v + (size_t)t * dv;
        const double b = (double)beta[t], al = alpha[t];
        for (int j = 0; j < dv; ++j) {
            double s = 0.0;
            for (int i = 0; i < dk; ++i) s += (double)kt[i] * S[(size_t)i * dv + j];
            kS[j] = s;
        }
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) {
                double e = S[(size_t)i * dv + j] - b * (double)kt[i] * kS[j];
                S[(size_t)i * dv + j] = al * e + b * (double)kt[i] * (double)vt[j];
            }
        for (int j = 0; j < dv; ++j) {
            double s = 0.0;
            for (int i = 0; i < dk; ++i) s += (double)qt[i] * S[(size_t)i * dv + j];
            o[(size_t)t * dv + j] = s;
        }
    }
    if (S_final) memcpy(S_final, S, sizeof(double) * (size_t)dk * dv);
    free(S);
    free(kS);
}
