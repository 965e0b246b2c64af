/*
 * gdr_oracle.c -- test infrastructure, NOT part of the product path.
 *
 * Plain, slow, obviously-correct CPU oracle for the gated delta rule, in fp64.
 * Only the tests, the smoke check and the bench's CPU-baseline leg load it.
 *
 * What it computes (column vectors, state S in R^{d_v x d_k}, stored S[v][c]):
 *
 *   scalar gate (Gated DeltaNet):  S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T
 *   channel gate (KDA):            S_t = S_{t-1} Diag(a_t) (I - b_t k_t k_t^T) + b_t v_t k_t^T
 *   output:                        o_t = S_t q_t
 *
 * with a_t = exp(g_t) (g is the log-decay the library takes) and b_t = beta_t.
 * Sources: "Linear Attention, Visualized" (snowchord.com), sections "Recurrent
 * form", "Gated DeltaNet (GDN)" (note "Decay also changes the correction rows":
 * u_t = b_t (v_t - a_t k_t S_{t-1}) in that page's row convention) and "Kimi
 * Delta Attention (KDA)" (decay channel by channel first, then the delta
 * correction); "Gated DeltaNet: Householder Transitions..." (mohakchugh.is-a.dev),
 * section "The gated delta rule"; the video-delta-rule post, Preliminaries.
 *
 * Each token is processed in the order those sections give:
 *   1. decay        S <- a_t S            (KDA: column c scaled by a_t[c])
 *   2. prediction   p = S k_t             (uses the decayed state)
 *   3. correction   u = b_t (v_t - p)
 *   4. write        S <- S + u k_t^T
 *   5. read         o_t = S q_t           (after the write)
 * Steps 1-4 expand to a S (I - b k k^T) + b v k^T exactly.
 *
 * Inputs are float32 arrays holding the exact values given to the GPU (bf16
 * values are exactly representable in float32); every element is widened to
 * double before use and all arithmetic is double.  No blocking, no fusion.
 *
 * Layouts (row-major, contiguous):
 *   q, k  [BH][T][d_k]     v [BH][T][d_v]     beta [BH][T]
 *   g     [BH][T] (scalar gate) or [BH][T][d_k] (channel gate)
 *   S0    [BH][d_v][d_k] (double) or NULL for zeros
 *   o     [BH][T][d_v] (double)   S_final [BH][d_v][d_k] (double)
 * BH = B*H independent sequences, processed in parallel with OpenMP.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_GATE_SCALAR 0
#define ORACLE_GATE_CHANNEL 1

/* One token of the recurrence on one sequence's state S[d_v][d_k]. */
static void token_step(int dk, int dv, int gate, const float *q, const float *k,
                       const float *v, const float *g, double beta, double *S,
                       double *o, double *u)
{
    /* 1. decay */
    if (gate == ORACLE_GATE_SCALAR) {
        double a = exp((double)g[0]);
        for (int i = 0; i < dv * dk; ++i) S[i] *= a;
    } else {
        for (int c = 0; c < dk; ++c) {
            double a = exp((double)g[c]);
            for (int r = 0; r < dv; ++r) S[r * dk + c] *= a;
        }
    }
    /* 2-3. prediction from the decayed state, scaled correction */
    for (int r = 0; r < dv; ++r) {
        double p = 0.0;
        for (int c = 0; c < dk; ++c) p += S[r * dk + c] * (double)k[c];
        u[r] = beta * ((double)v[r] - p);
    }
    /* 4. rank-one write */
    for (int r = 0; r < dv; ++r)
        for (int c = 0; c < dk; ++c) S[r * dk + c] += u[r] * (double)k[c];
    /* 5. read after the write */
    if (o) {
        for (int r = 0; r < dv; ++r) {
            double acc = 0.0;
            for (int c = 0; c < dk; ++c) acc += S[r * dk + c] * (double)q[c];
            o[r] = acc;
        }
    }
}

/*
 * Full token recurrence over T tokens for BH independent sequences.
 * Returns 0 on success, -1 on bad arguments, -2 on allocation failure.
 */
int oracle_gdr_forward(long BH, long T, int dk, int dv, int gate,
                       const float *q, const float *k, const float *v,
                       const float *g, const float *beta, const double *S0,
                       double *o, double *S_final, int nthreads)
{
    if (BH < 0 || T < 0 || dk <= 0 || dv <= 0) return -1;
    if (gate != ORACLE_GATE_SCALAR && gate != ORACLE_GATE_CHANNEL) return -1;
    if (!S_final) return -1;
    if (T > 0 && (!q || !k || !v || !g || !beta || !o)) return -1;
    const long gstride = (gate == ORACLE_GATE_SCALAR) ? 1 : dk;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
#endif
    for (long bh = 0; bh < BH; ++bh) {
        double *S = S_final + bh * (long)dv * dk;
        double *u = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!u) { failed |= 1; continue; }
        if (S0) memcpy(S, S0 + bh * (long)dv * dk, sizeof(double) * (size_t)dv * dk);
        else memset(S, 0, sizeof(double) * (size_t)dv * dk);
        for (long t = 0; t < T; ++t) {
            const long tok = bh * T + t;
            token_step(dk, dv, gate, q + tok * dk, k + tok * dk, v + tok * dv,
                       g + tok * gstride, (double)beta[tok], S, o + tok * dv, u);
        }
        free(u);
    }
    return failed ? -2 : 0;
}

/*
 * One decode step: the same token update applied in place to resident states.
 *   q, k [NH][d_k]; v [NH][d_v]; beta [NH]; g [NH] or [NH][d_k];
 *   S [NH][d_v][d_k] (double, updated in place); o [NH][d_v] (double).
 */
int oracle_gdr_decode_step(long NH, int dk, int dv, int gate,
                           const float *q, const float *k, const float *v,
                           const float *g, const float *beta, double *S,
                           double *o, int nthreads)
{
    if (NH < 0 || dk <= 0 || dv <= 0 || !S || !o) return -1;
    if (gate != ORACLE_GATE_SCALAR && gate != ORACLE_GATE_CHANNEL) return -1;
    if (NH > 0 && (!q || !k || !v || !g || !beta)) return -1;
    const long gstride = (gate == ORACLE_GATE_SCALAR) ? 1 : dk;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static) reduction(| : failed)
#endif
    for (long n = 0; n < NH; ++n) {
        double *u = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!u) { failed |= 1; continue; }
        token_step(dk, dv, gate, q + n * dk, k + n * dk, v + n * dv, g + n * gstride,
                   (double)beta[n], S + n * (long)dv * dk, o + n * dv, u);
        free(u);
    }
    return failed ? -2 : 0;
}

/*
 * Gated Delta Product, token by token, in the page's own (row-vector) notation:
 * "Linear Attention, Visualized", section "Gated Delta Product (GDP)".
 *
 * The page keeps the state as P = S^T in R^{d_k x d_v} (rows = key channels).  Each real
 * token t carries n_h substeps j with their own k_{t,j}, v_{t,j}, beta_{t,j}; with
 *     A_{t,j} = I - beta_{t,j} k_{t,j}^T k_{t,j}      (d_k x d_k, formed explicitly here)
 *     X_{t,j} = beta_{t,j} k_{t,j}^T v_{t,j}          (d_k x d_v)
 * the token update is
 *     P_{t,0} = a_t P_{t-1},   P_{t,j} = A_{t,j} P_{t,j-1} + X_{t,j} (j = 1..n_h),
 *     P_t = P_{t,n_h},         o_t = q_t P_t.
 * The decay acts once, before the first substep; the query reads after the last.
 *
 * Layouts (row-major, contiguous):
 *   q [BH][T][d_k]   k [BH][T][n_h][d_k]   v [BH][T][n_h][d_v]   beta [BH][T][n_h]
 *   g [BH][T] (log-decay, a_t = exp(g_t))
 *   S0, S_final [BH][d_v][d_k] (double; the library's S = P^T), S0 may be NULL
 *   o [BH][T][d_v] (double)
 * Returns 0 on success, -1 on bad arguments, -2 on allocation failure.
 */
int oracle_gdp_forward(long BH, long T, int nh, int dk, int dv,
                       const float *q, const float *k, const float *v,
                       const float *g, const float *beta, const double *S0,
                       double *o, double *S_final, int nthreads)
{
    if (BH < 0 || T < 0 || nh <= 0 || dk <= 0 || dv <= 0 || !S_final) return -1;
    if (T > 0 && (!q || !k || !v || !g || !beta || !o)) return -1;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
#endif
    for (long bh = 0; bh < BH; ++bh) {
        double *P = (double *)malloc(sizeof(double) * (size_t)dk * dv);   /* P[c][r]  */
        double *Pn = (double *)malloc(sizeof(double) * (size_t)dk * dv);
        double *A = (double *)malloc(sizeof(double) * (size_t)dk * dk);   /* A[c][c'] */
        if (!P || !Pn || !A) { free(P); free(Pn); free(A); failed |= 1; continue; }
        double *Sf = S_final + bh * (long)dv * dk;
        for (int c = 0; c < dk; ++c)
            for (int r = 0; r < dv; ++r)
                P[c * dv + r] = S0 ? S0[bh * (long)dv * dk + (long)r * dk + c] : 0.0;
        for (long t = 0; t < T; ++t) {
            const long tok = bh * T + t;
            /* P_{t,0} = a_t P_{t-1} */
            const double a = exp((double)g[tok]);
            for (int i = 0; i < dk * dv; ++i) P[i] *= a;
            for (int jj = 0; jj < nh; ++jj) {
                const long sub = tok * nh + jj;
                const float *kk = k + sub * dk, *vv = v + sub * dv;
                const double b = (double)beta[sub];
                /* A_{t,j} = I - b k^T k */
                for (int c = 0; c < dk; ++c)
                    for (int c2 = 0; c2 < dk; ++c2)
                        A[c * dk + c2] = (c == c2 ? 1.0 : 0.0) - b * (double)kk[c] * (double)kk[c2];
                /* P <- A P + b k^T v */
                for (int c = 0; c < dk; ++c)
                    for (int r = 0; r < dv; ++r) {
                        double acc = b * (double)kk[c] * (double)vv[r];
                        for (int c2 = 0; c2 < dk; ++c2) acc += A[c * dk + c2] * P[c2 * dv + r];
                        Pn[c * dv + r] = acc;
                    }
                double *sw = P; P = Pn; Pn = sw;
            }
            /* o_t = q_t P_t */
            for (int r = 0; r < dv; ++r) {
                double acc = 0.0;
                for (int c = 0; c < dk; ++c) acc += (double)q[tok * dk + c] * P[c * dv + r];
                o[tok * dv + r] = acc;
            }
        }
        for (int c = 0; c < dk; ++c)
            for (int r = 0; r < dv; ++r) Sf[(long)r * dk + c] = P[c * dv + r];
        free(P); free(Pn); free(A);
    }
    return failed ? -2 : 0;
}

/*
 * Gated DeltaNet-2, token by token: "Gated DeltaNet-2, and the gate that was doing two jobs"
 * (aigenapps.com), section 2 "What decoupling actually means here".  The scalar beta of the delta rule is split into a key-side erase gate
 * b_t in [0,1]^{d_k} and a value-side write gate w_t in [0,1]^{d_v}; with e_t = b_t (.) k_t and
 * z_t = w_t (.) v_t the page's update (row notation, state P in R^{d_k x d_v}) is
 *     P_t = (I - k_t e_t^T) D_t P_{t-1} + k_t z_t^T,       D_t = Diag(a_t) (KDA's decay),
 * i.e. in this file's column convention S = P^T:
 *     S_t = S_{t-1} D_t (I - e_t k_t^T) + z_t k_t^T.
 * Steps per token, as that formula orders them:
 *   1. decay        S <- S D_t              (column c scaled by a_t[c] = exp(g_t[c]))
 *   2. erase read   p = S e_t               (the decayed state read along e_t)
 *   3. correction   u = z_t - p
 *   4. write        S <- S + u k_t^T        (written along k_t)
 *   5. read         o_t = S q_t
 * Layouts: q, k, g, b [BH][T][d_k]; v, w [BH][T][d_v]; S0, S_final [BH][d_v][d_k] (double,
 * S0 may be NULL); o [BH][T][d_v] (double).  Returns 0, -1 on bad arguments, -2 on
 * allocation failure.
 */
int oracle_gdn2_forward(long BH, long T, int dk, int dv,
                        const float *q, const float *k, const float *v,
                        const float *g, const float *b, const float *w,
                        const double *S0, double *o, double *S_final, int nthreads)
{
    if (BH < 0 || T < 0 || dk <= 0 || dv <= 0 || !S_final) return -1;
    if (T > 0 && (!q || !k || !v || !g || !b || !w || !o)) return -1;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
#endif
    for (long bh = 0; bh < BH; ++bh) {
        double *S = S_final + bh * (long)dv * dk;
        double *u = (double *)malloc(sizeof(double) * (size_t)dv);
        double *e = (double *)malloc(sizeof(double) * (size_t)dk);
        if (!u || !e) { free(u); free(e); failed |= 1; continue; }
        if (S0) memcpy(S, S0 + bh * (long)dv * dk, sizeof(double) * (size_t)dv * dk);
        else memset(S, 0, sizeof(double) * (size_t)dv * dk);
        for (long t = 0; t < T; ++t) {
            const long tok = bh * T + t;
            const float *qt = q + tok * dk, *kt = k + tok * dk, *gt = g + tok * dk, *bt = b + tok * dk;
            const float *vt = v + tok * dv, *wt = w + tok * dv;
            for (int c = 0; c < dk; ++c) {               /* 1. decay */
                const double a = exp((double)gt[c]);
                for (int r = 0; r < dv; ++r) S[r * dk + c] *= a;
            }
            for (int c = 0; c < dk; ++c) e[c] = (double)bt[c] * (double)kt[c];
            for (int r = 0; r < dv; ++r) {                /* 2-3. erase read, correction */
                double p = 0.0;
                for (int c = 0; c < dk; ++c) p += S[r * dk + c] * e[c];
                u[r] = (double)wt[r] * (double)vt[r] - p;
            }
            for (int r = 0; r < dv; ++r)                  /* 4. write along k */
                for (int c = 0; c < dk; ++c) S[r * dk + c] += u[r] * (double)kt[c];
            for (int r = 0; r < dv; ++r) {                /* 5. read */
                double acc = 0.0;
                for (int c = 0; c < dk; ++c) acc += S[r * dk + c] * (double)qt[c];
                o[tok * dv + r] = acc;
            }
        }
        free(u); free(e);
    }
    return failed ? -2 : 0;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
