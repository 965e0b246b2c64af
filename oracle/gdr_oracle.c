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

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
