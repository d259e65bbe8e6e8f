/*
 * Kimi Delta Attention (KDA): plain fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do.  It shares no code, header, table or constant with the HIP
 * library.
 *
 * What it computes, per independent (batch b, head h) pair, in fp64:
 *
 *   gate     g_t = gmin * sigmoid(exp(A) * z_t),  gmin = -5,  alpha_t = exp(g_t)
 *            ("Kimi K3 internal structure analysis", section "Sequence mixing:
 *            3 KDA layers per global MLA layer": the K3 retention
 *            parameterisation with its lower bound of -5)
 *   retain   S' = Diag(alpha_t) S_{t-1}
 *            (same section: the channel-wise retention factor decides how
 *            much of the previous state survives BEFORE the current key/value
 *            pair is written; "channel" is read as the key channel, the row
 *            index of S in R^{dk x dv})
 *   write    u_t = beta_t (v_t - S'^T k_t);   S_t = S' + k_t u_t^T
 *            (same section: the fixed-size state is updated by the delta rule;
 *            this equals S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1}
 *            + beta_t k_t v_t^T)
 *   read     o_t = S_t^T q_t   (the post-update state)
 *
 * Layouts (row-major, contiguous): q,k,g,z [B,T,H,dk]; v,o [B,T,H,dv];
 * beta [B,T,H]; A [H,dk]; S0,ST [B,H,dk,dv].  S0 may be NULL (zero state).
 *
 * Parallelism: the columns n of S evolve independently of one another (each
 * step touches column n only through v_t[n] and u_t[n]), so the work is split
 * over (b, h, column block) with OpenMP.  Inside one work item the loops are
 * the token recurrence exactly as written above.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define KDA_ORACLE_GMIN (-5.0)

static double oracle_sigmoid(double x)
{
    /* evaluated so that no exp() overflows */
    if (x >= 0.0)
        return 1.0 / (1.0 + exp(-x));
    double e = exp(x);
    return e / (1.0 + e);
}

/* g = gmin * sigmoid(exp(A[h,c]) * z[b,t,h,c]) for every element. */
void kda_oracle_gate(const double *z, const double *A, double *g,
                     int64_t B, int64_t T, int64_t H, int64_t dk)
{
    int64_t rows = B * T;
#pragma omp parallel for schedule(static)
    for (int64_t bt = 0; bt < rows; ++bt) {
        for (int64_t h = 0; h < H; ++h) {
            for (int64_t c = 0; c < dk; ++c) {
                int64_t i = (bt * H + h) * dk + c;
                g[i] = KDA_ORACLE_GMIN * oracle_sigmoid(exp(A[h * dk + c]) * z[i]);
            }
        }
    }
}

/* The token recurrence for one (b, h) pair restricted to columns [n0, n1). */
static void oracle_chain(const double *q, const double *k, const double *v,
                         const double *g, const double *beta, const double *S0,
                         double *o, double *ST, int64_t b, int64_t h,
                         int64_t T, int64_t H, int64_t dk, int64_t dv,
                         int64_t n0, int64_t n1, double *S, double *p, double *u)
{
    int64_t w = n1 - n0;
    /* S is dk x w (row-major) */
    for (int64_t c = 0; c < dk; ++c)
        for (int64_t n = 0; n < w; ++n)
            S[c * w + n] = S0 ? S0[((b * H + h) * dk + c) * dv + n0 + n] : 0.0;

    for (int64_t t = 0; t < T; ++t) {
        int64_t row_k = ((b * T + t) * H + h) * dk;
        int64_t row_v = ((b * T + t) * H + h) * dv;
        double bt = beta[(b * T + t) * H + h];

        /* retain: S' = Diag(exp(g_t)) S */
        for (int64_t c = 0; c < dk; ++c) {
            double a = exp(g[row_k + c]);
            for (int64_t n = 0; n < w; ++n)
                S[c * w + n] *= a;
        }
        /* prediction S'^T k_t */
        for (int64_t n = 0; n < w; ++n)
            p[n] = 0.0;
        for (int64_t c = 0; c < dk; ++c) {
            double kc = k[row_k + c];
            for (int64_t n = 0; n < w; ++n)
                p[n] += S[c * w + n] * kc;
        }
        /* delta-rule correction and write */
        for (int64_t n = 0; n < w; ++n)
            u[n] = bt * (v[row_v + n0 + n] - p[n]);
        for (int64_t c = 0; c < dk; ++c) {
            double kc = k[row_k + c];
            for (int64_t n = 0; n < w; ++n)
                S[c * w + n] += kc * u[n];
        }
        /* read with the post-update state */
        if (o) {
            for (int64_t n = 0; n < w; ++n)
                p[n] = 0.0;
            for (int64_t c = 0; c < dk; ++c) {
                double qc = q[row_k + c];
                for (int64_t n = 0; n < w; ++n)
                    p[n] += S[c * w + n] * qc;
            }
            for (int64_t n = 0; n < w; ++n)
                o[row_v + n0 + n] = p[n];
        }
    }
    if (ST)
        for (int64_t c = 0; c < dk; ++c)
            for (int64_t n = 0; n < w; ++n)
                ST[((b * H + h) * dk + c) * dv + n0 + n] = S[c * w + n];
}

/*
 * Full forward over T tokens.  o (nullable) receives every output, ST
 * (nullable) the final state.  col_block > 0 sets the column-block width used
 * for parallelism (it does not change any result: columns are independent);
 * nthreads <= 0 keeps the OpenMP default.
 */
void kda_oracle_forward(const double *q, const double *k, const double *v,
                        const double *g, const double *beta, const double *S0,
                        double *o, double *ST,
                        int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                        int64_t col_block, int nthreads)
{
    if (col_block <= 0 || col_block > dv)
        col_block = dv;
    int64_t nblk = (dv + col_block - 1) / col_block;
    int64_t items = B * H * nblk;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        double *S = (double *)malloc(sizeof(double) * (size_t)(dk * col_block));
        double *p = (double *)malloc(sizeof(double) * (size_t)col_block);
        double *u = (double *)malloc(sizeof(double) * (size_t)col_block);
#pragma omp for schedule(dynamic, 1)
        for (int64_t it = 0; it < items; ++it) {
            int64_t bh = it / nblk, blk = it % nblk;
            int64_t b = bh / H, h = bh % H;
            int64_t n0 = blk * col_block;
            int64_t n1 = n0 + col_block < dv ? n0 + col_block : dv;
            oracle_chain(q, k, v, g, beta, S0, o, ST, b, h, T, H, dk, dv, n0, n1, S, p, u);
        }
        free(S);
        free(p);
        free(u);
    }
}

/*
 * One decode step for N independent sequences x H heads: the gate is
 * evaluated from (z, A) and one token is applied to `state` in place.
 * q,k,z [N,H,dk]; v,o [N,H,dv]; beta [N,H]; A [H,dk]; state [N,H,dk,dv].
 */
void kda_oracle_decode_step(const double *q, const double *k, const double *v,
                            const double *z, const double *A, const double *beta,
                            double *state, double *o,
                            int64_t N, int64_t H, int64_t dk, int64_t dv)
{
#pragma omp parallel
    {
        double *g = (double *)malloc(sizeof(double) * (size_t)dk);
        double *p = (double *)malloc(sizeof(double) * (size_t)dv);
        double *u = (double *)malloc(sizeof(double) * (size_t)dv);
#pragma omp for schedule(static)
        for (int64_t nh = 0; nh < N * H; ++nh) {
            int64_t h = nh % H;
            const double *qq = q + nh * dk, *kk = k + nh * dk, *zz = z + nh * dk;
            const double *vv = v + nh * dv;
            double *S = state + nh * dk * dv;
            double bt = beta[nh];
            for (int64_t c = 0; c < dk; ++c)
                g[c] = KDA_ORACLE_GMIN * oracle_sigmoid(exp(A[h * dk + c]) * zz[c]);
            for (int64_t c = 0; c < dk; ++c) {
                double a = exp(g[c]);
                for (int64_t n = 0; n < dv; ++n)
                    S[c * dv + n] *= a;
            }
            for (int64_t n = 0; n < dv; ++n)
                p[n] = 0.0;
            for (int64_t c = 0; c < dk; ++c)
                for (int64_t n = 0; n < dv; ++n)
                    p[n] += S[c * dv + n] * kk[c];
            for (int64_t n = 0; n < dv; ++n)
                u[n] = bt * (vv[n] - p[n]);
            for (int64_t c = 0; c < dk; ++c)
                for (int64_t n = 0; n < dv; ++n)
                    S[c * dv + n] += kk[c] * u[n];
            for (int64_t n = 0; n < dv; ++n)
                p[n] = 0.0;
            for (int64_t c = 0; c < dk; ++c)
                for (int64_t n = 0; n < dv; ++n)
                    p[n] += S[c * dv + n] * qq[c];
            for (int64_t n = 0; n < dv; ++n)
                o[nh * dv + n] = p[n];
        }
        free(g);
        free(p);
        free(u);
    }
}

int kda_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
