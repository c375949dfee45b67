/*
 * kda_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, token-by-token fp64 CPU reference for the Kimi Delta Attention
 * (KDA) forward recurrence.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library; the product path
 * (the HIP library and its Python binding) never does, and the two share no
 * code.
 *
 * What it computes (per batch b and head h, independently):
 *
 *   S <- S0                                       (d_k x d_v, fp64)
 *   for t = 0 .. T-1:
 *     S   <- Diag(exp(g_t)) S        decay: every key channel i of the state
 *                                    is multiplied by exp(g_t[i])
 *     r   <- S^T k_t                 recall the value stored under k_t
 *     e   <- beta_t (v_t - r)        only the difference is written
 *     S   <- S + k_t e^T             erase + write, i.e. (I - beta k k^T) S + beta k v^T
 *     o_t <- scale * S^T q_t         read after the write
 *
 * Sources:
 *  - "Kimi K3 Architecture Explained: How the World's Largest Open Source AI
 *    Model Works", section 3 "Kimi Delta Attention (KDA)": the lineage
 *    linear attention -> DeltaNet (recall with the incoming key, write only
 *    the difference) -> Gated DeltaNet (forget gate alpha, write gate beta)
 *    -> KDA (decay first, then erase, then write).
 *  - Kimi K3 paper digest (devpress.csdn.net), section 2.1 (1) "KDA 原理":
 *    delta-rule recursion with a per-channel forget gate on a fixed-size
 *    recurrent state.
 *  - The three update lines (S' = Diag(exp g) S; S = S' + beta k (v - S'^T k)^T;
 *    o = d_k^-1/2 S^T q) are the benchmark spec's own formulation of the above;
 *    the pages give the order in prose only.
 *
 * Readings where the pages are silent: the gate decays the d_k (key) channels;
 * the erase uses the decayed state; the output reads the state after the
 * write; the caller supplies the scale (d_k^-1/2 by default in the wrapper).
 *
 * Layouts (all contiguous, row-major):
 *   q, k, g : [B, T, H, Dk]     v, o : [B, T, H, Dv]     beta : [B, T, H]
 *   S       : [B, H, Dk, Dv]    (in: initial state, out: final state)
 * Inputs are fp64 copies of the stored values (bf16 and fp32 convert exactly).
 * Parallel over (b, h) with OpenMP when built with -fopenmp.
 */
#include <math.h>
#include <stdlib.h>

int kda_oracle_fwd(const double *q, const double *k, const double *v,
                   const double *g, const double *beta, double *S, double *o,
                   long B, long T, long H, long Dk, long Dv, double scale)
{
    if (B < 0 || T < 0 || H < 0 || Dk <= 0 || Dv <= 0) return 1;
    int failed = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (long b = 0; b < B; ++b) {
        for (long h = 0; h < H; ++h) {
            double *St = S + (b * H + h) * Dk * Dv;
            double *r = (double *)malloc(sizeof(double) * (size_t)Dv);
            if (!r) {
#pragma omp atomic write
                failed = 1;
                continue;
            }
            for (long t = 0; t < T; ++t) {
                const long row = (b * T + t) * H + h;
                const double *qt = q + row * Dk;
                const double *kt = k + row * Dk;
                const double *gt = g + row * Dk;
                const double *vt = v + row * Dv;
                double *ot = o + row * Dv;
                const double bt = beta[row];

                /* 1. decay each key channel */
                for (long i = 0; i < Dk; ++i) {
                    const double a = exp(gt[i]);
                    double *Si = St + i * Dv;
                    for (long j = 0; j < Dv; ++j) Si[j] *= a;
                }
                /* 2. recall with the incoming key: r = S^T k */
                for (long j = 0; j < Dv; ++j) r[j] = 0.0;
                for (long i = 0; i < Dk; ++i) {
                    const double ki = kt[i];
                    const double *Si = St + i * Dv;
                    for (long j = 0; j < Dv; ++j) r[j] += Si[j] * ki;
                }
                /* 3. write only the difference, weighted by beta */
                for (long j = 0; j < Dv; ++j) r[j] = bt * (vt[j] - r[j]);
                for (long i = 0; i < Dk; ++i) {
                    const double ki = kt[i];
                    double *Si = St + i * Dv;
                    for (long j = 0; j < Dv; ++j) Si[j] += ki * r[j];
                }
                /* 4. read the updated state with the query */
                for (long j = 0; j < Dv; ++j) ot[j] = 0.0;
                for (long i = 0; i < Dk; ++i) {
                    const double qi = qt[i];
                    const double *Si = St + i * Dv;
                    for (long j = 0; j < Dv; ++j) ot[j] += Si[j] * qi;
                }
                for (long j = 0; j < Dv; ++j) ot[j] *= scale;
            }
            free(r);
        }
    }
    return failed;
}

int kda_oracle_decode(const double *q, const double *k, const double *v,
                      const double *g, const double *beta, double *S, double *o,
                      long B, long H, long Dk, long Dv, double scale)
{
    /* One token per sequence: the same recurrence with T = 1, where the
     * [B, 1, H, D] and [B, H, D] layouts coincide. */
    return kda_oracle_fwd(q, k, v, g, beta, S, o, B, 1, H, Dk, Dv, scale);
}

int kda_oracle_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
