/*
 * kda_oracle_bwd.c -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain fp64 CPU reference for the gradient of the Kimi Delta Attention (KDA)
 * forward recurrence (the training direction the FlashKDA kernel of the Kimi
 * K3 paper digest, devpress.csdn.net, section 2.4 (1), also serves).  Only the
 * test suite, the smoke check and the benchmark's CPU leg may load it; the
 * HIP library never does and the two share no code.
 *
 * The forward recurrence (kda_oracle.c), per (b, h):
 *   S'_t = Diag(exp g_t) S_{t-1}      decay
 *   r_t  = S'_t^T k_t                 recall with the incoming key
 *   e_t  = beta_t (v_t - r_t)         the difference that is written
 *   S_t  = S'_t + k_t e_t^T           erase + write
 *   o_t  = scale S_t^T q_t            read after the write
 * with S_0 = h0 and hT = S_T.
 *
 * Given dO = dL/do and dhT = dL/dhT, this computes every input gradient by the
 * plain reverse-mode adjoint of those lines, token by token from the last to
 * the first.  dS is dL/dS_t when token t is processed (dhT before the last):
 *   dS   += scale q_t do_t^T            (o_t reads S_t)
 *   dq_t  = scale S_t do_t
 *   de    = dS^T k_t                    (S_t = S'_t + k_t e_t^T)
 *   dk_t  = dS e_t
 *   dbeta_t = de . (v_t - r_t)          (e_t = beta_t (v_t - r_t))
 *   dv_t  = beta_t de
 *   dr    = -beta_t de
 *   dS'   = dS + k_t dr^T               (r_t = S'_t^T k_t)
 *   dk_t += S'_t dr
 *   dg_t  = rowsum(dS' .* S'_t)         (S'_t = Diag(exp g_t) S_{t-1}:
 *                                        d/dg_t[i] of S'_t[i][:] is S'_t[i][:])
 *   dS    = Diag(exp g_t) dS'           (the gradient of S_{t-1})
 * and finally dh0 = dS.
 *
 * The states S_{t-1} needed on the way back are recomputed from fp64
 * checkpoints every BLK tokens, one block at a time (the same token recurrence;
 * this only bounds memory).
 *
 * Layouts as in kda_oracle.c; dO like o, dhT and dh0 like the states.  h0 and
 * dhT may be NULL (zeros); dh0 may be NULL (not written).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

#define BLK 64

int kda_oracle_bwd(const double *q, const double *k, const double *v,
                   const double *g, const double *beta, const double *h0,
                   const double *dO, const double *dhT,
                   double *dq, double *dk, double *dv, double *dg,
                   double *dbeta, double *dh0,
                   long B, long T, long H, long Dk, long Dv, double scale)
{
    if (B < 0 || T < 0 || H < 0 || Dk <= 0 || Dv <= 0) return 1;
    const long nblk = (T + BLK - 1) / BLK;
    const long SS = Dk * Dv;
    int failed = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (long b = 0; b < B; ++b) {
        for (long h = 0; h < H; ++h) {
            /* checkpoints: ck[m] is the state before token m * BLK */
            double *ck = (double *)malloc(sizeof(double) * (size_t)((nblk > 0 ? nblk : 1) * SS));
            double *blk = (double *)malloc(sizeof(double) * (size_t)(BLK * SS)); /* S_{t-1} of a block */
            double *S = (double *)malloc(sizeof(double) * (size_t)SS);
            double *Sp = (double *)malloc(sizeof(double) * (size_t)SS);
            double *dS = (double *)malloc(sizeof(double) * (size_t)SS);
            double *vec = (double *)malloc(sizeof(double) * (size_t)(4 * Dv + Dk));
            if (!ck || !blk || !S || !Sp || !dS || !vec) {
#pragma omp atomic write
                failed = 1;
                free(ck); free(blk); free(S); free(Sp); free(dS); free(vec);
                continue;
            }
            double *r = vec, *e = vec + Dv, *de = vec + 2 * Dv, *dr = vec + 3 * Dv, *a = vec + 4 * Dv;
            const long sh = (b * H + h) * SS;

            /* one forward token step: S <- S_t from S = S_{t-1}; also leaves S'_t in Sp, r_t, e_t */
#define FWD_STEP(t)                                                                     \
    do {                                                                                \
        const long row = (b * T + (t)) * H + h;                                         \
        const double *kt = k + row * Dk, *gt = g + row * Dk, *vt = v + row * Dv;        \
        for (long i = 0; i < Dk; ++i) {                                                 \
            const double ai = exp(gt[i]);                                               \
            for (long j = 0; j < Dv; ++j) Sp[i * Dv + j] = ai * S[i * Dv + j];          \
        }                                                                               \
        for (long j = 0; j < Dv; ++j) r[j] = 0.0;                                       \
        for (long i = 0; i < Dk; ++i)                                                   \
            for (long j = 0; j < Dv; ++j) r[j] += Sp[i * Dv + j] * kt[i];               \
        for (long j = 0; j < Dv; ++j) e[j] = beta[row] * (vt[j] - r[j]);                \
        for (long i = 0; i < Dk; ++i)                                                   \
            for (long j = 0; j < Dv; ++j) S[i * Dv + j] = Sp[i * Dv + j] + kt[i] * e[j]; \
    } while (0)

            if (h0) memcpy(S, h0 + sh, sizeof(double) * (size_t)SS);
            else memset(S, 0, sizeof(double) * (size_t)SS);
            for (long t = 0; t < T; ++t) {
                if (t % BLK == 0) memcpy(ck + (t / BLK) * SS, S, sizeof(double) * (size_t)SS);
                FWD_STEP(t);
            }
            if (dhT) memcpy(dS, dhT + sh, sizeof(double) * (size_t)SS);
            else memset(dS, 0, sizeof(double) * (size_t)SS);

            for (long m = nblk - 1; m >= 0; --m) {
                const long t0 = m * BLK, t1 = (t0 + BLK < T) ? t0 + BLK : T;
                memcpy(S, ck + m * SS, sizeof(double) * (size_t)SS);
                for (long t = t0; t < t1; ++t) {
                    memcpy(blk + (t - t0) * SS, S, sizeof(double) * (size_t)SS);
                    FWD_STEP(t);
                }
                for (long t = t1 - 1; t >= t0; --t) {
                    /* re-form S'_t, r_t, e_t and S_t from S_{t-1} */
                    memcpy(S, blk + (t - t0) * SS, sizeof(double) * (size_t)SS);
                    FWD_STEP(t);
                    const long row = (b * T + t) * H + h;
                    const double *qt = q + row * Dk, *kt = k + row * Dk, *gt = g + row * Dk, *vt = v + row * Dv;
                    const double *dot = dO + row * Dv;
                    const double bt = beta[row];
                    double *dqt = dq + row * Dk, *dkt = dk + row * Dk, *dgt = dg + row * Dk, *dvt = dv + row * Dv;
                    /* o_t = scale S_t^T q_t */
                    for (long i = 0; i < Dk; ++i)
                        for (long j = 0; j < Dv; ++j) dS[i * Dv + j] += scale * qt[i] * dot[j];
                    for (long i = 0; i < Dk; ++i) {
                        double s = 0.0;
                        for (long j = 0; j < Dv; ++j) s += S[i * Dv + j] * dot[j];
                        dqt[i] = scale * s;
                    }
                    /* S_t = S'_t + k_t e_t^T */
                    for (long j = 0; j < Dv; ++j) de[j] = 0.0;
                    for (long i = 0; i < Dk; ++i)
                        for (long j = 0; j < Dv; ++j) de[j] += dS[i * Dv + j] * kt[i];
                    for (long i = 0; i < Dk; ++i) {
                        double s = 0.0;
                        for (long j = 0; j < Dv; ++j) s += dS[i * Dv + j] * e[j];
                        dkt[i] = s;
                    }
                    /* e_t = beta_t (v_t - r_t) */
                    double db = 0.0;
                    for (long j = 0; j < Dv; ++j) {
                        db += de[j] * (vt[j] - r[j]);
                        dvt[j] = bt * de[j];
                        dr[j] = -bt * de[j];
                    }
                    dbeta[row] = db;
                    /* r_t = S'_t^T k_t: dS' = dS + k_t dr^T, dk_t += S'_t dr */
                    for (long i = 0; i < Dk; ++i)
                        for (long j = 0; j < Dv; ++j) dS[i * Dv + j] += kt[i] * dr[j];
                    for (long i = 0; i < Dk; ++i) {
                        double s = 0.0;
                        for (long j = 0; j < Dv; ++j) s += Sp[i * Dv + j] * dr[j];
                        dkt[i] += s;
                    }
                    /* S'_t = Diag(exp g_t) S_{t-1} */
                    for (long i = 0; i < Dk; ++i) {
                        double s = 0.0;
                        for (long j = 0; j < Dv; ++j) s += dS[i * Dv + j] * Sp[i * Dv + j];
                        dgt[i] = s;
                        a[i] = exp(gt[i]);
                        for (long j = 0; j < Dv; ++j) dS[i * Dv + j] *= a[i];
                    }
                }
            }
            if (dh0) memcpy(dh0 + sh, dS, sizeof(double) * (size_t)SS);
#undef FWD_STEP
            free(ck); free(blk); free(S); free(Sp); free(dS); free(vec);
        }
    }
    return failed;
}
