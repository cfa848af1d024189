/*
 * Oracle for the gated delta rule: a plain, slow, fp64 CPU implementation.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product (GPU) path may include,
 * link or call this file; only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark use it.  It shares no code, header, table or
 * helper with the HIP library.
 *
 * What it computes (per independent (batch, head) sequence, token by token):
 *
 *   Gated Delta Rule-2 update, as stated on "Gated DeltaNet-2 — decoupling
 *   erase and write in linear attention" (jkf87, Q3) and on "Gated DeltaNet-2
 *   Review" (dimensionstp, §3-1):
 *       S_t = (I - k_t (b_t ⊙ k_t)^T) D_t S_{t-1} + k_t (w_t ⊙ v_t)^T,
 *       D_t = diag(alpha_t),  alpha_t = exp(log_alpha_t)  (log-decay in fp32,
 *       "Gated DeltaNet-2 Review" §3-2 item 2).
 *   Read-out from the current state, as on the "Gated DeltaNet" explainer
 *   (lanes-ecd, section "mechanism"): o_t = S_t^T q_t.
 *
 *   The update is evaluated in the equivalent order
 *       S <- D_t S;  r = S^T (b_t ⊙ k_t);  S <- S + k_t (w_t ⊙ v_t - r)^T,
 *   which is the same expression with the erase term multiplied out:
 *   (I - k e^T) D S + k x^T = D S + k (x - (D S)^T e)^T with e = b ⊙ k,
 *   x = w ⊙ v.  The erase reads the *decayed* state (the decay D_t sits to
 *   the right of the erase factor in the equation).
 *
 * Layouts (row-major, fp64):
 *   q, k, log_alpha, b : [BH][T][dk]       v, w : [BH][T][dv]
 *   S0, S_final        : [BH][dk][dv]      (S0 may be NULL -> zeros)
 *   o                  : [BH][T][dv]
 * Gate broadcasting (scalar gates) is done by the caller, who expands them to
 * full channel arrays before the call.
 *
 * The reverse mode (oracle_bwd) is hand-derived reverse-mode differentiation
 * of exactly the loop in oracle_fwd, for the loss
 *     L = sum_t <dO_t, o_t> + <dS_final, S_T>.
 * It recomputes the forward in segments from checkpoints taken every SEG
 * tokens so that long sequences fit in memory.  The erase-side gate gradient
 * (db) and the write-side one (dw) come out as separate terms, which is the
 * "gate-aware" accumulation described on the Gated DeltaNet-2 Q&A page (Q4).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* One token step on a single head.  S is dk x dv, updated in place.
 * o receives S_t^T q_t (dv values); r is scratch for the erase read. */
static void token_step(int dk, int dv, double* S, const double* q,
                       const double* k, const double* v, const double* la,
                       const double* b, const double* w, double* o,
                       double* r /* scratch dv */)
{
    /* S <- D_t S */
    for (int i = 0; i < dk; ++i) {
        double a = exp(la[i]);
        for (int j = 0; j < dv; ++j) S[i * dv + j] *= a;
    }
    /* r = S^T (b ⊙ k) : what the decayed memory predicts along the erase key */
    for (int j = 0; j < dv; ++j) r[j] = 0.0;
    for (int i = 0; i < dk; ++i) {
        double e = b[i] * k[i];
        for (int j = 0; j < dv; ++j) r[j] += S[i * dv + j] * e;
    }
    /* S <- S + k (w ⊙ v - r)^T */
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
            S[i * dv + j] += k[i] * (w[j] * v[j] - r[j]);
    /* o = S^T q */
    if (o) {
        for (int j = 0; j < dv; ++j) o[j] = 0.0;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) o[j] += S[i * dv + j] * q[i];
    }
}

/* Threads for one call: nthreads if positive, else the OpenMP default.  The
 * count goes into each loop's num_threads clause, so a call on one thread
 * leaves later calls' default unchanged. */
static int call_threads(int nthreads)
{
#ifdef _OPENMP
    return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Forward over BH independent sequences of T tokens. */
void oracle_fwd(int BH, int T, int dk, int dv,
                const double* q, const double* k, const double* v,
                const double* la, const double* b, const double* w,
                const double* S0, double* o, double* S_final, int nthreads)
{
    const int nt = call_threads(nthreads);
    (void)nt;
#pragma omp parallel for num_threads(nt) schedule(dynamic, 1)
    for (int h = 0; h < BH; ++h) {
        double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
        double* r = (double*)malloc(sizeof(double) * (size_t)dv);
        if (S0) memcpy(S, S0 + (size_t)h * dk * dv, sizeof(double) * (size_t)dk * dv);
        else memset(S, 0, sizeof(double) * (size_t)dk * dv);
        for (int t = 0; t < T; ++t) {
            size_t xk = ((size_t)h * T + t) * dk, xv = ((size_t)h * T + t) * dv;
            token_step(dk, dv, S, q + xk, k + xk, v + xv, la + xk, b + xk, w + xv,
                       o ? o + xv : NULL, r);
        }
        if (S_final) memcpy(S_final + (size_t)h * dk * dv, S, sizeof(double) * (size_t)dk * dv);
        free(S);
        free(r);
    }
}

/* One decode step for NH independent (sequence, head) states, in place.
 * Inputs are one token each: q, k, la, b : [NH][dk]; v, w : [NH][dv]. */
void oracle_decode(int NH, int dk, int dv,
                   const double* q, const double* k, const double* v,
                   const double* la, const double* b, const double* w,
                   double* S, double* o, int nthreads)
{
    const int nt = call_threads(nthreads);
    (void)nt;
#pragma omp parallel for num_threads(nt) schedule(static)
    for (int h = 0; h < NH; ++h) {
        double* r = (double*)malloc(sizeof(double) * (size_t)dv);
        token_step(dk, dv, S + (size_t)h * dk * dv, q + (size_t)h * dk, k + (size_t)h * dk,
                   v + (size_t)h * dv, la + (size_t)h * dk, b + (size_t)h * dk,
                   w + (size_t)h * dv, o + (size_t)h * dv, r);
        free(r);
    }
}

#define SEG 64

/* Reverse mode of oracle_fwd.  Outputs dq, dk_, dla, db : [BH][T][dk];
 * dv_, dw : [BH][T][dv]; dS0 : [BH][dk][dv].  dO : [BH][T][dv];
 * dS_final may be NULL (zero). */
void oracle_bwd(int BH, int T, int dk, int dv,
                const double* q, const double* k, const double* v,
                const double* la, const double* b, const double* w,
                const double* S0, const double* dO, const double* dS_final,
                double* dq, double* dk_, double* dv_, double* dla,
                double* db, double* dw, double* dS0, int nthreads)
{
    const int nt = call_threads(nthreads);
    (void)nt;
    const size_t SS = (size_t)dk * dv;
    const int nseg = (T + SEG - 1) / SEG;
#pragma omp parallel for num_threads(nt) schedule(dynamic, 1)
    for (int h = 0; h < BH; ++h) {
        /* checkpoints: state before each segment */
        double* ck = (double*)malloc(sizeof(double) * SS * (size_t)nseg);
        /* states S_{t-1} for every token of one segment */
        double* seg = (double*)malloc(sizeof(double) * SS * SEG);
        double* S = (double*)malloc(sizeof(double) * SS);
        double* G = (double*)malloc(sizeof(double) * SS);
        double* Sh = (double*)malloc(sizeof(double) * SS);
        double* r = (double*)malloc(sizeof(double) * (size_t)dv);
        double* dlt = (double*)malloc(sizeof(double) * (size_t)dv);
        double* ddl = (double*)malloc(sizeof(double) * (size_t)dv);
        double* de = (double*)malloc(sizeof(double) * (size_t)dk);

        if (S0) memcpy(S, S0 + (size_t)h * SS, sizeof(double) * SS);
        else memset(S, 0, sizeof(double) * SS);
        for (int s = 0; s < nseg; ++s) {
            memcpy(ck + (size_t)s * SS, S, sizeof(double) * SS);
            int t1 = (s + 1) * SEG < T ? (s + 1) * SEG : T;
            for (int t = s * SEG; t < t1; ++t) {
                size_t xk = ((size_t)h * T + t) * dk, xv = ((size_t)h * T + t) * dv;
                token_step(dk, dv, S, q + xk, k + xk, v + xv, la + xk, b + xk, w + xv, NULL, r);
            }
        }
        /* S now holds S_T.  G = dL/dS_T. */
        if (dS_final) memcpy(G, dS_final + (size_t)h * SS, sizeof(double) * SS);
        else memset(G, 0, sizeof(double) * SS);

        for (int s = nseg - 1; s >= 0; --s) {
            int t0 = s * SEG;
            int t1 = (s + 1) * SEG < T ? (s + 1) * SEG : T;
            /* recompute S_{t-1} for t in [t0, t1) */
            memcpy(S, ck + (size_t)s * SS, sizeof(double) * SS);
            for (int t = t0; t < t1; ++t) {
                size_t xk = ((size_t)h * T + t) * dk, xv = ((size_t)h * T + t) * dv;
                memcpy(seg + (size_t)(t - t0) * SS, S, sizeof(double) * SS);
                token_step(dk, dv, S, q + xk, k + xk, v + xv, la + xk, b + xk, w + xv, NULL, r);
            }
            for (int t = t1 - 1; t >= t0; --t) {
                size_t xk = ((size_t)h * T + t) * dk, xv = ((size_t)h * T + t) * dv;
                const double* Sp = seg + (size_t)(t - t0) * SS; /* S_{t-1} */
                const double *qt = q + xk, *kt = k + xk, *lat = la + xk, *bt = b + xk;
                const double *vt = v + xv, *wt = w + xv, *dOt = dO + xv;
                /* rebuild this step's intermediates */
                for (int i = 0; i < dk; ++i) {
                    double a = exp(lat[i]);
                    for (int j = 0; j < dv; ++j) Sh[i * dv + j] = a * Sp[i * dv + j];
                }
                for (int j = 0; j < dv; ++j) r[j] = 0.0;
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j) r[j] += Sh[i * dv + j] * bt[i] * kt[i];
                for (int j = 0; j < dv; ++j) dlt[j] = wt[j] * vt[j] - r[j]; /* delta */
                /* S_t = Sh + k delta^T ; o_t = S_t^T q */
                /* dq_t = S_t dO_t ; G += q dO^T */
                for (int i = 0; i < dk; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < dv; ++j)
                        acc += (Sh[i * dv + j] + kt[i] * dlt[j]) * dOt[j];
                    dq[xk + i] = acc;
                }
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j) G[i * dv + j] += qt[i] * dOt[j];
                /* through S_t = Sh + k delta^T */
                for (int j = 0; j < dv; ++j) ddl[j] = 0.0;
                for (int i = 0; i < dk; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < dv; ++j) {
                        acc += G[i * dv + j] * dlt[j];
                        ddl[j] += G[i * dv + j] * kt[i];
                    }
                    dk_[xk + i] = acc;
                }
                /* delta = w ⊙ v - r */
                for (int j = 0; j < dv; ++j) {
                    dw[xv + j] = ddl[j] * vt[j];
                    dv_[xv + j] = ddl[j] * wt[j];
                }
                /* r = Sh^T e, e = b ⊙ k:  dr = -ddl ; de = Sh dr ; dSh += e dr^T */
                for (int i = 0; i < dk; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < dv; ++j) acc -= Sh[i * dv + j] * ddl[j];
                    de[i] = acc;
                }
                for (int i = 0; i < dk; ++i) {
                    db[xk + i] = de[i] * kt[i];
                    dk_[xk + i] += de[i] * bt[i];
                }
                /* dSh = G - e ddl^T ; Sh = D S_{t-1} */
                for (int i = 0; i < dk; ++i) {
                    double a = exp(lat[i]);
                    double e = bt[i] * kt[i];
                    double acc = 0.0;
                    for (int j = 0; j < dv; ++j) {
                        double g = G[i * dv + j] - e * ddl[j];
                        acc += g * Sp[i * dv + j];
                        G[i * dv + j] = a * g;
                    }
                    dla[xk + i] = acc * a;
                }
            }
        }
        memcpy(dS0 + (size_t)h * SS, G, sizeof(double) * SS);
        free(ck); free(seg); free(S); free(G); free(Sh);
        free(r); free(dlt); free(ddl); free(de);
    }
}
