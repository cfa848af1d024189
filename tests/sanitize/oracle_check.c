/* The oracle's C entry points on small ragged inputs, built with
 * AddressSanitizer and UndefinedBehaviorSanitizer (gdr_oracle.c is compiled
 * into this program with the same flags): forward, decode and reverse mode,
 * lengths on both sides of the reverse mode's checkpoint segment of 64
 * tokens, head sizes that are not powers of two, with and without an initial
 * state.  Checks that every output is finite and that a forward split in two
 * calls (the first call's final state as the second's initial state) agrees
 * with one call over the whole sequence. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

void oracle_fwd(int BH, int T, int dk, int dv, const double* q, const double* k, const double* v,
                const double* la, const double* b, const double* w, const double* S0, double* o,
                double* S_final, int nthreads);
void oracle_decode(int NH, int dk, int dv, const double* q, const double* k, const double* v,
                   const double* la, const double* b, const double* w, double* S, double* o, int nthreads);
void oracle_bwd(int BH, int T, int dk, int dv, const double* q, const double* k, const double* v,
                const double* la, const double* b, const double* w, const double* S0, const double* dO,
                const double* dS_final, double* dq, double* dk_, double* dv_, double* dla, double* db,
                double* dw, double* dS0, int nthreads);

static unsigned long long st = 88172645463325252ull;
static double rnd(void) {
    st ^= st << 13; st ^= st >> 7; st ^= st << 17;
    return (double)(st >> 11) / 9007199254740992.0 - 0.5;
}
static double* arr(size_t n, double scale, double shift) {
    double* a = malloc(sizeof(double) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) a[i] = shift + scale * rnd();
    return a;
}
static int finite_all(const double* a, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(a[i])) return 0;
    return 1;
}

int main(void) {
    int bad = 0;
    const int shapes[][4] = {{1, 1, 1, 1}, {2, 63, 5, 3}, {2, 64, 3, 5}, {3, 65, 4, 4}, {1, 130, 7, 2}, {2, 0, 3, 3}};
    for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; ++s) {
        const int BH = shapes[s][0], T = shapes[s][1], dk = shapes[s][2], dv = shapes[s][3];
        const size_t nk = (size_t)BH * T * dk, nv = (size_t)BH * T * dv, ns = (size_t)BH * dk * dv;
        double *q = arr(nk, 1, 0), *k = arr(nk, 1, 0), *v = arr(nv, 1, 0), *la = arr(nk, 0.1, -0.05);
        double *b = arr(nk, 0.5, 0.5), *w = arr(nv, 0.5, 0.5), *S0 = arr(ns, 0.04, 0), *dO = arr(nv, 1, 0);
        double *dSf = arr(ns, 1, 0), *o = arr(nv, 0, 0), *Sf = arr(ns, 0, 0);
        double *g[7];
        const size_t gn[7] = {nk, nk, nv, nk, nk, nv, ns};
        for (int i = 0; i < 7; ++i) g[i] = arr(gn[i], 0, 0);
        for (int withS0 = 0; withS0 < 2; ++withS0) {
            const double* s0 = withS0 ? S0 : NULL;
            oracle_fwd(BH, T, dk, dv, q, k, v, la, b, w, s0, o, Sf, 1);
            bad += !finite_all(o, nv) + !finite_all(Sf, ns);
            oracle_bwd(BH, T, dk, dv, q, k, v, la, b, w, s0, dO, withS0 ? dSf : NULL, g[0], g[1], g[2], g[3],
                       g[4], g[5], g[6], 1);
            for (int i = 0; i < 7; ++i) bad += !finite_all(g[i], gn[i]);
        }
        /* two halves on one head = one call (per head, the halves' inputs are
           contiguous slices of the full arrays when BH == 1) */
        if (BH == 1 && T > 1) {
            const int T1 = T / 2, T2 = T - T1;
            double *o1 = arr(nv, 0, 0), *S1 = arr(ns, 0, 0), *S2 = arr(ns, 0, 0);
            oracle_fwd(1, T, dk, dv, q, k, v, la, b, w, S0, o, Sf, 1);
            oracle_fwd(1, T1, dk, dv, q, k, v, la, b, w, S0, o1, S1, 1);
            oracle_fwd(1, T2, dk, dv, q + (size_t)T1 * dk, k + (size_t)T1 * dk, v + (size_t)T1 * dv,
                       la + (size_t)T1 * dk, b + (size_t)T1 * dk, w + (size_t)T1 * dv, S1,
                       o1 + (size_t)T1 * dv, S2, 1);
            for (size_t i = 0; i < nv; ++i) bad += fabs(o[i] - o1[i]) > 1e-12;
            for (size_t i = 0; i < ns; ++i) bad += fabs(Sf[i] - S2[i]) > 1e-12;
            free(o1); free(S1); free(S2);
        }
        if (T > 0) {   /* one decode step on each head's first token */
            double *S = arr(ns, 0.04, 0), *od = arr((size_t)BH * dv, 0, 0);
            oracle_decode(BH, dk, dv, q, k, v, la, b, w, S, od, 1);
            bad += !finite_all(S, ns) + !finite_all(od, (size_t)BH * dv);
            free(S); free(od);
        }
        free(q); free(k); free(v); free(la); free(b); free(w); free(S0); free(dO); free(dSf); free(o); free(Sf);
        for (int i = 0; i < 7; ++i) free(g[i]);
    }
    printf("%s: %d problems\n", bad ? "FAILED" : "ok", bad);
    return bad ? 1 : 0;
}
