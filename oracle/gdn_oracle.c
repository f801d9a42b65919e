/*
 * gdn_oracle.c -- plain fp64 CPU reference for the gated delta rule.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load this library.  It shares
 * no code, header, table or helper with the HIP path.
 *
 * What it computes (one independent chain per (batch, head)):
 *
 *   S_t = alpha_t * (I - beta_t * k_t * kread_t^T) * S_{t-1} + beta_t * k_t * v_t^T
 *   o_t = S_t^T * qread_t
 *
 * with kread = k, qread = q for real data and kread = conj(k), qread = conj(q)
 * for complex data.  S is dk x dv (row index = key dimension).
 *
 * Sources:
 *  - Delta-rule memory: readout with the conjugated key, error against the
 *    value, rank-one write of the error along the key -- DeltaPhase README,
 *    section 2 "Complex Phase Matrix Delta Memory" (readout / error / update).
 *  - Data-dependent forget gate alpha_t scaling the retained state -- Sykra
 *    0.3.3 README, "Architectural Highlights" (data-dependent forget gating),
 *    and the Gated DeltaNet line of work named in DeltaPhase's lineage list.
 *    Reading used here: the gate multiplies the whole Householder-updated
 *    state (decay is applied before the error is formed), which is the Gated
 *    DeltaNet ordering; the output reads the updated state S_t.
 *  - Fixed-size d x d state, O(d^2) per token -- Sykra README,
 *    "Computational Complexity" table.
 *
 * The loops below are the definition written out, token by token, in fp64
 * (complex128 for complex data).  Inputs are the already-rounded values the
 * GPU sees, upcast exactly.  No blocking, fusion or reordering.
 */
#include <complex.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef double _Complex cplx;

/* ------------------------------------------------------------------------ */
/* One token of the recurrence on a real state S (dk x dv, row-major).       */
/* r is caller scratch of length dv.                                         */
static void step_real(double *S, const double *q, const double *k, const double *v,
                      double alpha, double beta, double *o, double *r, int dk, int dv)
{
    /* r = k^T S  (what the memory currently returns for key k) */
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += k[i] * S[(size_t)i * dv + j];
        r[j] = acc;
    }
    /* S <- alpha * (S - beta * k r^T) + beta * k v^T */
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) {
            double s = S[(size_t)i * dv + j];
            S[(size_t)i * dv + j] = alpha * (s - beta * k[i] * r[j]) + beta * k[i] * v[j];
        }
    /* o = S^T q  (read of the updated state) */
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += S[(size_t)i * dv + j] * q[i];
        o[j] = acc;
    }
}

/* One token on a complex state.  The read side uses conj(k) and conj(q); the
 * write side uses k un-conjugated, so that with |k| = 1 and beta = 1 the key
 * reads back exactly the value just written. */
static void step_cplx(cplx *S, const cplx *q, const cplx *k, const cplx *v,
                      double alpha, double beta, cplx *o, cplx *r, int dk, int dv)
{
    for (int j = 0; j < dv; ++j) {
        cplx acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += conj(k[i]) * S[(size_t)i * dv + j];
        r[j] = acc;
    }
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) {
            cplx s = S[(size_t)i * dv + j];
            S[(size_t)i * dv + j] = alpha * (s - beta * k[i] * r[j]) + beta * k[i] * v[j];
        }
    for (int j = 0; j < dv; ++j) {
        cplx acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += S[(size_t)i * dv + j] * conj(q[i]);
        o[j] = acc;
    }
}

static int pick_threads(int nthreads)
{
#ifdef _OPENMP
    return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Whole-sequence forward.                                                   */
/*   q, k : [B, T, H, dk]   v : [B, T, H, dv]   alpha, beta : [B, T, H]       */
/*   S0   : [B, H, dk, dv] or NULL (zero initial state)                      */
/*   o    : [B, T, H, dv]   S : [B, H, dk, dv] final state                    */
/* Returns the number of threads used.                                       */
int gdn_ref_fwd_f64(const double *q, const double *k, const double *v,
                    const double *alpha, const double *beta, const double *S0,
                    double *o, double *S, int B, int T, int H, int dk, int dv,
                    int nthreads)
{
    int nt = pick_threads(nthreads);
    long nchain = (long)B * H;
#pragma omp parallel for num_threads(nt) schedule(dynamic, 1)
    for (long c = 0; c < nchain; ++c) {
        int b = (int)(c / H), h = (int)(c % H);
        double *St = S + (size_t)c * dk * dv;
        double *r = (double *)malloc(sizeof(double) * (size_t)dv);
        if (S0) memcpy(St, S0 + (size_t)c * dk * dv, sizeof(double) * (size_t)dk * dv);
        else memset(St, 0, sizeof(double) * (size_t)dk * dv);
        for (int t = 0; t < T; ++t) {
            size_t tok = ((size_t)b * T + t) * H + h;
            step_real(St, q + tok * dk, k + tok * dk, v + tok * dv, alpha[tok], beta[tok],
                      o + tok * dv, r, dk, dv);
        }
        free(r);
    }
    return nt;
}

/* Same contract, complex data (interleaved re/im doubles). */
int gdn_ref_fwd_c128(const double *q, const double *k, const double *v,
                     const double *alpha, const double *beta, const double *S0,
                     double *o, double *S, int B, int T, int H, int dk, int dv,
                     int nthreads)
{
    int nt = pick_threads(nthreads);
    long nchain = (long)B * H;
    const cplx *cq = (const cplx *)q, *ck = (const cplx *)k, *cv = (const cplx *)v;
    const cplx *cS0 = (const cplx *)S0;
    cplx *co = (cplx *)o, *cS = (cplx *)S;
#pragma omp parallel for num_threads(nt) schedule(dynamic, 1)
    for (long c = 0; c < nchain; ++c) {
        int b = (int)(c / H), h = (int)(c % H);
        cplx *St = cS + (size_t)c * dk * dv;
        cplx *r = (cplx *)malloc(sizeof(cplx) * (size_t)dv);
        if (cS0) memcpy(St, cS0 + (size_t)c * dk * dv, sizeof(cplx) * (size_t)dk * dv);
        else memset(St, 0, sizeof(cplx) * (size_t)dk * dv);
        for (int t = 0; t < T; ++t) {
            size_t tok = ((size_t)b * T + t) * H + h;
            step_cplx(St, cq + tok * dk, ck + tok * dk, cv + tok * dv, alpha[tok], beta[tok],
                      co + tok * dv, r, dk, dv);
        }
        free(r);
    }
    return nt;
}

/* ------------------------------------------------------------------------ */
/* Single-token decode step on N independent states, in place.               */
/*   q, k : [N, dk]  v : [N, dv]  alpha, beta : [N]  S : [N, dk, dv]  o : [N, dv] */
int gdn_ref_step_f64(const double *q, const double *k, const double *v,
                     const double *alpha, const double *beta, double *S, double *o,
                     int N, int dk, int dv, int nthreads)
{
    int nt = pick_threads(nthreads);
#pragma omp parallel for num_threads(nt) schedule(static)
    for (long n = 0; n < N; ++n) {
        double *r = (double *)malloc(sizeof(double) * (size_t)dv);
        step_real(S + (size_t)n * dk * dv, q + (size_t)n * dk, k + (size_t)n * dk,
                  v + (size_t)n * dv, alpha[n], beta[n], o + (size_t)n * dv, r, dk, dv);
        free(r);
    }
    return nt;
}

int gdn_ref_step_c128(const double *q, const double *k, const double *v,
                      const double *alpha, const double *beta, double *S, double *o,
                      int N, int dk, int dv, int nthreads)
{
    int nt = pick_threads(nthreads);
    const cplx *cq = (const cplx *)q, *ck = (const cplx *)k, *cv = (const cplx *)v;
    cplx *cS = (cplx *)S, *co = (cplx *)o;
#pragma omp parallel for num_threads(nt) schedule(static)
    for (long n = 0; n < N; ++n) {
        cplx *r = (cplx *)malloc(sizeof(cplx) * (size_t)dv);
        step_cplx(cS + (size_t)n * dk * dv, cq + (size_t)n * dk, ck + (size_t)n * dk,
                  cv + (size_t)n * dv, alpha[n], beta[n], co + (size_t)n * dv, r, dk, dv);
        free(r);
    }
    return nt;
}
