/* Driver for the sanitizer test of the C oracle: runs the whole-sequence
 * forward and the decode step, real and complex, on small seeded inputs
 * (ragged lengths, with and without S0), and checks two closed forms: beta = 0
 * leaves S_T = gamma_T S0, and T decode steps equal one forward. */
#include <complex.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

int gdn_ref_fwd_f64(const double *q, const double *k, const double *v, const double *alpha, const double *beta,
                    const double *S0, double *o, double *S, int B, int T, int H, int dk, int dv, int threads);
int gdn_ref_fwd_c128(const double *q, const double *k, const double *v, const double *alpha, const double *beta,
                     const double *S0, double *o, double *S, int B, int T, int H, int dk, int dv, int threads);
int gdn_ref_step_f64(const double *q, const double *k, const double *v, const double *alpha, const double *beta,
                     double *S, double *o, int N, int dk, int dv, int threads);

static unsigned long long rng = 88172645463325252ull;
static double urand(void) {
  rng ^= rng << 13;
  rng ^= rng >> 7;
  rng ^= rng << 17;
  return (double)(rng >> 11) / 9007199254740992.0;
}

int main(void) {
  int fails = 0;
  const int B = 2, H = 3, dk = 5, dv = 4;
  for (int T = 0; T <= 9; T += 3) {
    const int n = B * T * H;
    double *q = malloc(sizeof(double) * (n * dk + 1)), *k = malloc(sizeof(double) * (n * dk + 1));
    double *v = malloc(sizeof(double) * (n * dv + 1)), *o = malloc(sizeof(double) * (n * dv + 1));
    double *a = malloc(sizeof(double) * (n + 1)), *b = malloc(sizeof(double) * (n + 1));
    double *S0 = malloc(sizeof(double) * B * H * dk * dv), *S = malloc(sizeof(double) * B * H * dk * dv);
    for (int i = 0; i < n * dk; ++i) q[i] = urand() - 0.5, k[i] = urand() - 0.5;
    for (int i = 0; i < n * dv; ++i) v[i] = urand() - 0.5;
    for (int i = 0; i < n; ++i) a[i] = 0.5 + 0.5 * urand(), b[i] = 0.0;
    for (int i = 0; i < B * H * dk * dv; ++i) S0[i] = urand() - 0.5;
    gdn_ref_fwd_f64(q, k, v, a, b, S0, o, S, B, T, H, dk, dv, 2);
    for (int bb = 0; bb < B; ++bb)
      for (int h = 0; h < H; ++h) {
        double g = 1.0;
        for (int t = 0; t < T; ++t) g *= a[(bb * T + t) * H + h];
        for (int e = 0; e < dk * dv; ++e) {
          const int idx = (bb * H + h) * dk * dv + e;
          if (fabs(S[idx] - g * S0[idx]) > 1e-12) ++fails;
        }
      }
    for (int i = 0; i < n; ++i) b[i] = 2.0 * urand();
    gdn_ref_fwd_f64(q, k, v, a, b, NULL, o, S, B, T, H, dk, dv, 1);
    /* decode steps from zero, one token at a time, must match */
    double *Sd = calloc((size_t)B * H * dk * dv, sizeof(double)), *od = malloc(sizeof(double) * B * H * dv);
    double *qt = malloc(sizeof(double) * B * H * dk), *kt = malloc(sizeof(double) * B * H * dk);
    double *vt = malloc(sizeof(double) * B * H * dv), *at = malloc(sizeof(double) * B * H),
           *bt = malloc(sizeof(double) * B * H);
    for (int t = 0; t < T; ++t) {
      for (int bb = 0; bb < B; ++bb)
        for (int h = 0; h < H; ++h) {
          const int s = bb * H + h, tok = (bb * T + t) * H + h;
          for (int e = 0; e < dk; ++e) qt[s * dk + e] = q[tok * dk + e], kt[s * dk + e] = k[tok * dk + e];
          for (int e = 0; e < dv; ++e) vt[s * dv + e] = v[tok * dv + e];
          at[s] = a[tok];
          bt[s] = b[tok];
        }
      gdn_ref_step_f64(qt, kt, vt, at, bt, Sd, od, B * H, dk, dv, 1);
      for (int bb = 0; bb < B; ++bb)
        for (int h = 0; h < H; ++h)
          for (int e = 0; e < dv; ++e)
            if (fabs(od[(bb * H + h) * dv + e] - o[((bb * T + t) * H + h) * dv + e]) > 1e-12) ++fails;
    }
    for (int i = 0; i < B * H * dk * dv; ++i)
      if (fabs(Sd[i] - S[i]) > 1e-12) ++fails;
    /* complex, through the same buffers' sizes */
    double complex *qc = malloc(sizeof(double complex) * (n * dk + 1)), *kc = malloc(sizeof(double complex) * (n * dk + 1));
    double complex *vc = malloc(sizeof(double complex) * (n * dv + 1)), *oc = malloc(sizeof(double complex) * (n * dv + 1));
    double complex *Sc = malloc(sizeof(double complex) * B * H * dk * dv);
    for (int i = 0; i < n * dk; ++i) qc[i] = q[i] + I * k[i], kc[i] = k[i] - I * q[i];
    for (int i = 0; i < n * dv; ++i) vc[i] = v[i] + I * 0.5 * v[i];
    gdn_ref_fwd_c128((const double *)qc, (const double *)kc, (const double *)vc, a, b, NULL, (double *)oc, (double *)Sc, B,
                     T, H, dk, dv, 2);
    for (int i = 0; i < B * H * dk * dv; ++i)
      if (!isfinite(creal(Sc[i])) || !isfinite(cimag(Sc[i]))) ++fails;
    free(qc), free(kc), free(vc), free(oc), free(Sc);
    free(Sd), free(od), free(qt), free(kt), free(vt), free(at), free(bt);
    free(q), free(k), free(v), free(o), free(a), free(b), free(S0), free(S);
  }
  if (fails) {
    fprintf(stderr, "%d oracle checks failed\n", fails);
    return 1;
  }
  printf("oracle driver: all checks passed\n");
  return 0;
}
