/*
 * ssd_ref_complex.c -- the fp64 sequential oracle of the complex-A SSD scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this file; only the tests, the package's smoke check and the CPU
 * baseline leg of the benchmark load it.  It shares no code with the HIP path.
 *
 * Mamba-3-Lite "SSD Reference", section "Math: the recurrence both functions
 * implement", with the per-head scalar A_h complex and the step size real
 * (section "_discretise": abar_t = exp(softplus(dt_t) A_h)):
 *     h_t[n][d] = abar_t h_{t-1}[n][d] + B_t[n] x_t[d]      (state N x D)
 *     y_t[d]    = sum_n C_t[n] h_t[n][d]                    (no conjugation)
 * Every head has its own B and C (section "Shape contract": B_t, C_t are
 * (B, T, H, N)).  x, B, C, A and y are complex; dt is real.  An optional
 * initial state and the final state are held in the page's (D, N) layout
 * ("Shape contract", initial_states (B, H, D, N)), so they are transposed
 * against the running (N, D) state here.
 *
 * Complex values are interleaved (re, im) doubles.  Per token, per head:
 *   delta = softplus(dt)        (max(u, 0) + log1p(exp(-|u|)), the same function)
 *   abar  = exp(delta Re A) (cos(delta Im A) + i sin(delta Im A))
 *   for n, d: h[n][d] = abar h[n][d] + B[n] x[d]            (decay first, then add)
 *   for d:    y[d] = sum_n C[n] h[n][d]                      (n ascending)
 * Build with -ffp-contract=off so every operation rounds as written.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double cx_softplus(double u) {
  double m = u > 0.0 ? u : 0.0;
  return m + log1p(exp(-fabs(u)));
}

/* (ar + i ai)(br + i bi) */
static void cx_mul(double ar, double ai, double br, double bi, double* r, double* i) {
  *r = ar * br - ai * bi;
  *i = ar * bi + ai * br;
}

/*
 * ssd_ref_complex_fwd
 *
 *   ntok tokens on a packed axis, nseq sequences, sequence i owns [cu[i], cu[i+1])
 *   x  (ntok, H, D) complex     B, C (ntok, H, N) complex     dt (ntok, H) real
 *   A  (H) complex
 *   h0 (nseq, H, D, N) complex or NULL (zero)
 *   y  (ntok, H, D) complex, written
 *   hfinal (nseq, H, D, N) complex or NULL
 * Returns 0, -1 on an inconsistent argument, -2 when out of memory.
 */
int ssd_ref_complex_fwd(int64_t ntok, int nseq, const int64_t* cu, int H, int D, int N,
                        const double* x, const double* Bm, const double* Cm, const double* dt,
                        const double* A, const double* h0, double* y, double* hfinal,
                        int nthreads) {
  if (ntok < 0 || nseq < 0 || H <= 0 || D <= 0 || N <= 0) return -1;
  if (nseq > 0 && (cu == NULL || cu[0] != 0 || cu[nseq] != ntok)) return -1;
  for (int i = 0; i < nseq; ++i)
    if (cu[i + 1] < cu[i]) return -1;
  const int64_t npair = (int64_t)nseq * H;
  const size_t ND = (size_t)N * D;
  int err = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int64_t pair = 0; pair < npair; ++pair) {
    const int i = (int)(pair / H), h = (int)(pair % H);
    double* s = (double*)malloc(sizeof(double) * 2 * ND);  /* s[(n D + d) 2 + {0,1}] */
    if (!s) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      err = -2;
      continue;
    }
    for (int n = 0; n < N; ++n)
      for (int d = 0; d < D; ++d) {
        const size_t k = ((size_t)n * D + d) * 2;
        if (h0) {
          const double* src = h0 + ((((size_t)i * H + h) * D + d) * N + n) * 2;
          s[k] = src[0];
          s[k + 1] = src[1];
        } else {
          s[k] = s[k + 1] = 0.0;
        }
      }
    const double Ar = A[2 * h], Ai = A[2 * h + 1];
    for (int64_t t = cu[i]; t < cu[i + 1]; ++t) {
      const double delta = cx_softplus(dt[t * H + h]);
      const double mag = exp(delta * Ar);
      const double ar = mag * cos(delta * Ai), ai = mag * sin(delta * Ai);
      const double* xt = x + ((size_t)t * H + h) * D * 2;
      const double* bt = Bm + ((size_t)t * H + h) * N * 2;
      const double* ct = Cm + ((size_t)t * H + h) * N * 2;
      double* yt = y + ((size_t)t * H + h) * D * 2;
      for (int n = 0; n < N; ++n)
        for (int d = 0; d < D; ++d) {
          double* sk = s + ((size_t)n * D + d) * 2;
          double dr, di, ur, ui;
          cx_mul(ar, ai, sk[0], sk[1], &dr, &di);
          cx_mul(bt[2 * n], bt[2 * n + 1], xt[2 * d], xt[2 * d + 1], &ur, &ui);
          sk[0] = dr + ur;
          sk[1] = di + ui;
        }
      for (int d = 0; d < D; ++d) {
        double accr = 0.0, acci = 0.0;
        for (int n = 0; n < N; ++n) {
          const double* sk = s + ((size_t)n * D + d) * 2;
          double pr, pi;
          cx_mul(ct[2 * n], ct[2 * n + 1], sk[0], sk[1], &pr, &pi);
          accr += pr;
          acci += pi;
        }
        yt[2 * d] = accr;
        yt[2 * d + 1] = acci;
      }
    }
    if (hfinal)
      for (int n = 0; n < N; ++n)
        for (int d = 0; d < D; ++d) {
          double* dst = hfinal + ((((size_t)i * H + h) * D + d) * N + n) * 2;
          dst[0] = s[((size_t)n * D + d) * 2];
          dst[1] = s[((size_t)n * D + d) * 2 + 1];
        }
    free(s);
  }
  return err;
}
