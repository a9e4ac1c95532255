/*
 * ssd_ref.c -- the fp64 sequential oracle for the Mamba-2 SSD forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this file; only the tests, the package's smoke check and the CPU
 * baseline leg of the benchmark load it.  It shares no code with the HIP path.
 *
 * What it computes is the plain recurrence, one token at a time, in fp64:
 *
 *   Mamba-3-Lite "SSD Reference", section "Math: the recurrence both
 *   functions implement":
 *       h_t = abar_t * h_{t-1} + B_t (outer) x_t,   y_t = sum_n C_{t,n} h_{t,n}
 *   and section "_discretise": abar_t = exp(softplus(dt_t) * A).
 *
 * extended with what the Mamba-2 SSD stages on the other pages carry:
 *   - a per-head dt bias added before softplus, and an optional clamp of the
 *     step size (Mamba-2 chunk-cumsum stage, vLLM PR 27299 "Purpose");
 *   - grouped B/C: head h reads group g = h / (H/G) (mamba PR 1012
 *     "Measurements": 64 heads, 8 groups);
 *   - the D skip and the SiLU gate z, out = (C.h + D x) * silu(z)
 *     (cudnn-frontend PR 1133, description: "optional skip/SiLU");
 *   - an initial state that predates the first token and a final state
 *     (SSD Reference, "Inter-chunk propagation": the initial-state term;
 *     cudnn-frontend PR 1133: "initial/final-state");
 *   - packed variable-length batches, where the state restarts at every
 *     sequence boundary (vLLM PR 27299 "Test Plan": continuous batching).
 *
 * The state of one (sequence, head) is a P x N matrix S[p][n] (head dim
 * before state dim, SSD Reference "Shape contract").  Per token:
 *   u     = dt[t,h] + dt_bias[h]
 *   delta = softplus(u) if dt_softplus else u;   clamp to [dt_min, dt_max] if asked
 *   a     = delta * A[h]
 *   S     = exp(a) * S + x[t,h,:] (outer) B[t,g,:]      (decay first, then add)
 *   y     = S . C[t,g,:] + D[h] * x[t,h,:]
 *   out   = y * z / (1 + exp(-z))   if z is given, else y
 *
 * Floating-point order is fixed (p and n ascending, decay before add, readout
 * after update) so the invariants the tests check inside the oracle (split and
 * resume, packed = independent runs, group expansion) hold bit for bit.
 * Build with -ffp-contract=off so every operation rounds as written.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* softplus(u) = log(1 + e^u), written in the overflow-free form
 * max(u, 0) + log1p(exp(-|u|)), which is the same function exactly. */
static double ref_softplus(double u) {
  double m = u > 0.0 ? u : 0.0;
  return m + log1p(exp(-fabs(u)));
}

/*
 * ssd_ref_fwd
 *
 * Token axis is packed: ntok tokens, nseq sequences, sequence i owns tokens
 * [cu[i], cu[i+1]).  A batch of b equal-length sequences of length T laid out
 * contiguously is the case cu = {0, T, 2T, ..., bT}.
 *
 *   x      (ntok, H, P)   double, contiguous
 *   Bm, Cm (ntok, G, N)   double, contiguous
 *   dt     (ntok, H)      double, raw (before bias / softplus)
 *   A      (H)
 *   dt_bias(H) or NULL    (NULL = zero bias)
 *   D      (H) or NULL    (NULL = no skip)
 *   z      (ntok, H, P) or NULL (NULL = no gate)
 *   h0     (nseq, H, P, N) or NULL (NULL = zero initial state)
 *   dt_softplus: 1 = apply softplus to u, 0 = use u as the step size
 *   clamp: 1 = clamp the step size to [dt_min, dt_max] after softplus
 *   chunk: if > 0 and hchunk != NULL, the state after the last token of every
 *          sequence-aligned chunk is stored to hchunk.  Chunks of sequence i
 *          start at cu[i] + k*chunk and hold min(chunk, L_i - k*chunk) tokens;
 *          logical chunk ids run sequence-major (all chunks of sequence 0,
 *          then of sequence 1, ...), empty sequences own no chunk.
 *   y      (ntok, H, P)   output (after the gate)
 *   hfinal (nseq, H, P, N) or NULL: state after the last token of each sequence
 *          (equal to h0, or zero, for an empty sequence)
 *   hchunk (nchunks, H, P, N) or NULL
 *   nthreads: OpenMP threads; <= 0 keeps the runtime default
 *
 * Returns 0 on success, -1 on an inconsistent argument, -2 when out of memory.
 */
int ssd_ref_fwd(int64_t ntok, int nseq, const int64_t* cu, int H, int P, int N,
                int G, const double* x, const double* Bm, const double* Cm,
                const double* dt, const double* A, const double* dt_bias,
                const double* D, const double* z, const double* h0,
                int dt_softplus, int clamp, double dt_min, double dt_max,
                int chunk, double* y, double* hfinal, double* hchunk,
                int nthreads) {
  if (ntok < 0 || nseq < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0) return -1;
  if (H % G != 0) return -1;
  if (nseq > 0 && (cu == NULL || cu[0] != 0 || cu[nseq] != ntok)) return -1;
  for (int i = 0; i < nseq; ++i)
    if (cu[i + 1] < cu[i]) return -1;
  if (hchunk != NULL && chunk <= 0) return -1;

  /* first logical chunk id of every sequence (only used for hchunk) */
  int64_t* first = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nseq + 1));
  if (!first) return -2;
  first[0] = 0;
  for (int i = 0; i < nseq; ++i) {
    int64_t len = cu[i + 1] - cu[i];
    int64_t nck = chunk > 0 ? (len + chunk - 1) / chunk : 0;
    first[i + 1] = first[i] + nck;
  }

  const int hpg = H / G;
  const int64_t npair = (int64_t)nseq * H;
  int err = 0;

#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int64_t pair = 0; pair < npair; ++pair) {
    const int i = (int)(pair / H);
    const int h = (int)(pair % H);
    const int g = h / hpg;
    double* S = (double*)malloc(sizeof(double) * (size_t)P * (size_t)N);
    if (!S) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      err = -2;
      continue;
    }
    if (h0)
      memcpy(S, h0 + ((size_t)i * H + h) * (size_t)P * N,
             sizeof(double) * (size_t)P * N);
    else
      memset(S, 0, sizeof(double) * (size_t)P * N);

    const int64_t t0 = cu[i], t1 = cu[i + 1];
    for (int64_t t = t0; t < t1; ++t) {
      double u = dt[t * H + h] + (dt_bias ? dt_bias[h] : 0.0);
      double delta = dt_softplus ? ref_softplus(u) : u;
      if (clamp) {
        if (delta < dt_min) delta = dt_min;
        if (delta > dt_max) delta = dt_max;
      }
      const double decay = exp(delta * A[h]);
      const double* xt = x + ((size_t)t * H + h) * P;
      const double* bt = Bm + ((size_t)t * G + g) * N;
      const double* ct = Cm + ((size_t)t * G + g) * N;
      double* yt = y + ((size_t)t * H + h) * P;
      for (int p = 0; p < P; ++p) {
        double* row = S + (size_t)p * N;
        const double xp = xt[p];
        for (int n = 0; n < N; ++n) row[n] = decay * row[n] + xp * bt[n];
        double acc = 0.0;
        for (int n = 0; n < N; ++n) acc += row[n] * ct[n];
        double yp = acc + (D ? D[h] * xp : 0.0);
        if (z) {
          const double zz = z[((size_t)t * H + h) * P + p];
          yp = yp * zz / (1.0 + exp(-zz));
        }
        yt[p] = yp;
      }
      if (hchunk) {
        const int64_t k = (t - t0) / chunk;
        const int chunk_end = ((t - t0) % chunk == chunk - 1) || (t == t1 - 1);
        if (chunk_end)
          memcpy(hchunk + ((size_t)(first[i] + k) * H + h) * (size_t)P * N, S,
                 sizeof(double) * (size_t)P * N);
      }
    }
    if (hfinal)
      memcpy(hfinal + ((size_t)i * H + h) * (size_t)P * N, S,
             sizeof(double) * (size_t)P * N);
    free(S);
  }
  free(first);
  return err;
}

/* Number of sequence-aligned chunks the call above emits for hchunk. */
int64_t ssd_ref_num_chunks(int nseq, const int64_t* cu, int chunk) {
  if (chunk <= 0) return -1;
  int64_t k = 0;
  for (int i = 0; i < nseq; ++i) k += (cu[i + 1] - cu[i] + chunk - 1) / chunk;
  return k;
}
