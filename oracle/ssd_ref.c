/*
 * ssd_ref.c -- the fp64 sequential oracle for the Mamba-2 SSD forward pass and
 * its reverse-mode gradient (ssd_ref_bwd, at the end of the file).
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
 *     sequence boundary (vLLM PR 27299 "Test Plan": continuous batching);
 *   - optionally (input_dt = 1) the step size on the input term as well,
 *     S = exp(a) S + delta x (outer) B, the way Mamba-2 implementations
 *     discretise the input; the pages write the recurrence without it, so it
 *     is an option, off by default.  The D skip keeps the raw x.
 *
 * The state of one (sequence, head) is a P x N matrix S[p][n] (head dim
 * before state dim, SSD Reference "Shape contract").  Per token:
 *   u     = dt[t,h] + dt_bias[h]
 *   delta = softplus(u) if dt_softplus else u;   clamp to [dt_min, dt_max] if asked
 *   a     = delta * A[h]
 *   S     = exp(a) * S + xs (outer) B[t,g,:]      (decay first, then add)
 *           with xs = delta * x[t,h,:] if input_dt, else x[t,h,:]
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
 *   input_dt: 1 = scale the input term by the step size (see above)
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
                int dt_softplus, int clamp, double dt_min, double dt_max, int input_dt,
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
        const double xs = input_dt ? delta * xp : xp;
        for (int n = 0; n < N; ++n) row[n] = decay * row[n] + xs * bt[n];
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

/*
 * ssd_ref_bwd -- reverse-mode gradient of ssd_ref_fwd, in fp64.
 *
 * The backward pass the pages describe (mamba PR 1012, "Measurements": the
 * dx/ddt, dB, dC, dA-cumsum, state-passing and dstates backward stages;
 * cudnn-frontend PR 1133: first-order backward checked against fp64 gradients;
 * SSD Reference, section 6 "The autograd backward contract": exact gradients
 * of every input) is here the adjoint of the recurrence above, taken one
 * token at a time in reverse:
 *
 *   G      := dL/dS_t, starting from dL/dS_final (dfinal, or zero)
 *   per token t, newest first, with S_t and S_{t-1} recomputed:
 *     y_t    = S_t . C_t + D x_t              (before the gate)
 *     dy_t   = dout_t * silu(z_t)             (dout_t without a gate)
 *     dz_t   = dout_t * y_t * silu'(z_t),     silu'(z) = s (1 + z (1 - s)), s = sigmoid(z)
 *     G     += dy_t (outer) C_t               (now dL/dS_t, all paths)
 *     dC_t  += S_t^T dy_t                     (summed over the heads of the group)
 *     dx_t   = f G B_t + D dy_t               (f = delta_t with input_dt, else 1)
 *     dB_t  += f G^T x_t                      (summed over the heads of the group)
 *     dD    += dy_t . x_t
 *     da_t   = exp(a_t) <G, S_{t-1}>          (a_t = delta_t A)
 *     G      = exp(a_t) G                     (dL/dS_{t-1})
 *     dA    += da_t delta_t;  ddelta = da_t A (+ x_t . G B_t with input_dt)
 *     ddt_t  = ddelta * sigmoid(u_t)          (softplus' = sigmoid; ddelta itself
 *                                              without softplus; 0 where the
 *                                              clamp is active)
 *     ddt_bias += ddt_t
 *   dh0 = G after the sequence's first token.
 *
 * The loss this differentiates is L = sum(dout * y) + sum(dfinal * S_final).
 * States are recomputed from checkpoints taken every kCheck tokens, so memory
 * stays O(kCheck P N) per (sequence, head).  Work is split by group: one
 * thread owns every head of a group (all sequences), so the group-summed dB
 * and dC and the per-head dA, ddt_bias, dD need no atomics, and the order of
 * every sum is fixed.
 *
 *   dout   (ntok, H, P)      gradient of y (after the gate)
 *   dfinal (nseq, H, P, N) or NULL
 *   dx (ntok,H,P), dB and dC (ntok,G,N), ddt (ntok,H), dA (H), ddt_bias (H),
 *   dD (H) (may be NULL when D is NULL), dz (ntok,H,P) (NULL when z is NULL),
 *   dh0 (nseq,H,P,N) or NULL -- all written (not accumulated into).
 *
 * Returns 0 on success, -1 on an inconsistent argument, -2 when out of memory.
 */
enum { kCheck = 64 };

static void ref_step_size(double u, int dt_softplus, int clamp, double dt_min,
                          double dt_max, double* delta, double* ddelta_du) {
  double d = dt_softplus ? ref_softplus(u) : u;
  double g = dt_softplus ? 1.0 / (1.0 + exp(-u)) : 1.0;
  if (clamp) {
    if (d < dt_min) { d = dt_min; g = 0.0; }
    if (d > dt_max) { d = dt_max; g = 0.0; }
  }
  *delta = d;
  *ddelta_du = g;
}

int ssd_ref_bwd(int64_t ntok, int nseq, const int64_t* cu, int H, int P, int N,
                int G, const double* x, const double* Bm, const double* Cm,
                const double* dt, const double* A, const double* dt_bias,
                const double* D, const double* z, const double* h0,
                int dt_softplus, int clamp, double dt_min, double dt_max, int input_dt,
                const double* dout, const double* dfinal,
                double* dx, double* dB, double* dC, double* ddt, double* dA,
                double* ddt_bias, double* dD, double* dz, double* dh0,
                int nthreads) {
  if (ntok < 0 || nseq < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0) return -1;
  if (H % G != 0) return -1;
  if (nseq > 0 && (cu == NULL || cu[0] != 0 || cu[nseq] != ntok)) return -1;
  for (int i = 0; i < nseq; ++i)
    if (cu[i + 1] < cu[i]) return -1;
  if (!dout || !dx || !dB || !dC || !ddt || !dA || !ddt_bias) return -1;
  if (z && !dz) return -1;

  const int hpg = H / G;
  const size_t PN = (size_t)P * N;
  memset(dB, 0, sizeof(double) * (size_t)ntok * G * N);
  memset(dC, 0, sizeof(double) * (size_t)ntok * G * N);
  int err = 0;

#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int g = 0; g < G; ++g) {
    /* states of one checkpoint block (kCheck + 1 of them: the one entering
     * the block first), the running adjoint, and the block's checkpoints */
    double* blk = (double*)malloc(sizeof(double) * (size_t)(kCheck + 1) * PN);
    double* Gs = (double*)malloc(sizeof(double) * PN);
    double* ck = NULL;
    int64_t ck_cap = 0;
    if (!blk || !Gs) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      err = -2;
      free(blk); free(Gs);
      continue;
    }
    for (int hh = 0; hh < hpg; ++hh) {
      const int h = g * hpg + hh;
      double sA = 0.0, sBias = 0.0, sD = 0.0;
      for (int i = 0; i < nseq && !err; ++i) {
        const int64_t t0 = cu[i], t1 = cu[i + 1], L = t1 - t0;
        const int64_t nblk = (L + kCheck - 1) / kCheck;
        if (nblk > ck_cap) {
          free(ck);
          ck = (double*)malloc(sizeof(double) * (size_t)nblk * PN);
          ck_cap = ck ? nblk : 0;
          if (!ck) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            err = -2;
            break;
          }
        }
        /* forward sweep: the state entering every block */
        double* S = blk;
        if (h0)
          memcpy(S, h0 + ((size_t)i * H + h) * PN, sizeof(double) * PN);
        else
          memset(S, 0, sizeof(double) * PN);
        for (int64_t t = t0; t < t1; ++t) {
          if ((t - t0) % kCheck == 0)
            memcpy(ck + (size_t)((t - t0) / kCheck) * PN, S, sizeof(double) * PN);
          double delta, gd;
          ref_step_size(dt[t * H + h] + (dt_bias ? dt_bias[h] : 0.0), dt_softplus, clamp,
                        dt_min, dt_max, &delta, &gd);
          const double decay = exp(delta * A[h]);
          const double f = input_dt ? delta : 1.0;
          const double* xt = x + ((size_t)t * H + h) * P;
          const double* bt = Bm + ((size_t)t * G + g) * N;
          for (int p = 0; p < P; ++p)
            for (int n = 0; n < N; ++n)
              S[(size_t)p * N + n] = decay * S[(size_t)p * N + n] + (f * xt[p]) * bt[n];
        }
        /* reverse sweep */
        if (dfinal)
          memcpy(Gs, dfinal + ((size_t)i * H + h) * PN, sizeof(double) * PN);
        else
          memset(Gs, 0, sizeof(double) * PN);
        for (int64_t b = nblk - 1; b >= 0; --b) {
          const int64_t ta = t0 + b * kCheck;
          const int64_t tb = ta + kCheck < t1 ? ta + kCheck : t1;
          /* blk[k] = state before token ta + k, blk[k + 1] = after it */
          memcpy(blk, ck + (size_t)b * PN, sizeof(double) * PN);
          for (int64_t t = ta; t < tb; ++t) {
            double delta, gd;
            ref_step_size(dt[t * H + h] + (dt_bias ? dt_bias[h] : 0.0), dt_softplus, clamp,
                          dt_min, dt_max, &delta, &gd);
            const double decay = exp(delta * A[h]);
            const double f = input_dt ? delta : 1.0;
            const double* xt = x + ((size_t)t * H + h) * P;
            const double* bt = Bm + ((size_t)t * G + g) * N;
            const double* Sp = blk + (size_t)(t - ta) * PN;
            double* Sn = blk + (size_t)(t - ta + 1) * PN;
            for (int p = 0; p < P; ++p)
              for (int n = 0; n < N; ++n)
                Sn[(size_t)p * N + n] = decay * Sp[(size_t)p * N + n] + (f * xt[p]) * bt[n];
          }
          for (int64_t t = tb - 1; t >= ta; --t) {
            const double u = dt[t * H + h] + (dt_bias ? dt_bias[h] : 0.0);
            double delta, gd;
            ref_step_size(u, dt_softplus, clamp, dt_min, dt_max, &delta, &gd);
            const double decay = exp(delta * A[h]);
            const double* xt = x + ((size_t)t * H + h) * P;
            const double* bt = Bm + ((size_t)t * G + g) * N;
            const double* ct = Cm + ((size_t)t * G + g) * N;
            const double* dot = dout + ((size_t)t * H + h) * P;
            const double* St = blk + (size_t)(t - ta + 1) * PN;
            const double* Sp = blk + (size_t)(t - ta) * PN;
            double* dxt = dx + ((size_t)t * H + h) * P;
            double* dbt = dB + ((size_t)t * G + g) * N;
            double* dct = dC + ((size_t)t * G + g) * N;
            const double f = input_dt ? delta : 1.0;
            double da = 0.0, din = 0.0;
            for (int p = 0; p < P; ++p) {
              const double* srow = St + (size_t)p * N;
              double* grow = Gs + (size_t)p * N;
              double dy = dot[p];
              if (z) {
                double y = 0.0;
                for (int n = 0; n < N; ++n) y += srow[n] * ct[n];
                y += D ? D[h] * xt[p] : 0.0;
                const double zz = z[((size_t)t * H + h) * P + p];
                const double sg = 1.0 / (1.0 + exp(-zz));
                dz[((size_t)t * H + h) * P + p] = dy * y * (sg * (1.0 + zz * (1.0 - sg)));
                dy = dy * zz * sg;
              }
              sD += dy * xt[p];
              double acc = 0.0;
              for (int n = 0; n < N; ++n) {
                dct[n] += srow[n] * dy;
                grow[n] += dy * ct[n];
                acc += grow[n] * bt[n];
                dbt[n] += grow[n] * (f * xt[p]);
                da += grow[n] * Sp[(size_t)p * N + n];
              }
              din += xt[p] * acc;
              dxt[p] = f * acc + (D ? D[h] * dy : 0.0);
            }
            da *= decay;
            for (size_t q = 0; q < PN; ++q) Gs[q] *= decay;
            sA += da * delta;
            const double du = (da * A[h] + (input_dt ? din : 0.0)) * gd;
            ddt[t * H + h] = du;
            sBias += du;
          }
        }
        if (dh0) memcpy(dh0 + ((size_t)i * H + h) * PN, Gs, sizeof(double) * PN);
      }
      dA[h] = sA;
      ddt_bias[h] = sBias;
      if (dD) dD[h] = sD;
    }
    free(ck);
    free(blk);
    free(Gs);
  }
  return err;
}
