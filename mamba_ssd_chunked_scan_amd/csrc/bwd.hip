// bwd.hip -- the kernels of the SSD backward pass that are not scans.
//
// The backward of the recurrence (mamba PR 1012, "Measurements": the dx/ddt,
// dB, dC, dA-cumsum and dstates backward stages; SSD Reference, section 6 "The
// autograd backward contract") is run as three more SSD forward scans on
// operands this file prepares, plus the pieces below:
//
//   dL/dS_t = G_t obeys G_t = exp(a_{t+1}) G_{t+1} + dy_t (outer) C_t, a scan
//   backwards in time.  Read with B it gives dx, read with x (state
//   transposed) it gives the head's share of dB; the forward state S_t read
//   with dy (state transposed) gives the head's share of dC.  Run on reversed
//   sequences, each is an ordinary forward scan with the step sizes shifted by
//   one token (the decay between t and t+1 belongs to token t+1) and the final
//   state's gradient as the initial state.
//
//   For the step sizes, dL/da_t is the sum over the chunk's later tokens of
//   dL/dcs (see k_step_dcs): row and column sums of the strictly lower
//   triangle of M = exp(segsum) o (C.B^T) o (dy.x^T), plus the terms of the
//   states entering and leaving the chunk.  The state leaving a chunk gets its
//   gradient from the mirrored dx scan's carry-in states, because that scan
//   cuts each mirrored sequence so that its chunk boundaries fall on the
//   forward ones (a short first chunk of L mod C tokens).
//
// Products are fp32; sums that accumulate many terms are fp64.  Every sum has a
// fixed order, so the results are deterministic.
#include "kernels.hpp"
#include "stage_varlen.hpp"

namespace ssd {

namespace {

// ---- tokens on the packed axis (b * T in batch mode)

// Sequence span [s0, s1) of packed token tp.
__device__ __forceinline__ void seq_of(const BwdGeo& q, int tp, int& s0, int& s1) {
  if (!q.cu) {
    s0 = (tp / q.T) * q.T;
    s1 = s0 + q.T;
    return;
  }
  int lo = 0, hi = q.nseq;  // find the last i with cu[i] <= tp
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (clamp_tok(q.cu[mid], q.T) <= tp) lo = mid; else hi = mid;
  }
  s0 = clamp_tok(q.cu[lo], q.T);
  s1 = max(clamp_tok(q.cu[lo + 1], q.T), s0);
  if (tp < s0 || tp >= s1) {  // a token outside every sequence stands alone
    s0 = tp;
    s1 = tp + 1;
  }
}

// The token at the mirrored position of tp inside its sequence.
__device__ __forceinline__ int mirror(const BwdGeo& q, int tp) {
  int s0, s1;
  seq_of(q, tp, s0, s1);
  return s0 + s1 - 1 - tp;
}

template <typename T>
__device__ __forceinline__ const T* tok_row(const TArg& a, const BwdGeo& q, int tp, int hg) {
  return q.cu ? row_ptr<T>(a, 0, tp, hg) : row_ptr<T>(a, tp / q.T, tp % q.T, hg);
}
__device__ __forceinline__ float* tok_row_f32(const TArg& a, const BwdGeo& q, int tp, int hg) {
  return q.cu ? row_ptr_mut<float>(a, 0, tp, hg) : row_ptr_mut<float>(a, tp / q.T, tp % q.T, hg);
}

template <typename T>
__device__ __forceinline__ float load_f32(const TArg& a, const BwdGeo& q, int tp, int hg, int i) {
  return to_f32<T>(tok_row<T>(a, q, tp, hg)[i]);
}
__device__ __forceinline__ float load_any(const TArg& a, int dtype, const BwdGeo& q, int tp, int hg,
                                          int i) {
  return dtype == DT_BF16 ? load_f32<bf16>(a, q, tp, hg, i) : load_f32<float>(a, q, tp, hg, i);
}

__device__ __forceinline__ float sigmoid(float v) { return 1.0f / (1.0f + __expf(-v)); }

// Step size and d(step)/du of one token: softplus (or identity), clamp.
__device__ __forceinline__ void step_size(float u, int softplus, int clamp, float dt_min,
                                          float dt_max, float& delta, float& gd) {
  float d = u, g = 1.0f;
  if (softplus) {
    d = u > 20.0f ? u : log1pf(__expf(u));
    g = sigmoid(u);
  }
  if (clamp) {
    if (d < dt_min) { d = dt_min; g = 0.0f; }
    if (d > dt_max) { d = dt_max; g = 0.0f; }
  }
  delta = d;
  gd = g;
}

// ---- rows of width W (a multiple of 4): W / 4 threads per row, each on 4
// consecutive elements; 256 / (W / 4) rows per workgroup.  Indices stay 32-bit
// (the host checks that the row counts fit).
struct Row {
  int row, c, tpr;
  bool ok;
};
__device__ __forceinline__ Row row_of(int W, int nrows) {
  Row r;
  r.tpr = W / 4;
  const int rpb = 256 / r.tpr;
  const int k = threadIdx.x / r.tpr;
  r.row = blockIdx.x * rpb + k;
  r.c = (threadIdx.x % r.tpr) * 4;
  r.ok = k < rpb && r.row < nrows;
  return r;
}

__device__ __forceinline__ f32x4 load4(const TArg& a, int dtype, const BwdGeo& q, int tp, int hg,
                                       int c) {
  f32x4 v;
  if (dtype == DT_BF16) {
    const bf16x4 b = *reinterpret_cast<const bf16x4*>(tok_row<bf16>(a, q, tp, hg) + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (float)b[i];
  } else {
    v = *reinterpret_cast<const f32x4*>(tok_row<float>(a, q, tp, hg) + c);
  }
  return v;
}

// ---- dst (ntok, R, W) fp32 = rows of src, optionally mirrored in time and
// with dst row r reading src row r / rep (a group's row for each of its heads)
__global__ __launch_bounds__(256) void k_gather(BwdGeo q, TArg src, int dtype, int R, int W,
                                                int rep, int reverse, float* dst) {
  const Row rw = row_of(W, q.ntok * R);
  if (!rw.ok) return;
  const int tp = rw.row / R, r = rw.row % R;
  const int ts = reverse ? mirror(q, tp) : tp;
  *reinterpret_cast<f32x4*>(dst + (int64_t)rw.row * W + rw.c) = load4(src, dtype, q, ts, r / rep, rw.c);
}

// ---- the gate: dy = dout silu(z), dz = dout y silu'(z) (dy = dout without a
// gate); dy is written in token order (when dy is given) and mirrored; dz only
// when y is given
__global__ __launch_bounds__(256) void k_gate(BwdGeo q, TArg dout, int dout_dtype, TArg z,
                                              int z_dtype, const float* y, float* dy,
                                              float* dy_rev, TArg dz) {
  const Row rw = row_of(q.P, q.ntok * q.H);
  if (!rw.ok) return;
  const int tp = rw.row / q.H, h = rw.row % q.H;
  const int64_t o = (int64_t)rw.row * q.P + rw.c;
  const f32x4 go = load4(dout, dout_dtype, q, tp, h, rw.c);
  f32x4 g = go;
  if (z.p) {
    const f32x4 zz = load4(z, z_dtype, q, tp, h, rw.c);
#pragma unroll
    for (int i = 0; i < 4; ++i) g[i] = go[i] * zz[i] * sigmoid(zz[i]);
    if (y) {
      const f32x4 yy = *reinterpret_cast<const f32x4*>(y + o);
      f32x4 d;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float s = sigmoid(zz[i]);
        d[i] = go[i] * yy[i] * (s * (1.0f + zz[i] * (1.0f - s)));
      }
      *reinterpret_cast<f32x4*>(tok_row_f32(dz, q, tp, h) + rw.c) = d;
    }
  }
  if (dy) *reinterpret_cast<f32x4*>(dy + o) = g;
  *reinterpret_cast<f32x4*>(dy_rev + ((int64_t)mirror(q, tp) * q.H + h) * q.P + rw.c) = g;
}

// ---- per (token, head): step size, d(step)/du, and the mirrored, shifted
// step of the backward scans (the next token's step; 0 at a sequence's end)
__global__ __launch_bounds__(256) void k_steps(BwdGeo q, TArg dt, int dt_dtype, const float* A,
                                               const float* dt_bias, int softplus, int clamp,
                                               float dt_min, float dt_max, float* delta,
                                               float* gd, float* dt_rev) {
  const int64_t total = (int64_t)q.ntok * q.H;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int h = (int)(i % q.H);
    const int tp = (int)(i / q.H);
    const float bias = dt_bias ? dt_bias[h] : 0.0f;
    float d, g;
    step_size(load_any(dt, dt_dtype, q, tp, h, 0) + bias, softplus, clamp, dt_min, dt_max, d, g);
    delta[i] = d;
    gd[i] = g;
    if (!dt_rev) continue;
    int s0, s1;
    seq_of(q, tp, s0, s1);
    float dn = 0.0f;
    if (tp + 1 < s1)
      step_size(load_any(dt, dt_dtype, q, tp + 1, h, 0) + bias, softplus, clamp, dt_min, dt_max,
                dn, g);
    dt_rev[(int64_t)(s0 + s1 - 1 - tp) * q.H + h] = dn;
  }
}

// ---- per (token, head) row: dx = f (mirrored dx-scan output G B) + D dy, dy .
// x for dD and, when the step size f = delta scales the input term, x . G B
// for its gradient; the row's partial sums meet in LDS and its first thread
// adds them in order
__global__ __launch_bounds__(256) void k_tokens(BwdGeo q, TArg x, int x_dtype, const float* D,
                                                const float* dy, const float* gx_rev,
                                                const float* delta, TArg dx, float* dyx,
                                                float* xg) {
  __shared__ double part[2][256];
  const Row rw = row_of(q.P, q.ntok * q.H);
  double sx = 0.0, sg = 0.0;
  if (rw.ok) {
    const int tp = rw.row / q.H, h = rw.row % q.H;
    const int64_t o = (int64_t)rw.row * q.P + rw.c;
    const float Dh = D ? D[h] : 0.0f;
    const float f = delta ? delta[rw.row] : 1.0f;
    const f32x4 xv = load4(x, x_dtype, q, tp, h, rw.c);
    const f32x4 g = *reinterpret_cast<const f32x4*>(gx_rev + ((int64_t)mirror(q, tp) * q.H + h) * q.P + rw.c);
    const f32x4 d = *reinterpret_cast<const f32x4*>(dy + o);
    f32x4 out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[i] = f * g[i] + Dh * d[i];
      sx += (double)d[i] * xv[i];
      sg += (double)xv[i] * g[i];
    }
    *reinterpret_cast<f32x4*>(tok_row_f32(dx, q, tp, h) + rw.c) = out;
  }
  part[0][threadIdx.x] = sx;
  part[1][threadIdx.x] = sg;
  __syncthreads();
  if (rw.ok && rw.c == 0) {
    double c = 0.0, e = 0.0;
    for (int k = 0; k < rw.tpr; ++k) {
      c += part[0][threadIdx.x + k];
      e += part[1][threadIdx.x + k];
    }
    dyx[rw.row] = (float)c;
    if (xg) xg[rw.row] = (float)e;
  }
}

// ---- per (token, group) row: dB and dC summed over the group's heads (dB's
// scan ran mirrored)
__global__ __launch_bounds__(256) void k_group_sums(BwdGeo q, const float* gb_rev,
                                                    const float* gc, const float* delta,
                                                    TArg dB, TArg dC) {
  const Row rw = row_of(q.N, q.ntok * q.G);
  if (!rw.ok) return;
  const int tp = rw.row / q.G, g = rw.row % q.G;
  const int tm = mirror(q, tp);
  f32x4 sb = {0.0f, 0.0f, 0.0f, 0.0f}, sc = sb;
  for (int k = 0; k < q.hpg; ++k) {
    const int h = g * q.hpg + k;
    const float f = delta ? delta[(int64_t)tp * q.H + h] : 1.0f;  // (input term's step)
    sb += f * *reinterpret_cast<const f32x4*>(gb_rev + ((int64_t)tm * q.H + h) * q.N + rw.c);
    sc += *reinterpret_cast<const f32x4*>(gc + ((int64_t)tp * q.H + h) * q.N + rw.c);
  }
  *reinterpret_cast<f32x4*>(tok_row_f32(dB, q, tp, g) + rw.c) = sb;
  *reinterpret_cast<f32x4*>(tok_row_f32(dC, q, tp, g) + rw.c) = sc;
}

__device__ __forceinline__ double block_sum(double v, double* lds) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  v = wave_inclusive_sum_f64(v);
  if (lane == kWave - 1) lds[wave] = v;
  __syncthreads();
  const double t = lds[0] + lds[1] + lds[2] + lds[3];
  __syncthreads();
  return t;
}

// Sequence i's span on the packed axis (batch mode: cu == NULL, length T each).
__device__ __forceinline__ void span_of(const BwdGeo& q, int i, int& s0, int& L) {
  if (q.cu) {
    seq_span(q.cu, i, q.T, s0, L);
  } else {
    s0 = i * q.T;
    L = q.T;
  }
}

// ---- the chunk table of the mirrored scans (layout of ssd_varlen_meta_len):
// sequence i of length L is cut into the same number of chunks as forward,
// ceil(L / C), but shifted so that its boundaries mirror the forward ones:
// chunk k covers positions [max(0, kC - s), min(L, (k+1)C - s)) with
// s = (C - L mod C) mod C.  In batch mode it also writes cu = {0, T, 2T, ..}.
__global__ __launch_bounds__(256) void k_mirror_meta(BwdGeo q, int C, int K, int32_t* meta,
                                                     int32_t* cu_out) {
  __shared__ int lds_waves[4];
  int32_t* first = meta + kMetaHeader + 3 * K;
  int base = 0;
  for (int i0 = 0; i0 < q.nseq; i0 += blockDim.x) {
    const int i = i0 + threadIdx.x;
    int n = 0;
    if (i < q.nseq) {
      int st, L;
      span_of(q, i, st, L);
      n = (L + C - 1) / C;
      if (cu_out) cu_out[i] = st;
    }
    int tot;
    const int ex = block_exclusive_scan(n, lds_waves, tot);
    if (i < q.nseq) first[i] = min(base + ex, K);
    base = min(base + tot, K);
  }
  if (threadIdx.x == 0) {
    first[q.nseq] = base;
    meta[0] = base;
    meta[1] = q.nseq;
    meta[2] = C;
    meta[3] = K;
    if (cu_out) cu_out[q.nseq] = q.ntok;
  }
  __syncthreads();
  const int Kr = base;
  for (int j = threadIdx.x; j < K; j += blockDim.x) {
    int32_t* e = meta + kMetaHeader + 3 * j;
    if (j >= Kr) {
      e[0] = -1; e[1] = 0; e[2] = 0;
      continue;
    }
    int lo = 0, hi = q.nseq - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (first[mid] <= j) lo = mid; else hi = mid - 1;
    }
    const int k = j - first[lo];
    int st, L;
    span_of(q, lo, st, L);
    const int sh = (C - L % C) % C;
    const int a = max(0, k * C - sh), b = min(L, (k + 1) * C - sh);
    e[0] = lo;
    e[1] = st + a;
    e[2] = b - a;
  }
}

// ---- one workgroup per (forward chunk j, head h): the step-size gradients of
// the chunk's tokens and the chunk's shares of dA, ddt_bias and dD; at a
// sequence's first chunk also dh0 = exp(a_first) G_first.
//
// dL/da_t = sum over l >= t in the chunk of dL/dcs_l, with cs the chunk's
// inclusive cumsum of a and Lambda = cs at its last token:
//   dL/dcs_l = sum_{s<l} M_ls - sum_{l'>l} M_l'l + Q_l - R_l  (+ at the last
//              token: exp(Lambda) <dS, Hin> + sum_s R_s)
//   M_ls = exp(cs_l - cs_s) (C_l . B_s) (dy_l . x_s) f_s   (s < l: the diagonal
//          terms of the two sums are equal and cancel, so neither holds them)
//   Q_l  = exp(cs_l) dy_l . (Hin C_l),   R_l = exp(Lambda - cs_l) f_l x_l . (dS B_l)
// with f the step size where it scales the input term (xg != NULL), else 1;
// there the step size also reaches the loss through the input, and its
// gradient gains x_t . G_t B_t (xg, from k_tokens).
// Hin is the state entering the chunk (forward scan's carry-in), dS the
// gradient of the state leaving it through later tokens: exp(a_next) G_next
// (G_next the mirrored dx scan's carry-in for the next chunk) or dfinal at a
// sequence's last chunk.  Every term decays as it should, so nothing cancels
// however strong the decay.  The vectors in Q and R are the inter-chunk parts
// of the forward scan's output (Hin C_l, scaled by exp(cs_l)) and of the
// mirrored dx scan's output at the mirrored token (dS B_l, scaled by
// exp(Lambda - cs_l): that scan's chunk cumsum at token l), so only their dot
// products with dy_l and x_l are left here.  cs itself is summed in fp64 from
// the step sizes: with strong decay it reaches |cs| ~ 1e4 while the segments
// that still matter span |cs_l - cs_s| < ~100, and an fp32 sum would leave
// each such segment an absolute error of |cs| 2^-24.
//   CB:      forward scan's C.B^T (K, G, C, C)
//   DX:      dy.x^T per head (K, H, C, C), the dC scan's C.B^T
//   yo_f:    forward scan's inter-chunk output, (tokens, H, P)
//   yo_r:    mirrored dx scan's inter-chunk output, (tokens, H, P), mirrored
//   fwd_st:  forward scan's carry-in states, by forward chunk
//   mir_st:  mirrored dx scan's carry-in states, by mirrored chunk
//   gfirst:  mirrored dx scan's final states (G at each sequence's first token)
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int d = kWave / 2; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
  return v;  // (the same in every lane: each level adds the same two numbers)
}

template <int C>
__global__ __launch_bounds__(256) void k_step_dcs(BwdGeo q, Geo gf, const float* CB,
                                                  const float* DX, const float* yo_f,
                                                  const float* yo_r, const float* xf,
                                                  const float* dy, const float* dyx,
                                                  const float* delta, const float* gd,
                                                  const float* A, const float* fwd_st,
                                                  const float* mir_st, const float* gfirst,
                                                  const float* dfinal, const float* xg, TArg ddt,
                                                  double* part, float* dh0) {
  __shared__ double lds[4];
  __shared__ float s_a[256];
  __shared__ float s_f[256];
  __shared__ double s_cs[256];
  __shared__ double s_col[4][256];  // per-wave column sums of M
  __shared__ double s_row[256];     // row sums of M
  __shared__ double s_qr[2][256];   // per-thread partial dot products: Q, R
  __shared__ double s_r[256];       // R per row (for the Lambda term)
  __shared__ double s_dcs[256];
  const int j = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  Chunk c;
  const bool live = get_chunk(gf, j, c);
  double* pj = part + ((int64_t)j * q.H + h) * 3;
  if (!live) {
    if (tid == 0) pj[0] = pj[1] = pj[2] = 0.0;
    return;
  }
  int fi, li;
  seq_chunks(gf, c.seq, fi, li);
  const int jl = j - fi, len = c.len, g = h / q.hpg;
  const int64_t PN = (int64_t)q.P * q.N;
  const float Ah = A[h];
  const int tp0 = c.b * q.T + c.t0;  // the chunk's first token on the packed axis
  int s0, s1;
  seq_of(q, tp0, s0, s1);
  if (tid < len) {
    const float d = delta[(int64_t)(tp0 + tid) * q.H + h];
    s_a[tid] = d * Ah;
    s_f[tid] = xg ? d : 1.0f;
  }
  __syncthreads();
  if (tid < len) {
    double acc = 0.0;
    for (int k = 0; k <= tid; ++k) acc += (double)s_a[k];
    s_cs[tid] = acc;
  }
  __syncthreads();
  const double lam = s_cs[len - 1];

  // the states at the chunk's two ends (for the Lambda term)
  const float* Hin = fwd_st + ((int64_t)j * q.H + h) * PN;
  const bool last = j == li - 1;
  const float* dS = nullptr;
  float dscale = 1.0f;
  if (!last) {
    dS = mir_st + ((int64_t)(li - (jl + 1)) * q.H + h) * PN;
    dscale = __expf(delta[(int64_t)(tp0 + len) * q.H + h] * Ah);
  } else if (dfinal) {
    dS = dfinal + ((int64_t)c.seq * q.H + h) * PN;
  }

  // row and column sums of M: wave w takes rows l = w, w + 4, ..; lane k the
  // columns k, k + 64, ..  (coalesced rows of CB and DX); every M_ls is
  // formed once and added to both sums, in fp64.  Four rows per pass, their
  // loads issued together (clamped in bounds, masked after).
  {
    constexpr int NI = C >= kWave ? C / kWave : 1;
    const float* cbm = CB + ((int64_t)j * q.G + g) * C * C;
    const float* dxm = DX + ((int64_t)j * q.H + h) * C * C;
    double col[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) col[i] = 0.0;
    for (int l0 = wave; l0 < len; l0 += 16) {
      float cb[4][NI], dx[4][NI];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int lr = min(l0 + 4 * r, len - 1);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int sc = min(lane + kWave * i, C - 1);
          cb[r][i] = cbm[lr * C + sc];
          dx[r][i] = dxm[lr * C + sc];
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int l = l0 + 4 * r;
        const double csl = s_cs[min(l, len - 1)];
        double rp = 0.0;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int sc = lane + kWave * i;
          if (sc < l && l < len) {
            const float m = __expf((float)(csl - s_cs[sc])) * cb[r][i] * dx[r][i] * s_f[sc];
            rp += (double)m;
            col[i] += (double)m;
          }
        }
        rp = wave_sum_f64(rp);
        if (lane == 0 && l < len) s_row[l] = rp;
      }
    }
#pragma unroll
    for (int i = 0; i < NI; ++i)
      if (lane + kWave * i < C) s_col[wave][lane + kWave * i] = col[i];
  }

  // Q and R: tpr threads per row, each over an interleaved share of p
  constexpr int tpr = 256 / C;
  const int l = tid / tpr, part_k = tid % tpr;
  double qs = 0.0, rs = 0.0;
  if (l < len) {
    const int64_t rf = ((int64_t)(tp0 + l) * q.H + h) * q.P;
    const int64_t rr = ((int64_t)(s0 + s1 - 1 - (tp0 + l)) * q.H + h) * q.P;
#pragma unroll 2
    for (int p = part_k * 4; p < q.P; p += tpr * 4) {
      const f32x4 d = *reinterpret_cast<const f32x4*>(dy + rf + p);
      const f32x4 yf = *reinterpret_cast<const f32x4*>(yo_f + rf + p);
      const f32x4 xv = *reinterpret_cast<const f32x4*>(xf + rf + p);
      const f32x4 yr = *reinterpret_cast<const f32x4*>(yo_r + rr + p);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qs += (double)(d[i] * yf[i]);
        rs += (double)(xv[i] * yr[i]);
      }
    }
  }
  s_qr[0][tid] = qs;
  s_qr[1][tid] = rs;
  // <dS, Hin> for the last token's Lambda term
  double ip = 0.0;
  if (dS) {
#pragma unroll 4
    for (int64_t k = tid * 4; k < PN; k += 256 * 4) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(dS + k);
      const f32x4 b = *reinterpret_cast<const f32x4*>(Hin + k);
#pragma unroll
      for (int i = 0; i < 4; ++i) ip += (double)a[i] * b[i];
    }
  }
  ip = block_sum(ip, lds);  // (its barrier publishes s_row, s_col and s_qr)
  if (tid < len) {
    double qq = 0.0, r = 0.0;
    for (int k = 0; k < tpr; ++k) {
      qq += s_qr[0][tid * tpr + k];
      r += s_qr[1][tid * tpr + k];
    }
    const double b = s_col[0][tid] + s_col[1][tid] + s_col[2][tid] + s_col[3][tid];
    r *= s_f[tid];
    s_dcs[tid] = s_row[tid] - b + qq - r;
    s_r[tid] = r;
  }
  __syncthreads();
  if (tid == 0) {
    double sr = 0.0;
    for (int k = 0; k < len; ++k) sr += s_r[k];
    s_dcs[len - 1] += (double)dscale * __expf((float)lam) * ip + sr;
  }
  __syncthreads();
  double sa = 0.0, sb2 = 0.0, sx = 0.0;
  if (tid < len) {
    double da = 0.0;
    for (int k = len - 1; k >= tid; --k) da += s_dcs[k];
    const int64_t it = (int64_t)(tp0 + tid) * q.H + h;
    const double gg = (da * Ah + (xg ? (double)xg[it] : 0.0)) * gd[it];
    tok_row_f32(ddt, q, tp0 + tid, h)[0] = (float)gg;
    sa = da * delta[it];
    sb2 = gg;
    sx = dyx[it];
  }
  sa = block_sum(sa, lds);
  sb2 = block_sum(sb2, lds);
  sx = block_sum(sx, lds);
  if (tid == 0) {
    pj[0] = sa;
    pj[1] = sb2;
    pj[2] = sx;
  }
  if (jl == 0 && dh0) {
    const float* Gf = gfirst + ((int64_t)c.seq * q.H + h) * PN;
    const float e = __expf(delta[(int64_t)tp0 * q.H + h] * Ah);
    float* dst = dh0 + ((int64_t)c.seq * q.H + h) * PN;
    for (int64_t k = tid; k < PN; k += 256) dst[k] = e * Gf[k];
  }
}

// ---- per head: dA, ddt_bias, dD from the chunks' shares (in chunk order),
// and dh0 = G_first for sequences without tokens
__global__ __launch_bounds__(256) void k_step_heads(BwdGeo q, int K, const double* part,
                                                    const float* gfirst, float* dA,
                                                    float* ddt_bias, float* dD, float* dh0) {
  const int h = blockIdx.x, tid = threadIdx.x;
  // the chunks' shares are loaded 256 at a time by all threads and added by
  // one, in chunk order
  __shared__ double s_p[3][256];
  double a = 0.0, b = 0.0, x = 0.0;
  for (int j0 = 0; j0 < K; j0 += 256) {
    if (j0 + tid < K) {
      const double* pj = part + ((int64_t)(j0 + tid) * q.H + h) * 3;
      s_p[0][tid] = pj[0];
      s_p[1][tid] = pj[1];
      s_p[2][tid] = pj[2];
    }
    __syncthreads();
    if (tid == 0) {
      const int n = min(256, K - j0);
      for (int k = 0; k < n; ++k) {
        a += s_p[0][k];
        b += s_p[1][k];
        x += s_p[2][k];
      }
    }
    __syncthreads();
  }
  if (tid == 0) {
    dA[h] = (float)a;
    ddt_bias[h] = (float)b;
    if (dD) dD[h] = (float)x;
  }
  if (!dh0) return;
  const int64_t PN = (int64_t)q.P * q.N;
  for (int i = 0; i < q.nseq; ++i) {
    int s0, L;
    span_of(q, i, s0, L);
    if (L > 0) continue;
    const int64_t o = ((int64_t)i * q.H + h) * PN;
    for (int64_t k = tid; k < PN; k += 256) dh0[o + k] = gfirst[o + k];
  }
}

// workgroups for `rows` rows of width W (see row_of)
unsigned row_blocks(int rows, int W) {
  const int rpb = 256 / (W / 4);
  return (unsigned)((rows + rpb - 1) / rpb);
}

int grid_for(int64_t n) {
  const int64_t g = (n + 255) / 256;
  return (int)(g < 8192 ? g : 8192);
}

}  // namespace

hipError_t launch_bwd_gather(const BwdGeo& q, TArg src, int dtype, int R, int W, int rep,
                             int reverse, float* dst, hipStream_t s) {
  const int rows = q.ntok * R;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(k_gather, dim3(row_blocks(rows, W)), dim3(256), 0, s, q, src, dtype, R, W,
                     rep, reverse, dst);
  return hipGetLastError();
}

hipError_t launch_bwd_gate(const BwdGeo& q, TArg dout, int dout_dtype, TArg z, int z_dtype,
                           const float* y, float* dy, float* dy_rev, TArg dz, hipStream_t s) {
  const int rows = q.ntok * q.H;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(k_gate, dim3(row_blocks(rows, q.P)), dim3(256), 0, s, q, dout, dout_dtype,
                     z, z_dtype, y, dy, dy_rev, dz);
  return hipGetLastError();
}

hipError_t launch_bwd_steps(const BwdGeo& q, TArg dt, int dt_dtype, const float* A,
                            const float* dt_bias, int softplus, int clamp, float dt_min,
                            float dt_max, float* delta, float* gd, float* dt_rev, hipStream_t s) {
  const int64_t n = (int64_t)q.ntok * q.H;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_steps, dim3(grid_for(n)), dim3(256), 0, s, q, dt, dt_dtype, A, dt_bias,
                     softplus, clamp, dt_min, dt_max, delta, gd, dt_rev);
  return hipGetLastError();
}

hipError_t launch_bwd_tokens(const BwdGeo& q, TArg x, int x_dtype, const float* D,
                             const float* dy, const float* gx_rev, const float* delta, TArg dx,
                             float* dyx, float* xg, hipStream_t s) {
  const int rows = q.ntok * q.H;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(k_tokens, dim3(row_blocks(rows, q.P)), dim3(256), 0, s, q, x, x_dtype, D,
                     dy, gx_rev, delta, dx, dyx, xg);
  return hipGetLastError();
}

hipError_t launch_bwd_group_sums(const BwdGeo& q, const float* gb_rev, const float* gc,
                                 const float* delta, TArg dB, TArg dC, hipStream_t s) {
  const int rows = q.ntok * q.G;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(k_group_sums, dim3(row_blocks(rows, q.N)), dim3(256), 0, s, q, gb_rev, gc,
                     delta, dB, dC);
  return hipGetLastError();
}

hipError_t launch_bwd_mirror_meta(const BwdGeo& q, int C, int K, int32_t* meta, int32_t* cu_out,
                                 hipStream_t s) {
  hipLaunchKernelGGL(k_mirror_meta, dim3(1), dim3(256), 0, s, q, C, K, meta, cu_out);
  return hipGetLastError();
}

hipError_t launch_bwd_step_grads(const BwdGeo& q, const Geo& gf, const float* CB,
                                 const float* DX, const float* yo_f, const float* yo_r,
                                 const float* xf, const float* dy,
                                 const float* dyx, const float* delta, const float* gd,
                                 const float* A, const float* fwd_st, const float* mir_st,
                                 const float* gfirst, const float* dfinal, const float* xg,
                                 TArg ddt, double* part, float* dA, float* ddt_bias, float* dD,
                                 float* dh0, hipStream_t s) {
  if (gf.K > 0) {
    auto kern = gf.C == 32 ? k_step_dcs<32> : gf.C == 64 ? k_step_dcs<64>
              : gf.C == 128 ? k_step_dcs<128> : k_step_dcs<256>;
    hipLaunchKernelGGL(kern, dim3(gf.K, q.H), dim3(256), 0, s, q, gf, CB, DX, yo_f, yo_r, xf, dy,
                       dyx, delta, gd, A, fwd_st, mir_st, gfirst, dfinal, xg, ddt, part, dh0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_step_heads, dim3(q.H), dim3(256), 0, s, q, gf.K, part, gfirst, dA,
                     ddt_bias, dD, dh0);
  return hipGetLastError();
}

hipError_t launch_bwd_step_heads(const BwdGeo& q, int K, const double* part,
                                 const float* gfirst, float* dA, float* ddt_bias, float* dD,
                                 float* dh0, hipStream_t s) {
  hipLaunchKernelGGL(k_step_heads, dim3(q.H), dim3(256), 0, s, q, K, part, gfirst, dA,
                     ddt_bias, dD, dh0);
  return hipGetLastError();
}

}  // namespace ssd
