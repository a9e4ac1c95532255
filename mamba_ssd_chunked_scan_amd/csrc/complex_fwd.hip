// complex_fwd.hip -- the complex-A SSD forward (Mamba-3-Lite, "SSD Reference").
//
// Per head h the decay is complex, A_h = a_r + i a_i, and the step size real,
// delta_t = softplus(dt_t) (SSD Reference, "_discretise": abar = exp(softplus(dt) A)):
//     h_t = abar_t h_{t-1} + B_t (outer) x_t,     y_t = sum_n C_t[n] h_t[n, :]
// with per-head complex B, C (N), x (P) and no conjugation ("Math: the recurrence
// both functions implement").  The chunkwise form is the page's ("Chunking and the
// discretized log-decay", "Intra-chunk outputs and per-chunk states", "Inter-chunk
// propagation", "Readout"):
//   cs_l       = (sum_{u<=l} delta_u) A            within a chunk (A is constant, so
//                the complex cumsum is the real cumsum of delta times A)
//   state_c    = sum_s exp(cs_last - cs_s) x_s (outer) B_s           (P x N)
//   Hin_{c+1}  = exp(cs_last(c)) Hin_c + state_c                     (decay_chunk, init term)
//   y_l        = sum_{s<=l} exp(cs_l - cs_s) (C_l . B_s) x_s + exp(cs_l) C_l . Hin_c
//
// Three kernels:
//   k_cx_chunk_state  one workgroup per (chunk, head): the chunk's end state from a
//                     zero start, and the chunk's total step sum;
//   k_cx_state_pass   the sequential scan over chunks, in place, two complex state
//                     elements per thread, loads issued eight chunks ahead;
//   k_cx_chunk_scan   one workgroup per (chunk, head): C.B^T, the decay mask, the
//                     intra-chunk product and the carry-in readout, writing the
//                     real part (or the full complex output).
// Unlike the page's kernel, the intra-chunk output never goes to memory: it is formed
// in the same accumulators as the readout of the carried state.
//
// Complex products on the matrix cores: each complex product is four real fp32
// products (re = ar br - ai bi, im = ar bi + ai br), each a v_mfma_f32_16x16x4_f32
// chain.  When only the real part of y is wanted, the two imaginary-part products of
// the output contractions are skipped.  Inputs are fp32 (complex64), so the fp32
// matrix instructions keep the full input precision; accumulation is fp32.
//
// Matrix-core operand placement (16x16x4 fp32): A operand lane L holds row L%16 at
// k-slot L/16; B operand lane L holds column L%16 at k-slot L/16; the accumulator lane
// L holds column L%16, rows 4(L/16) + 0..3.  Which k a (lane group, instruction) pair
// stands for is free as long as both operands agree; it is chosen per contraction so
// that operands load straight from memory or from an accumulator already in registers.
#include "common.hpp"
#include "kernels.hpp"

namespace ssd {
namespace {

constexpr int kCxMaxChunk = 256;

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

// exp(d (ar + i ai)) = e^{d ar} (cos(d ai) + i sin(d ai)).
__device__ __forceinline__ float2 cexp_step(float d, float ar, float ai) {
  const float m = __expf(d * ar);
  float s, c;
  sincosf(d * ai, &s, &c);
  return make_float2(m * c, m * s);
}

__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
  return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}

template <typename T>
__device__ __forceinline__ const T* cx_row(const TArg& a, int b, int t, int h) {
  return reinterpret_cast<const T*>(a.p) + (int64_t)b * a.s0 + (int64_t)t * a.s1 +
         (int64_t)h * a.s2;
}

// Inclusive cumsum of delta = softplus(dt) over the chunk's positions into sd[0..C);
// positions past the chunk's end add 0 (their step is neutral).  Ends with a barrier.
__device__ __forceinline__ void cx_delta_cumsum(const Geo& g, const TArg& dt, int b, int t0,
                                                int len, int h, float* sd) {
  if (threadIdx.x < kWave) {
    float carry = 0.0f;
    for (int base = 0; base < g.C; base += kWave) {
      const int l = base + (int)threadIdx.x;
      float d = 0.0f;
      if (l < len) d = softplus_f32(*cx_row<float>(dt, b, t0 + l, h));
      const float v = wave_inclusive_sum(d) + carry;
      if (l < g.C) sd[l] = v;
      carry = __shfl(v, kWave - 1, kWave);
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------- chunk state

// state[j, h, p, n] = sum_{s < len} w_s x[s, p] B[s, n],  w_s = exp((sd_last - sd_s) A).
// Wave w computes p-tiles w, w + 4, ...; each p-tile holds all NT n-tiles.
// Contraction over tokens: k-slot q of the 4-token step u is token s0 + 4u + q.
template <int NT>
__global__ __launch_bounds__(256) void k_cx_chunk_state(Geo g, TArg x, TArg B, TArg dt,
                                                        const float* A, float* states,
                                                        float* lam) {
  __shared__ float sd[kCxMaxChunk];
  __shared__ float2 w[kCxMaxChunk];
  const int j = blockIdx.x, h = blockIdx.y;
  Chunk ch;
  if (!get_chunk(g, j, ch)) return;  // a packed batch's unused chunk slots
  const int bb = ch.b, t0 = ch.t0, len = ch.len;
  cx_delta_cumsum(g, dt, bb, t0, len, h, sd);
  const float ar = A[2 * h], ai = A[2 * h + 1];
  const float last = sd[len - 1];
  for (int s = threadIdx.x; s < g.C; s += 256)
    w[s] = s < len ? cexp_step(last - sd[s], ar, ai) : make_float2(0.0f, 0.0f);
  if (threadIdx.x == 0) lam[(int64_t)h * g.K + j] = last;
  __syncthreads();

  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int r16 = lane % 16, q = lane / 16;
  float2* out = reinterpret_cast<float2*>(states) + ((int64_t)j * g.H + h) * g.P * g.N;
  for (int pt = wave; pt < g.P / 16; pt += 4) {
    f32x4 are[NT], aim[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) { are[t] = zero4(); aim[t] = zero4(); }
    const int p = pt * 16 + r16;
    // 16 tokens per pass: all their x and B values are requested before the products
    for (int s0 = 0; s0 < len; s0 += 16) {
      float2 xv[4], bv[4][NT];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int s = s0 + 4 * u + q;  // < C: C is a multiple of 16
        const bool sv = s < len;
        const float2* xr = cx_row<float2>(x, bb, t0 + (sv ? s : 0), h);
        const float2* br = cx_row<float2>(B, bb, t0 + (sv ? s : 0), h);
        xv[u] = sv ? xr[p] : make_float2(0.0f, 0.0f);
#pragma unroll
        for (int t = 0; t < NT; ++t) bv[u][t] = sv ? br[t * 16 + r16] : make_float2(0.0f, 0.0f);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float2 ws = w[s0 + 4 * u + q];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const float2 bw = cmul(ws, bv[u][t]);
          are[t] = mfma4(xv[u].x, bw.x, are[t]);
          are[t] = mfma4(-xv[u].y, bw.y, are[t]);
          aim[t] = mfma4(xv[u].x, bw.y, aim[t]);
          aim[t] = mfma4(xv[u].y, bw.x, aim[t]);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        out[(int64_t)(pt * 16 + 4 * q + i) * g.N + t * 16 + r16] =
            make_float2(are[t][i], aim[t][i]);
  }
}

// ---------------------------------------------------------------- state passing

// Hin[j] for every chunk j of (sequence i, head h), in place over the chunk states, and
// the final state; each sequence starts from its initial state (or zero).  Thread:
// complex elements e, e + 1 of the P x N state (one 16-byte word).
__global__ __launch_bounds__(256) void k_cx_state_pass(Geo g, const float* A,
                                                       const float* lam, const float* h0,
                                                       float* states, float* hfinal) {
  __shared__ float2 dec[256];
  const int ih = blockIdx.y;
  const int i = ih / g.H, h = ih - i * g.H;
  int first, last;
  seq_chunks(g, i, first, last);
  const int nch = last - first;
  const int64_t PN = (int64_t)g.P * g.N;
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 2;
  const bool act = e < PN;
  float4 run = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (act && h0) run = *reinterpret_cast<const float4*>(h0 + (ih * PN + e) * 2);
  const float ar = A[2 * h], ai = A[2 * h + 1];
  for (int cb = 0; cb < nch; cb += 256) {
    const int nb = min(256, nch - cb);
    __syncthreads();
    if ((int)threadIdx.x < nb)
      dec[threadIdx.x] = cexp_step(lam[(int64_t)h * g.K + first + cb + threadIdx.x], ar, ai);
    __syncthreads();
    if (!act) continue;
    for (int k = 0; k < nb; k += 8) {
      float4 sv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (k + u < nb)
          sv[u] = *reinterpret_cast<const float4*>(
              states + ((((int64_t)first + cb + k + u) * g.H + h) * PN + e) * 2);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (k + u >= nb) break;
        float4* dst = reinterpret_cast<float4*>(
            states + ((((int64_t)first + cb + k + u) * g.H + h) * PN + e) * 2);
        *dst = run;
        const float2 d = dec[k + u];
        const float2 r0 = cmul(d, make_float2(run.x, run.y));
        const float2 r1 = cmul(d, make_float2(run.z, run.w));
        run = make_float4(r0.x + sv[u].x, r0.y + sv[u].y, r1.x + sv[u].z, r1.y + sv[u].w);
      }
    }
  }
  if (act && hfinal) *reinterpret_cast<float4*>(hfinal + (ih * PN + e) * 2) = run;
}

// ---------------------------------------------------------------- chunk scan

// Output rows of l-tile lt (wave w takes l-tiles w, w + 4, ...), all PT p-tiles:
//   Y_off:  A = exp(cs_l) C[l, n] (row l, k = n), B = Hin[p, n] (column p, k = n);
//           k-slot q of a 16-wide n block is n = 4q + instruction.
//   C.B^T:  computed transposed, CBt[s, l] = sum_n B[s, n] C[l, n], so that the
//           accumulator (column l, rows s = 4q + r) is directly the A operand of
//           Y_diag (row l, k-slot q, instruction r <-> s = 4q + r).
//   Y_diag: B operand x[s, p] for the same s of each (q, r).
// With STAGE the carry-in state (P x N complex) is first copied into LDS
// (dynamic shared memory, rows of N + 2 complex), so that the four waves, each
// reading all of it for its l-tiles' readout, read it from there rather than
// through the caches (chosen when it fits in 64 KB).
template <int PT, bool CPLX, bool STAGE>
__global__ __launch_bounds__(256) void k_cx_chunk_scan(Geo g, TArg x, TArg B, TArg Cm,
                                                       TArg dt, const float* A,
                                                       const float* states, TArg out) {
  __shared__ float sd[kCxMaxChunk];
  __shared__ float2 ecs[kCxMaxChunk];
  extern __shared__ __align__(16) float2 s_hin[];
  const int j = blockIdx.x, h = blockIdx.y;
  Chunk ch;
  if (!get_chunk(g, j, ch)) return;  // a packed batch's unused chunk slots
  const int bb = ch.b, t0 = ch.t0, len = ch.len;
  const float2* hsrc = reinterpret_cast<const float2*>(states) + ((int64_t)j * g.H + h) * g.P * g.N;
  const int HLDc = g.N + 2;  // complex per staged row
  if (STAGE) {
    // issued before the cumsum, whose barrier then also orders these writes
    const int rowv = g.N / 2;  // float4 (two complex) per row
    for (int v = threadIdx.x; v < g.P * rowv; v += 256) {
      const int p = v / rowv, n = (v % rowv) * 2;
      *reinterpret_cast<float4*>(&s_hin[p * HLDc + n]) =
          *reinterpret_cast<const float4*>(hsrc + (int64_t)p * g.N + n);
    }
  }
  cx_delta_cumsum(g, dt, bb, t0, len, h, sd);
  const float ar = A[2 * h], ai = A[2 * h + 1];
  for (int l = threadIdx.x; l < g.C; l += 256) ecs[l] = cexp_step(sd[l], ar, ai);
  __syncthreads();

  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int r16 = lane % 16, q = lane / 16;
  const float2* hin = STAGE ? s_hin : hsrc;
  const int hld = STAGE ? HLDc : g.N;  // complex per row of hin
  const int nkb = g.N / 16;
  for (int lt = wave; lt * 16 < len; lt += 4) {
    f32x4 yre[PT], yim[PT];
#pragma unroll
    for (int t = 0; t < PT; ++t) { yre[t] = zero4(); yim[t] = zero4(); }
    const int lrow = lt * 16 + r16;
    const bool lval = lrow < len;
    const float2* crow = cx_row<float2>(Cm, bb, t0 + (lval ? lrow : 0), h);

    // carry-in readout: exp(cs_l) C_l . Hin
    {
      const float2 el = ecs[lrow];
      for (int kb = 0; kb < nkb; ++kb) {
        const int n0 = kb * 16 + 4 * q;
        float4 c01 = make_float4(0.0f, 0.0f, 0.0f, 0.0f), c23 = c01;
        if (lval) {
          c01 = *reinterpret_cast<const float4*>(crow + n0);
          c23 = *reinterpret_cast<const float4*>(crow + n0 + 2);
        }
        float2 cv[4] = {cmul(el, make_float2(c01.x, c01.y)), cmul(el, make_float2(c01.z, c01.w)),
                        cmul(el, make_float2(c23.x, c23.y)), cmul(el, make_float2(c23.z, c23.w))};
#pragma unroll
        for (int t = 0; t < PT; ++t) {
          const float2* hr = hin + (t * 16 + r16) * hld + n0;
          const float4 h01 = *reinterpret_cast<const float4*>(hr);
          const float4 h23 = *reinterpret_cast<const float4*>(hr + 2);
          const float2 hv[4] = {make_float2(h01.x, h01.y), make_float2(h01.z, h01.w),
                                make_float2(h23.x, h23.y), make_float2(h23.z, h23.w)};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            yre[t] = mfma4(cv[i].x, hv[i].x, yre[t]);
            yre[t] = mfma4(-cv[i].y, hv[i].y, yre[t]);
            if (CPLX) {
              yim[t] = mfma4(cv[i].x, hv[i].y, yim[t]);
              yim[t] = mfma4(cv[i].y, hv[i].x, yim[t]);
            }
          }
        }
      }
    }

    // intra-chunk part, one 16-token source tile at a time (s-tiles st <= lt)
    for (int st = 0; st <= lt; ++st) {
      const int srow = st * 16 + r16;
      const bool sval = srow < len;
      const float2* brow = cx_row<float2>(B, bb, t0 + (sval ? srow : 0), h);
      // this source tile's x rows (s = 16 st + 4q + r), requested before the C.B^T
      // products so that they have arrived when Y_diag needs them
      float2 xv[4][PT];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int s = st * 16 + 4 * q + r;
        const bool xs = s < len;
        const float2* xrow = cx_row<float2>(x, bb, t0 + (xs ? s : 0), h);
#pragma unroll
        for (int t = 0; t < PT; ++t)
          xv[r][t] = xs ? xrow[t * 16 + r16] : make_float2(0.0f, 0.0f);
      }
      f32x4 cbr = zero4(), cbi = zero4();
      for (int kb = 0; kb < nkb; ++kb) {
        const int n0 = kb * 16 + 4 * q;
        float4 b01 = make_float4(0.0f, 0.0f, 0.0f, 0.0f), b23 = b01, c01 = b01, c23 = b01;
        if (sval) {
          b01 = *reinterpret_cast<const float4*>(brow + n0);
          b23 = *reinterpret_cast<const float4*>(brow + n0 + 2);
        }
        if (lval) {
          c01 = *reinterpret_cast<const float4*>(crow + n0);
          c23 = *reinterpret_cast<const float4*>(crow + n0 + 2);
        }
        const float br[4] = {b01.x, b01.z, b23.x, b23.z}, bi[4] = {b01.y, b01.w, b23.y, b23.w};
        const float cr[4] = {c01.x, c01.z, c23.x, c23.z}, ci[4] = {c01.y, c01.w, c23.y, c23.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          cbr = mfma4(br[i], cr[i], cbr);
          cbr = mfma4(-bi[i], ci[i], cbr);
          cbi = mfma4(br[i], ci[i], cbi);
          cbi = mfma4(bi[i], cr[i], cbi);
        }
      }
      // decay mask: M^T[s, l] = CBt[s, l] exp(cs_l - cs_s) for s <= l, else 0
      float mr[4], mi[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int s = st * 16 + 4 * q + r;
        if (s <= lrow && s < len && lval) {
          const float2 f = cexp_step(sd[lrow] - sd[s], ar, ai);
          const float2 m = cmul(make_float2(cbr[r], cbi[r]), f);
          mr[r] = m.x;
          mi[r] = m.y;
        } else {
          mr[r] = 0.0f;
          mi[r] = 0.0f;
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int t = 0; t < PT; ++t) {
          yre[t] = mfma4(mr[r], xv[r][t].x, yre[t]);
          yre[t] = mfma4(-mi[r], xv[r][t].y, yre[t]);
          if (CPLX) {
            yim[t] = mfma4(mr[r], xv[r][t].y, yim[t]);
            yim[t] = mfma4(mi[r], xv[r][t].x, yim[t]);
          }
        }
    }

    // lane holds y[l = 16 lt + 4q + i, p = 16 t + r16]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int l = lt * 16 + 4 * q + i;
      if (l >= len) continue;
      if (CPLX) {
        float2* orow = reinterpret_cast<float2*>(const_cast<void*>(out.p)) +
                       (int64_t)bb * out.s0 + (int64_t)(t0 + l) * out.s1 + (int64_t)h * out.s2;
#pragma unroll
        for (int t = 0; t < PT; ++t) orow[t * 16 + r16] = make_float2(yre[t][i], yim[t][i]);
      } else {
        float* orow = reinterpret_cast<float*>(const_cast<void*>(out.p)) +
                      (int64_t)bb * out.s0 + (int64_t)(t0 + l) * out.s1 + (int64_t)h * out.s2;
#pragma unroll
        for (int t = 0; t < PT; ++t) orow[t * 16 + r16] = yre[t][i];
      }
    }
  }
}

template <int NT>
hipError_t launch_state_nt(const Geo& g, TArg x, TArg B, TArg dt, const float* A,
                           float* states, float* lam, hipStream_t s) {
  dim3 grid(g.K, g.H);
  hipLaunchKernelGGL(k_cx_chunk_state<NT>, grid, dim3(256), 0, s, g, x, B, dt, A, states, lam);
  return hipGetLastError();
}

template <int PT>
hipError_t launch_scan_pt(const Geo& g, TArg x, TArg B, TArg Cm, TArg dt, const float* A,
                          const float* states, TArg out, int cplx, hipStream_t s) {
  dim3 grid(g.K, g.H);
  const size_t hbytes = (size_t)g.P * (g.N + 2) * sizeof(float2);
  if (hbytes <= 64 * 1024) {
    if (cplx)
      hipLaunchKernelGGL((k_cx_chunk_scan<PT, true, true>), grid, dim3(256), hbytes, s, g, x, B,
                         Cm, dt, A, states, out);
    else
      hipLaunchKernelGGL((k_cx_chunk_scan<PT, false, true>), grid, dim3(256), hbytes, s, g, x, B,
                         Cm, dt, A, states, out);
  } else if (cplx) {
    hipLaunchKernelGGL((k_cx_chunk_scan<PT, true, false>), grid, dim3(256), 0, s, g, x, B, Cm, dt,
                       A, states, out);
  } else {
    hipLaunchKernelGGL((k_cx_chunk_scan<PT, false, false>), grid, dim3(256), 0, s, g, x, B, Cm,
                       dt, A, states, out);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_cx_chunk_state(const Geo& g, TArg x, TArg B, TArg dt, const float* A,
                                 float* states, float* lam, hipStream_t s) {
  if (g.K == 0) return hipSuccess;
  switch (g.N / 16) {
    case 1: return launch_state_nt<1>(g, x, B, dt, A, states, lam, s);
    case 2: return launch_state_nt<2>(g, x, B, dt, A, states, lam, s);
    case 3: return launch_state_nt<3>(g, x, B, dt, A, states, lam, s);
    case 4: return launch_state_nt<4>(g, x, B, dt, A, states, lam, s);
    case 5: return launch_state_nt<5>(g, x, B, dt, A, states, lam, s);
    case 6: return launch_state_nt<6>(g, x, B, dt, A, states, lam, s);
    case 7: return launch_state_nt<7>(g, x, B, dt, A, states, lam, s);
    default: return launch_state_nt<8>(g, x, B, dt, A, states, lam, s);
  }
}

hipError_t launch_cx_state_pass(const Geo& g, const float* A, const float* lam,
                                const float* h0, float* states, float* hfinal, hipStream_t s) {
  const int64_t PN = (int64_t)g.P * g.N;
  dim3 grid((unsigned)((PN + 511) / 512), g.nseq * g.H);
  hipLaunchKernelGGL(k_cx_state_pass, grid, dim3(256), 0, s, g, A, lam, h0, states, hfinal);
  return hipGetLastError();
}

hipError_t launch_cx_chunk_scan(const Geo& g, TArg x, TArg B, TArg Cm, TArg dt,
                                const float* A, const float* states, TArg out, int out_complex,
                                hipStream_t s) {
  if (g.K == 0) return hipSuccess;
  switch (g.P / 16) {
    case 1: return launch_scan_pt<1>(g, x, B, Cm, dt, A, states, out, out_complex, s);
    case 2: return launch_scan_pt<2>(g, x, B, Cm, dt, A, states, out, out_complex, s);
    case 3: return launch_scan_pt<3>(g, x, B, Cm, dt, A, states, out, out_complex, s);
    case 4: return launch_scan_pt<4>(g, x, B, Cm, dt, A, states, out, out_complex, s);
    case 5: return launch_scan_pt<5>(g, x, B, Cm, dt, A, states, out, out_complex, s);
    case 6: return launch_scan_pt<6>(g, x, B, Cm, dt, A, states, out, out_complex, s);
    case 7: return launch_scan_pt<7>(g, x, B, Cm, dt, A, states, out, out_complex, s);
    default: return launch_scan_pt<8>(g, x, B, Cm, dt, A, states, out, out_complex, s);
  }
}

}  // namespace ssd
