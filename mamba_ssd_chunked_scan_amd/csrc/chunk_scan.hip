// chunk_scan.hip -- the standalone chunk-scan kernels.  The bf16 body and the
// LDS helpers live in stage_scan.hpp; fp32 inputs use the generic kernel below,
// with fp32 matrix instructions, or (SP) every operand split into bf16 hi + lo
// and three bf16 matrix instructions per product.
#include <type_traits>

#include "kernels.hpp"
#include "stage_scan.hpp"

namespace ssd {

// F: the step size scales the input term (dtc is read), compiled in only then.
// st_trans: the carry-in states are stored transposed, (K, H, N, P) -- the
// chunk states of a scan whose head and state dims are this one's swapped.
// x_div: head h reads row h / x_div of x (x shared by groups of heads).
template <typename T, typename ST, typename TO, bool F, bool SP>
__global__ __launch_bounds__(256) void k_chunk_scan_generic(Geo g, const float* __restrict__ CB, TArg x,
                                                    TArg Cm, const float* __restrict__ cs,
                                                    const float* __restrict__ dtc,
                                                    const ST* __restrict__ states,
                                                    const float* __restrict__ D, TArg z,
                                                    TArg out, float* __restrict__ yoff,
                                                    int st_trans, int x_div) {
  using Pr = Prec<T>;
  using HL = typename std::conditional<SP, HinLds<bf16, ST>, HinLds<T, ST>>::type;
  extern __shared__ __align__(16) char smem[];
  const int j = blockIdx.x, h = blockIdx.y, p0 = blockIdx.z * 64;
  Chunk c;
  if (!get_chunk(g, j, c)) return;
  const int C = g.C, N = g.N, P = g.P;
  const int grp = h / g.hpg;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int r16 = lane % 16, q = lane / 16;
  const ScanLayout lay = SP ? scan_layout_split<ST>(C, N) : scan_layout<T, ST>(C, N);
  float* s_cs = reinterpret_cast<float*>(smem);
  float* s_f = s_cs + C;
  T* s_xt = reinterpret_cast<T*>(smem + lay.off_x);
  bf16* s_xh = reinterpret_cast<bf16*>(smem + lay.off_x);  // (SP: hi and lo planes)
  bf16* s_xl = s_xh + 64 * lay.ldx;
  char* s_h = smem + lay.off_h;
  float* s_y = reinterpret_cast<float*>(smem + lay.off_h);

  // ---- stage cumsum, x^T and the carry-in state
  const float* csr = cs + ((int64_t)j * g.H + h) * C;
  const float* dtr = dtc ? dtc + ((int64_t)j * g.H + h) * C : nullptr;
  for (int l = tid; l < C; l += 256) {
    s_cs[l] = csr[l];
    s_f[l] = dtr ? dtr[l] : 1.0f;
  }
  const int pw = min(64, P - p0);           // p columns in this block (multiple of 16)
  const int nvec_x = C * 8;                 // C rows x 8 vectors of 8 p
  for (int v = tid; v < nvec_x; v += 256) {
    const int s = v / 8, pp = (v % 8) * 8;
    f32x8 val = {0, 0, 0, 0, 0, 0, 0, 0};
    if (s < c.len && pp < pw)
      val = Vec8<T>::load(row_ptr<T>(x, c.b, c.t0 + s, h / x_div) + p0 + pp);
    if constexpr (SP) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bf16 hv = (bf16)val[i];
        s_xh[(pp + i) * lay.ldx + s] = hv;
        s_xl[(pp + i) * lay.ldx + s] = (bf16)(val[i] - (float)hv);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) s_xt[(pp + i) * lay.ldx + s] = from_f32<T>(val[i]);
    }
  }
  const ST* hsrc = states + ((int64_t)j * g.H + h) * P * N;
  if (!st_trans) {
    const int nvec_h = 64 * (N / 8);
    for (int v = tid; v < nvec_h; v += 256) {
      const int pr = v / (N / 8), n = (v % (N / 8)) * 8;
      f32x8 val = {0, 0, 0, 0, 0, 0, 0, 0};
      if (pr < pw) val = StLoad<ST>::load(hsrc + (int64_t)(p0 + pr) * N + n);
      HL::stage(s_h, hsrc, N, pr, n, val);
    }
  } else {
    // row n of the stored state holds this block's 64 p columns contiguously
    for (int v = tid; v < N * 8; v += 256) {
      const int n = v / 8, pp = (v % 8) * 8;
      f32x8 val = {0, 0, 0, 0, 0, 0, 0, 0};
      if (pp < pw) val = StLoad<ST>::load(hsrc + (int64_t)n * P + p0 + pp);
#pragma unroll
      for (int i = 0; i < 8; ++i) HL::stage1(s_h, N, pp + i, n, val[i]);
    }
  }
  __syncthreads();

  // ---- matrix-core phase
  const int nlt = C / 16;
  const int npt = pw / 16;
  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = zero4();

  const float* cbm = CB + ((int64_t)j * g.G + grp) * C * C;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int grp8 = u / 2;
    const int lt = grp8 * 8 + ((u & 1) ? 7 - wave : wave);
    if (lt >= nlt) continue;
    const int lrow = lt * 16 + r16;               // A-operand row of this lane
    const bool lok = lrow < c.len;
    // Y_off = C_l . Hin^T over n
    const T* crow = row_ptr<T>(Cm, c.b, c.t0 + (lok ? lrow : 0), grp);
    // each k-block's C fragment is loaded one block ahead (the address clamped
    // into N; past the end it re-reads the last block, unused)
    typename Pr::Exact anext = Pr::load_exact(crow + min(q * 8, N - 8));
    for (int k0 = 0; k0 < N; k0 += 32) {
      // lanes whose k-quad lies past N (N % 32 == 16) contribute zeros on both
      // sides; the matrix instruction itself always runs wave-wide
      const int k = k0 + q * 8;
      const bool kok = k < N;
      const typename Pr::Exact araw = anext;
      anext = Pr::load_exact(crow + min(k + 32, N - 8));
      const typename Pr::Exact a = (lok && kok) ? araw : Pr::zero_exact();
      auto as = [&] {
        if constexpr (SP) return split_f32x8(a.v);
        else return a;
      }();
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        if (pt < npt) {
          auto b = HL::frag(s_h, N, pt * 16 + r16, kok ? k : 0);
          mma(acc[u][pt], as, b);
        }
      }
    }
    // scale rows by exp(cs[l])
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = fast_exp(s_cs[lt * 16 + q * 4 + i]);
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) acc[u][pt][i] *= e;
    }
    // optionally keep Y_off on its own, (tokens, H, P) fp32 on the packed axis
    if (yoff) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int l = lt * 16 + q * 4 + i;
        if (l >= c.len) continue;
        float* yr = yoff + ((int64_t)(c.b * g.T + c.t0 + l) * g.H + h) * P + p0;
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
          if (pt < npt) yr[pt * 16 + r16] = acc[u][pt][i];
      }
    }
    // Y_diag = (L o CB) x over s <= l
    const float csl = s_cs[min(lrow, C - 1)];
    const int kend = lt * 16 + 16;                 // s < kend covers the diagonal tile
    // the C.B^T row fragment one block ahead, as above (rows past the chunk
    // read a row of the tile and are discarded)
    const float* cbr = cbm + (int64_t)min(lrow, C - 1) * C;
    f32x8 cbnext = Vec8<float>::load(cbr + q * 8);
    for (int k0 = 0; k0 < kend; k0 += 32) {
      const int s0 = k0 + q * 8;
      const f32x8 cb = cbnext;
      cbnext = Vec8<float>::load(cbr + min(s0 + 32, C - 8));
      f32x8 m;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int s = s0 + e;
        const bool keep = lok && (s <= lrow) && (s < c.len);
        m[e] = keep ? fast_exp(csl - s_cs[s]) * cb[e] * (F ? s_f[s] : 1.0f) : 0.0f;
      }
      if constexpr (SP) {
        const FragSplit mf = split_f32x8(m);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          if (pt < npt) {
            FragSplit xb;
            xb.hi = *reinterpret_cast<const bf16x8*>(&s_xh[(pt * 16 + r16) * lay.ldx + s0]);
            xb.lo = *reinterpret_cast<const bf16x8*>(&s_xl[(pt * 16 + r16) * lay.ldx + s0]);
            mma(acc[u][pt], mf, xb);
          }
        }
      } else {
        const auto mf = Pr::derive(m);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          if (pt < npt) {
            typename Pr::Exact xb = Pr::load_exact(s_xt + (pt * 16 + r16) * lay.ldx + s0);
            mma(acc[u][pt], mf, xb);
          }
        }
      }
    }
  }
  __syncthreads();  // everyone is done with x^T and the state; reuse the state area for y

#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int lt = (u / 2) * 8 + ((u & 1) ? 7 - wave : wave);
    if (lt >= nlt) continue;
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      if (pt >= npt) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        s_y[(lt * 16 + q * 4 + i) * lay.ldy + pt * 16 + r16] = acc[u][pt][i];
    }
  }
  __syncthreads();

  // ---- epilogue: D skip, SiLU gate, store; coalesced 8-element rows
  const float Dh = D ? D[h] : 0.0f;
  const int vpr = pw / 8;  // vectors per row
  for (int v = tid; v < c.len * vpr; v += 256) {
    const int l = v / vpr, pp = (v % vpr) * 8;
    f32x8 y = Vec8<float>::load(s_y + l * lay.ldy + pp);
    const int t = c.t0 + l;
    if (D) {
      const f32x8 xv = Vec8<T>::load(row_ptr<T>(x, c.b, t, h) + p0 + pp);
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] += Dh * xv[i];
    }
    if (z.p) {
      const f32x8 zv = Vec8<T>::load(row_ptr<T>(z, c.b, t, h) + p0 + pp);
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] *= silu(zv[i]);
    }
    Vec8<TO>::store(row_ptr_mut<TO>(out, c.b, t, h) + p0 + pp, y);
  }
}

template <typename ST, typename TO, int C, bool F>
__global__ __launch_bounds__(256, C <= 128 ? 3 : 2) void k_chunk_scan_bf16(Geo g, const float* __restrict__ CB,
                                                         TArg x, TArg Cm,
                                                         const float* __restrict__ cs,
                                                         const float* __restrict__ dtc,
                                                         const ST* __restrict__ states,
                                                         const float* __restrict__ D, TArg z,
                                                         TArg out, float* __restrict__ yoff) {
  extern __shared__ __align__(16) char smem[];
  chunk_scan_block<ST, TO, C, F>(g, CB, x, Cm, cs, dtc, states, D, z, out, yoff, blockIdx.x,
                                 blockIdx.y, blockIdx.z, smem);
}

template <typename ST, typename TO, int C, bool F>
static hipError_t launch_scan_bf16_c(const Geo& g, const float* CB, TArg x, TArg Cm,
                                     const float* cs, const float* dtc, const ST* st,
                                     const float* D, TArg z, TArg out, float* yoff,
                                     hipStream_t s) {
  const ScanLayout lay = scan_layout_bf16<ST>(C, g.N);
  auto kern = k_chunk_scan_bf16<ST, TO, C, F>;
  if (lay.bytes > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lay.bytes);
    if (e != hipSuccess) return e;
  }
  dim3 grid(g.K, g.H, (g.P + 63) / 64);
  hipLaunchKernelGGL(kern, grid, dim3(256), lay.bytes, s, g, CB, x, Cm, cs, dtc, st, D, z, out,
                     yoff);
  return hipGetLastError();
}

template <typename ST, typename TO, bool F>
static hipError_t launch_scan_bf16_f(const Geo& g, const float* CB, TArg x, TArg Cm,
                                     const float* cs, const float* dtc, const void* states,
                                     const float* D, TArg z, TArg out, float* yoff,
                                     hipStream_t s) {
  const ST* st = (const ST*)states;
  switch (g.C) {
    case 32: return launch_scan_bf16_c<ST, TO, 32, F>(g, CB, x, Cm, cs, dtc, st, D, z, out, yoff, s);
    case 64: return launch_scan_bf16_c<ST, TO, 64, F>(g, CB, x, Cm, cs, dtc, st, D, z, out, yoff, s);
    case 128: return launch_scan_bf16_c<ST, TO, 128, F>(g, CB, x, Cm, cs, dtc, st, D, z, out, yoff, s);
    default: return launch_scan_bf16_c<ST, TO, 256, F>(g, CB, x, Cm, cs, dtc, st, D, z, out, yoff, s);
  }
}

template <typename ST, typename TO>
static hipError_t launch_scan_bf16(const Geo& g, const float* CB, TArg x, TArg C, const float* cs,
                                   const float* dtc, const void* states, const float* D, TArg z,
                                   TArg out, float* yoff, hipStream_t s) {
  return dtc ? launch_scan_bf16_f<ST, TO, true>(g, CB, x, C, cs, dtc, states, D, z, out, yoff, s)
             : launch_scan_bf16_f<ST, TO, false>(g, CB, x, C, cs, dtc, states, D, z, out, yoff,
                                                 s);
}

template <typename T, typename ST, typename TO, bool F, bool SP>
static hipError_t launch_scan_tf(const Geo& g, const float* CB, TArg x, TArg C, const float* cs,
                                 const float* dtc, const void* states, const float* D, TArg z,
                                 TArg out, float* yoff, int st_trans, int x_div, hipStream_t s) {
  const ScanLayout lay = SP ? scan_layout_split<ST>(g.C, g.N) : scan_layout<T, ST>(g.C, g.N);
  auto kern = k_chunk_scan_generic<T, ST, TO, F, SP>;
  if (lay.bytes > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lay.bytes);
    if (e != hipSuccess) return e;
  }
  dim3 grid(g.K, g.H, (g.P + 63) / 64);
  hipLaunchKernelGGL(kern, grid, dim3(256), lay.bytes, s, g, CB, x, C, cs, dtc, (const ST*)states,
                     D, z, out, yoff, st_trans, x_div);
  return hipGetLastError();
}

template <typename T, typename ST, typename TO>
static hipError_t launch_scan_t(const Geo& g, const float* CB, TArg x, TArg C, const float* cs,
                                const float* dtc, const void* states, const float* D, TArg z,
                                TArg out, float* yoff, int st_trans, int x_div, int split,
                                hipStream_t s) {
  if (split)
    return dtc ? launch_scan_tf<T, ST, TO, true, true>(g, CB, x, C, cs, dtc, states, D, z, out,
                                                       yoff, st_trans, x_div, s)
               : launch_scan_tf<T, ST, TO, false, true>(g, CB, x, C, cs, dtc, states, D, z, out,
                                                        yoff, st_trans, x_div, s);
  return dtc ? launch_scan_tf<T, ST, TO, true, false>(g, CB, x, C, cs, dtc, states, D, z, out,
                                                      yoff, st_trans, x_div, s)
             : launch_scan_tf<T, ST, TO, false, false>(g, CB, x, C, cs, dtc, states, D, z, out,
                                                       yoff, st_trans, x_div, s);
}

hipError_t launch_chunk_scan(const Geo& g, const float* CB, TArg x, TArg C, int in_dtype,
                             const float* cs, const float* dtc, const void* states, int st_dtype,
                             const float* D, TArg z, TArg out, int out_dtype, hipStream_t s,
                             float* yoff, int st_trans, int x_div, int split) {
  if (g.K == 0) return hipSuccess;
  const bool ib = in_dtype == DT_BF16, sb = st_dtype == DT_BF16, ob = out_dtype == DT_BF16;
  if (ib) {
    // only the fp32 kernel reads transposed states, shares x between heads or
    // splits fp32 operands
    if (st_trans || x_div != 1 || split) return hipErrorInvalidValue;
    if (sb) return ob ? launch_scan_bf16<bf16, bf16>(g, CB, x, C, cs, dtc, states, D, z, out, yoff, s)
                      : launch_scan_bf16<bf16, float>(g, CB, x, C, cs, dtc, states, D, z, out, yoff, s);
    return ob ? launch_scan_bf16<float, bf16>(g, CB, x, C, cs, dtc, states, D, z, out, yoff, s)
              : launch_scan_bf16<float, float>(g, CB, x, C, cs, dtc, states, D, z, out, yoff, s);
  }
  if (sb) return ob ? launch_scan_t<float, bf16, bf16>(g, CB, x, C, cs, dtc, states, D, z, out, yoff, st_trans, x_div, split, s)
                    : launch_scan_t<float, bf16, float>(g, CB, x, C, cs, dtc, states, D, z, out, yoff, st_trans, x_div, split, s);
  return ob ? launch_scan_t<float, float, bf16>(g, CB, x, C, cs, dtc, states, D, z, out, yoff, st_trans, x_div, split, s)
            : launch_scan_t<float, float, float>(g, CB, x, C, cs, dtc, states, D, z, out, yoff, st_trans, x_div, split, s);
}

}  // namespace ssd
