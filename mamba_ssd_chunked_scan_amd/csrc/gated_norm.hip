// gated_norm.hip -- the gated RMSNorm that follows the scan in the Mamba-2 mixer
// (mamba PR 1012, "Summary" and "Measurements": the gated-LayerNorm and its backward,
// layer_norm_bwd).  The pages do not write its formula; the one computed is Mamba-2's
// gated RMSNorm with the gate applied first, over contiguous groups of gs channels of
// the flattened (H, P) axis of every token:
//     g = y silu(z),   r = 1 / sqrt(mean_group(g^2) + eps),   out = g r weight
// Gradient of sum(dout out), with xhat = g r:
//     dg = r (dout w - xhat mean_group(dout w xhat)),  dy = dg silu(z),
//     dz = dg y sigma(z) (1 + z (1 - sigma(z))),        dweight = sum_tokens dout xhat
//
// Both passes are HBM streams (each input read once, each output written once).  A lane
// holds 8 consecutive channels of a 512-channel strip, so every access is a 16-byte
// (bf16) or 32-byte (fp32) vector; groups of up to 512 channels reduce over their lanes
// within the wave, wider groups take a statistics pass first.  The weight gradient is
// reduced deterministically: per 64-token tile into a partial row (fixed order), then
// over tiles by a second kernel (fixed order, fp64).
#include "common.hpp"
#include "kernels.hpp"

namespace ssd {
namespace {

constexpr int kNormTile = 64;   // tokens per weight-gradient partial row
constexpr int kStrip = 512;     // channels per wave-wide strip (64 lanes x 8)

// Sum over aligned segments of `seg` lanes (seg a power of two, 1..64).
__device__ __forceinline__ float seg_sum(float v, int seg) {
  for (int d = seg >> 1; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
  return v;
}

template <typename T>
__device__ __forceinline__ const T* norm_ptr(const NormGeo& g, const TArg& a, int tok, int c) {
  const int b = tok / g.T, t = tok - b * g.T, h = c / g.P, p = c - h * g.P;
  return reinterpret_cast<const T*>(a.p) + (int64_t)b * a.s0 + (int64_t)t * a.s1 +
         (int64_t)h * a.s2 + p;
}

template <typename T>
__device__ __forceinline__ f32x8 load8(const NormGeo& g, const TArg& a, int tok, int c) {
  return Vec8<T>::load(norm_ptr<T>(g, a, tok, c));
}

template <typename T>
__device__ __forceinline__ void store8(const NormGeo& g, const TArg& a, int tok, int c, f32x8 v) {
  Vec8<T>::store(const_cast<T*>(norm_ptr<T>(g, a, tok, c)), v);
}

__device__ __forceinline__ float sigmoid(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// g = y silu(z) for 8 channels (z absent: g = y)
template <typename TI>
__device__ __forceinline__ f32x8 gate8(const NormGeo& g, const TArg& y, const TArg& z, int tok,
                                       int c, f32x8& yv, f32x8& zv) {
  yv = load8<TI>(g, y, tok, c);
  f32x8 gv = yv;
  if (z.p) {
    zv = load8<TI>(g, z, tok, c);
#pragma unroll
    for (int i = 0; i < 8; ++i) gv[i] = yv[i] * zv[i] * sigmoid(zv[i]);
  }
  return gv;
}

// Forward.  gs <= 512: one wave per (token, 512-channel strip), every group inside the
// strip reduced over its gs / 8 lanes.  gs > 512 (a multiple of 512): one wave per
// (token, group), a first loop over the group's strips for the mean square and a second
// (reloading, from cache) for the output.
template <typename TI, typename TO>
__global__ __launch_bounds__(256) void k_norm_fwd(NormGeo g, TArg y, TArg z, const float* w,
                                                  TArg out, float* rstd) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int W = g.H * g.P;
  const int item = blockIdx.x * 4 + wave;
  if (g.gs <= kStrip) {
    const int nstrip = (W + kStrip - 1) / kStrip;
    if (item >= g.ntok * nstrip) return;
    const int tok = item / nstrip, c = (item - tok * nstrip) * kStrip + lane * 8;
    const bool act = c < W;
    f32x8 yv, zv, gv;
    float ss = 0.0f;
    if (act) {
      gv = gate8<TI>(g, y, z, tok, c, yv, zv);
#pragma unroll
      for (int i = 0; i < 8; ++i) ss += gv[i] * gv[i];
    }
    ss = seg_sum(ss, g.gs / 8);
    const float r = 1.0f / sqrtf(ss / (float)g.gs + g.eps);
    if (act) {
      const f32x8 wv = Vec8<float>::load(w + c);
      f32x8 ov;
#pragma unroll
      for (int i = 0; i < 8; ++i) ov[i] = gv[i] * r * wv[i];
      store8<TO>(g, out, tok, c, ov);
      if (rstd && c % g.gs == 0) rstd[(int64_t)tok * (W / g.gs) + c / g.gs] = r;
    }
    return;
  }
  const int ngr = W / g.gs;
  if (item >= g.ntok * ngr) return;
  const int tok = item / ngr, c0 = (item - tok * ngr) * g.gs + lane * 8;
  float ss = 0.0f;
  for (int o = 0; o < g.gs; o += kStrip) {
    f32x8 yv, zv;
    const f32x8 gv = gate8<TI>(g, y, z, tok, c0 + o, yv, zv);
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += gv[i] * gv[i];
  }
  ss = seg_sum(ss, kWave);
  const float r = 1.0f / sqrtf(ss / (float)g.gs + g.eps);
  for (int o = 0; o < g.gs; o += kStrip) {
    f32x8 yv, zv;
    const f32x8 gv = gate8<TI>(g, y, z, tok, c0 + o, yv, zv);
    const f32x8 wv = Vec8<float>::load(w + c0 + o);
    f32x8 ov;
#pragma unroll
    for (int i = 0; i < 8; ++i) ov[i] = gv[i] * r * wv[i];
    store8<TO>(g, out, tok, c0 + o, ov);
  }
  if (rstd && lane == 0) rstd[item] = r;
}

// The normalisation of the forward with the gated RMSNorm fused in: the scan's
// epilogue has written g = y silu(z) to `out` and, per token and 64-channel
// block, sum(g^2) (from the fp32 g) to psum; this pass scales `out` in place,
// out = g r weight with r = 1 / sqrt(sum over the group's blocks / gs + eps).
// One wave per token: the group factors first (into LDS), then the token's
// channels in 16-byte (bf16) or 32-byte (fp32) vectors.
template <typename TO>
__global__ __launch_bounds__(256) void k_norm_finish(NormGeo g, const float* psum,
                                                     const float* w, TArg out, float* rstd) {
  __shared__ float s_r[4][kNormFinishGroups];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int tok = blockIdx.x * 4 + wave;
  if (tok >= g.ntok) return;
  const int W = g.H * g.P, U = W / 64, gu = g.gs / 64, ngr = W / g.gs;
  const float* ps = psum + (int64_t)tok * U;
  if (gu >= kWave) {
    // wide groups: the wave sums each group's blocks
    for (int j = 0; j < ngr; ++j) {
      float ss = 0.0f;
      for (int k = lane; k < gu; k += kWave) ss += ps[j * gu + k];
      ss = seg_sum(ss, kWave);
      const float r = 1.0f / sqrtf(ss / (float)g.gs + g.eps);
      if (lane == 0) {
        s_r[wave][j] = r;
        if (rstd) rstd[(int64_t)tok * ngr + j] = r;
      }
    }
  } else {
    for (int j = lane; j < ngr; j += kWave) {
      float ss = 0.0f;
      for (int k = 0; k < gu; ++k) ss += ps[j * gu + k];
      const float r = 1.0f / sqrtf(ss / (float)g.gs + g.eps);
      s_r[wave][j] = r;
      if (rstd) rstd[(int64_t)tok * ngr + j] = r;
    }
  }
  // (a wave's LDS accesses are performed in order: its reads below see its
  // writes above)
  for (int c = lane * 8; c < W; c += kStrip) {
    const float r = s_r[wave][c / g.gs];
    const f32x8 gv = load8<TO>(g, out, tok, c);
    const f32x8 wv = Vec8<float>::load(w + c);
    f32x8 ov;
#pragma unroll
    for (int i = 0; i < 8; ++i) ov[i] = gv[i] * r * wv[i];
    store8<TO>(g, out, tok, c, ov);
  }
}

// Backward statistics of groups wider than a strip: per (token, group), r and
// mean(dxhat xhat) = r mean(dout w g).  One wave per (token, group).
template <typename TI>
__global__ __launch_bounds__(256) void k_norm_stats(NormGeo g, TArg y, TArg z, const float* w,
                                                    TArg dout, float2* stats) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int ngr = g.H * g.P / g.gs;
  const int item = blockIdx.x * 4 + wave;
  if (item >= g.ntok * ngr) return;
  const int tok = item / ngr, c0 = (item - tok * ngr) * g.gs + lane * 8;
  float ss = 0.0f, dg = 0.0f;
  for (int o = 0; o < g.gs; o += kStrip) {
    f32x8 yv, zv;
    const f32x8 gv = gate8<TI>(g, y, z, tok, c0 + o, yv, zv);
    const f32x8 dv = load8<TI>(g, dout, tok, c0 + o);
    const f32x8 wv = Vec8<float>::load(w + c0 + o);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ss += gv[i] * gv[i];
      dg += dv[i] * wv[i] * gv[i];
    }
  }
  ss = seg_sum(ss, kWave);
  dg = seg_sum(dg, kWave);
  const float r = 1.0f / sqrtf(ss / (float)g.gs + g.eps);
  if (lane == 0) stats[item] = make_float2(r, r * dg / (float)g.gs);
}

// Backward.  One workgroup per (64-token tile, 512-channel strip); wave w takes tokens
// w, w + 4, ... of the tile; lane: 8 channels.  Groups within the strip reduce over
// their lanes (gs <= 512) or read the statistics pass (gs > 512).  Weight-gradient
// partial rows: part[tile][channel].
template <typename TI>
__global__ __launch_bounds__(256) void k_norm_bwd(NormGeo g, TArg y, TArg z, const float* w,
                                                  TArg dout, const float2* stats, TArg dy,
                                                  TArg dz, float* part) {
  __shared__ float red[4][kStrip];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int W = g.H * g.P;
  const int tile = blockIdx.x, c = blockIdx.y * kStrip + lane * 8;
  const bool act = c < W;
  f32x8 dwa;
#pragma unroll
  for (int i = 0; i < 8; ++i) dwa[i] = 0.0f;
  f32x8 wv;
  if (act) wv = Vec8<float>::load(w + c);
  const int tend = min(g.ntok, (tile + 1) * kNormTile);
  for (int tok = tile * kNormTile + wave; tok < tend; tok += 4) {
    f32x8 yv, zv, gv, dv;
    float ss = 0.0f, dgs = 0.0f;
    if (act) {
      gv = gate8<TI>(g, y, z, tok, c, yv, zv);
      dv = load8<TI>(g, dout, tok, c);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ss += gv[i] * gv[i];
        dgs += dv[i] * wv[i] * gv[i];
      }
    }
    float r, sd;
    if (g.gs <= kStrip) {
      ss = seg_sum(ss, g.gs / 8);
      dgs = seg_sum(dgs, g.gs / 8);
      r = 1.0f / sqrtf(ss / (float)g.gs + g.eps);
      sd = r * dgs / (float)g.gs;
    } else {
      const float2 st = stats[(int64_t)tok * (W / g.gs) + (act ? c : 0) / g.gs];
      r = st.x;
      sd = st.y;
    }
    if (act) {
      f32x8 dyv, dzv;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float xh = gv[i] * r;
        dwa[i] += dv[i] * xh;
        const float dg = r * (dv[i] * wv[i] - xh * sd);
        if (z.p) {
          const float s = sigmoid(zv[i]);
          dyv[i] = dg * zv[i] * s;
          dzv[i] = dg * yv[i] * s * (1.0f + zv[i] * (1.0f - s));
        } else {
          dyv[i] = dg;
        }
      }
      store8<float>(g, dy, tok, c, dyv);
      if (z.p) store8<float>(g, dz, tok, c, dzv);
    }
  }
  // the four waves' partials, summed in wave order
#pragma unroll
  for (int i = 0; i < 8; ++i) red[wave][lane * 8 + i] = dwa[i];
  __syncthreads();
  float* prow = part + (int64_t)tile * W + blockIdx.y * kStrip;
  for (int e = threadIdx.x; e < kStrip; e += 256)
    if (blockIdx.y * kStrip + e < W) prow[e] = ((red[0][e] + red[1][e]) + red[2][e]) + red[3][e];
}

// dweight[c] = sum over tiles of part[tile][c]: a workgroup takes 16 channels; thread
// (slice, channel) sums tiles slice, slice + 16, ... in fp64, then the 16 slices are
// added in slice order.  Fixed order throughout.
__global__ __launch_bounds__(256) void k_norm_dw(int W, const float* part, int ntile, float* dw) {
  __shared__ double red[16][17];
  const int cl = threadIdx.x % 16, sl = threadIdx.x / 16;
  const int c = blockIdx.x * 16 + cl;
  double acc = 0.0;
  if (c < W) {
    int t = sl;
    for (; t + 48 < ntile; t += 64) {
      const float a = part[(int64_t)t * W + c], b = part[(int64_t)(t + 16) * W + c];
      const float d = part[(int64_t)(t + 32) * W + c], e = part[(int64_t)(t + 48) * W + c];
      acc += (double)a;
      acc += (double)b;
      acc += (double)d;
      acc += (double)e;
    }
    for (; t < ntile; t += 16) acc += (double)part[(int64_t)t * W + c];
  }
  red[sl][cl] = acc;
  __syncthreads();
  if (sl == 0 && c < W) {
    double s = 0.0;
    for (int i = 0; i < 16; ++i) s += red[i][cl];
    dw[c] = (float)s;
  }
}

}  // namespace

int norm_tiles(const NormGeo& g) { return (g.ntok + kNormTile - 1) / kNormTile; }

hipError_t launch_norm_fwd(const NormGeo& g, TArg y, TArg z, int in_dtype, const float* w,
                           TArg out, int out_dtype, float* rstd, hipStream_t s) {
  const int W = g.H * g.P;
  const int per_tok = g.gs <= kStrip ? (W + kStrip - 1) / kStrip : W / g.gs;
  const int64_t items = (int64_t)g.ntok * per_tok;
  if (items == 0) return hipSuccess;
  dim3 grid((unsigned)((items + 3) / 4));
  if (in_dtype == DT_BF16) {
    if (out_dtype == DT_BF16)
      hipLaunchKernelGGL((k_norm_fwd<bf16, bf16>), grid, dim3(256), 0, s, g, y, z, w, out, rstd);
    else
      hipLaunchKernelGGL((k_norm_fwd<bf16, float>), grid, dim3(256), 0, s, g, y, z, w, out, rstd);
  } else {
    if (out_dtype == DT_BF16)
      hipLaunchKernelGGL((k_norm_fwd<float, bf16>), grid, dim3(256), 0, s, g, y, z, w, out, rstd);
    else
      hipLaunchKernelGGL((k_norm_fwd<float, float>), grid, dim3(256), 0, s, g, y, z, w, out,
                         rstd);
  }
  return hipGetLastError();
}

hipError_t launch_norm_finish(const NormGeo& g, const float* psum, const float* w, TArg out,
                              int out_dtype, float* rstd, hipStream_t s) {
  if (g.ntok == 0) return hipSuccess;
  dim3 grid((unsigned)((g.ntok + 3) / 4));
  if (out_dtype == DT_BF16)
    hipLaunchKernelGGL((k_norm_finish<bf16>), grid, dim3(256), 0, s, g, psum, w, out, rstd);
  else
    hipLaunchKernelGGL((k_norm_finish<float>), grid, dim3(256), 0, s, g, psum, w, out, rstd);
  return hipGetLastError();
}

hipError_t launch_norm_bwd(const NormGeo& g, TArg y, TArg z, int in_dtype, const float* w,
                           TArg dout, TArg dy, TArg dz, float* dw, float* part, float2* stats,
                           hipStream_t s) {
  const int ntile = norm_tiles(g);
  const int W = g.H * g.P;
  if (ntile > 0) {
    if (g.gs > kStrip) {
      const int64_t items = (int64_t)g.ntok * (W / g.gs);
      dim3 grid((unsigned)((items + 3) / 4));
      if (in_dtype == DT_BF16)
        hipLaunchKernelGGL((k_norm_stats<bf16>), grid, dim3(256), 0, s, g, y, z, w, dout, stats);
      else
        hipLaunchKernelGGL((k_norm_stats<float>), grid, dim3(256), 0, s, g, y, z, w, dout, stats);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    dim3 grid(ntile, (W + kStrip - 1) / kStrip);
    if (in_dtype == DT_BF16)
      hipLaunchKernelGGL((k_norm_bwd<bf16>), grid, dim3(256), 0, s, g, y, z, w, dout, stats, dy,
                         dz, part);
    else
      hipLaunchKernelGGL((k_norm_bwd<float>), grid, dim3(256), 0, s, g, y, z, w, dout, stats, dy,
                         dz, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_norm_dw, dim3((W + 15) / 16), dim3(256), 0, s, W, part, ntile, dw);
  return hipGetLastError();
}

}  // namespace ssd
