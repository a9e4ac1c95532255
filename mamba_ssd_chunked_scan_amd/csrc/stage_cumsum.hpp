// stage_cumsum.hpp -- stage 1: step sizes and the within-chunk log-decay cumsum.
//
// delta = softplus(dt + dt_bias) (optionally clamped), a = delta * A_h and
// dA_cumsum[j, h, l] = sum_{l' <= l} a over the chunk's positions; positions
// past a short chunk's end have a = 0 (SSD Reference, "Chunking and the
// discretized log-decay": A_log = softplus(dt) * A, A_cumsum = cumsum over the
// chunk axis; the Mamba-2 chunk-cumsum stage of vLLM PR 27299 "Purpose").
//
// One wavefront per (chunk, head): each lane owns C/64 consecutive positions
// (one position for C = 32 and 64, lanes past C idle), sums them serially, and
// the lane totals are combined with a wave-wide prefix sum.  The stage moves
// ~3 MB at the Nemotron-Nano size and is launch-bound.
//
// The prefix sums are accumulated in fp64 and rounded to fp32 once.  Later
// stages use differences cs[l] - cs[s] of nearby positions as exponents; with
// an fp32 running sum the rounding error grows with the magnitude of the total
// (|cs| reaches hundreds for fast-decaying heads) and would show up as a
// relative error of the same size in the near-diagonal decay weights.
#pragma once
#include "common.hpp"

namespace ssd {

// One wavefront computes chunk j of head h.
template <typename TDt>
__device__ __forceinline__ void cumsum_wave(const Geo& g, const TArg& dt, const float* A,
                                            const float* dt_bias, int softplus, int clamp,
                                            float dt_min, float dt_max, float* cs, float* dt_out,
                                            int j, int h) {
  const int lane = threadIdx.x % kWave;
  Chunk c;
  if (!get_chunk(g, j, c)) return;

  const int C = g.C;
  const int per = (C + kWave - 1) / kWave;  // positions per lane: 1, 1, 2 or 4
  const float Ah = A[h];
  const float bias = dt_bias ? dt_bias[h] : 0.0f;
  float d[4];
  double a[4];
  double run = 0.0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    a[e] = 0.0;
    d[e] = 0.0f;
    const int l = lane * per + e;
    if (e < per && l < c.len) {
      const TDt* p = row_ptr<TDt>(dt, c.b, c.t0 + l, h);
      float u = to_f32<TDt>(*p) + bias;
      float delta = softplus ? softplus_f32(u) : u;
      if (clamp) delta = fminf(fmaxf(delta, dt_min), dt_max);
      d[e] = delta;
      a[e] = (double)(delta * Ah);
    }
    run += a[e];
    a[e] = run;  // lane-local inclusive prefix
  }
  const double incl = wave_inclusive_sum_f64(run);
  const double excl = incl - run;
  float* out = cs + ((int64_t)j * g.H + h) * C;
  float* dout = dt_out ? dt_out + ((int64_t)j * g.H + h) * C : nullptr;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int l = lane * per + e;
    if (e < per && l < C) {
      out[l] = (float)(excl + a[e]);
      if (dout) dout[l] = d[e];
    }
  }
}

}  // namespace ssd
