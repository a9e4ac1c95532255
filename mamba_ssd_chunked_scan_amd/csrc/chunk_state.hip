// chunk_state.hip -- stage 3: every chunk's end state from a zero start,
//
//   S[j, h, p, n] = sum_{s < len} w_s x[t0 + s, h, p] B[t0 + s, g, n],
//   w_s = exp(cs[len - 1] - cs[s])
//
// SSD Reference, "Intra-chunk outputs and per-chunk states" (the states einsum
// with decay_states = exp(A_cumsum[-1] - A_cumsum)) and "Algorithm and
// tensor-shape contract" step 6 (state = Xc^T (decay_states * Bc)).  Unlike the
// page, the decay weight is folded into x rather than B: x is the per-head
// operand, B is shared by the heads of a group.
//
// Matrix-core formulation: S (P x N) = Xw^T (P x s) * B (s x N) with the
// reduction over tokens s.  Tokens are the strided axis in memory, so each
// 32-token slab of x and B is staged through LDS transposed ([p][s] and [n][s],
// s contiguous), the weighted x split into bf16 hi + lo on the way in.  One
// workgroup covers up to 64 (p) x 128 (n) of one (chunk, head): wave w owns
// p-tile w and all n-tiles, accumulating 8 16x16 fp32 tiles in registers.
#include "kernels.hpp"

namespace ssd {

constexpr int kSlab = 32;

template <typename T> struct StateLds;
template <> struct StateLds<bf16> {
  static constexpr int LD = kSlab + 8;  // 80-byte rows
  bf16 xh[64 * LD];
  bf16 xl[64 * LD];
  bf16 bt[128 * LD];
  float w[256];
};
template <> struct StateLds<float> {
  static constexpr int LD = kSlab + 4;  // 144-byte rows
  float x[64 * LD];
  float bt[128 * LD];
  float w[256];
};

// Stage tokens [s0, s0 + 32) of x (weighted, transposed) and B (transposed).
__device__ __forceinline__ void stage_slab(StateLds<bf16>& L, const Geo& g, const Chunk& c,
                                           const TArg& x, const TArg& B, int h, int grp, int p0,
                                           int n0, int s0) {
  constexpr int LD = StateLds<bf16>::LD;
  const int tid = threadIdx.x;
  {  // x: 32 tokens x 64 p = 256 vectors of 8
    const int s = tid / 8, pp = (tid % 8) * 8;
    f32x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
    const int p = p0 + pp;
    if (s0 + s < c.len && p < g.P) {
      v = Vec8<bf16>::load(row_ptr<bf16>(x, c.b, c.t0 + s0 + s, h) + p);
      const float ws = L.w[s0 + s];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] *= ws;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bf16 hi = (bf16)v[i];
      L.xh[(pp + i) * LD + s] = hi;
      L.xl[(pp + i) * LD + s] = (bf16)(v[i] - (float)hi);
    }
  }
#pragma unroll
  for (int r = 0; r < 2; ++r) {  // B: 32 tokens x 128 n = 512 vectors of 8
    const int v8 = tid + r * 256;
    const int s = v8 / 16, nn = (v8 % 16) * 8;
    const int n = n0 + nn;
    bf16x8 v;
    if (s0 + s < c.len && n < g.N) {
      v = *reinterpret_cast<const bf16x8*>(row_ptr<bf16>(B, c.b, c.t0 + s0 + s, grp) + n);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = (bf16)0.0f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) L.bt[(nn + i) * LD + s] = v[i];
  }
}

__device__ __forceinline__ void stage_slab(StateLds<float>& L, const Geo& g, const Chunk& c,
                                           const TArg& x, const TArg& B, int h, int grp, int p0,
                                           int n0, int s0) {
  constexpr int LD = StateLds<float>::LD;
  const int tid = threadIdx.x;
  {
    const int s = tid / 8, pp = (tid % 8) * 8;
    f32x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
    const int p = p0 + pp;
    if (s0 + s < c.len && p < g.P) {
      v = Vec8<float>::load(row_ptr<float>(x, c.b, c.t0 + s0 + s, h) + p);
      const float ws = L.w[s0 + s];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] *= ws;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) L.x[(pp + i) * LD + s] = v[i];
  }
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int v8 = tid + r * 256;
    const int s = v8 / 16, nn = (v8 % 16) * 8;
    const int n = n0 + nn;
    f32x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
    if (s0 + s < c.len && n < g.N) v = Vec8<float>::load(row_ptr<float>(B, c.b, c.t0 + s0 + s, grp) + n);
#pragma unroll
    for (int i = 0; i < 8; ++i) L.bt[(nn + i) * LD + s] = v[i];
  }
}

__device__ __forceinline__ FragSplit frag_a(const StateLds<bf16>& L, int p, int q) {
  constexpr int LD = StateLds<bf16>::LD;
  FragSplit f;
  f.hi = *reinterpret_cast<const bf16x8*>(&L.xh[p * LD + q * 8]);
  f.lo = *reinterpret_cast<const bf16x8*>(&L.xl[p * LD + q * 8]);
  return f;
}
__device__ __forceinline__ FragBF frag_b(const StateLds<bf16>& L, int n, int q) {
  constexpr int LD = StateLds<bf16>::LD;
  FragBF f;
  f.v = *reinterpret_cast<const bf16x8*>(&L.bt[n * LD + q * 8]);
  return f;
}
__device__ __forceinline__ FragF32 frag_a(const StateLds<float>& L, int p, int q) {
  constexpr int LD = StateLds<float>::LD;
  FragF32 f;
  f.v = Vec8<float>::load(&L.x[p * LD + q * 8]);
  return f;
}
__device__ __forceinline__ FragF32 frag_b(const StateLds<float>& L, int n, int q) {
  constexpr int LD = StateLds<float>::LD;
  FragF32 f;
  f.v = Vec8<float>::load(&L.bt[n * LD + q * 8]);
  return f;
}

template <typename T, typename ST>
__global__ __launch_bounds__(256) void k_chunk_state(Geo g, TArg x, TArg B,
                                                     const float* __restrict__ cs,
                                                     ST* __restrict__ states) {
  __shared__ StateLds<T> L;
  const int j = blockIdx.x, h = blockIdx.y;
  Chunk c;
  if (!get_chunk(g, j, c)) return;
  const int nzn = (g.N + 127) / 128;
  const int p0 = (blockIdx.z / nzn) * 64, n0 = (blockIdx.z % nzn) * 128;
  const int grp = h / g.hpg;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int r16 = lane % 16, q = lane / 16;

  const float* csr = cs + ((int64_t)j * g.H + h) * g.C;
  const float last = csr[c.len - 1];
  for (int s = threadIdx.x; s < g.C; s += blockDim.x)
    L.w[s] = s < c.len ? fast_exp(last - csr[s]) : 0.0f;
  __syncthreads();

  const int pt0 = p0 + wave * 16;       // this wave's p-tile
  const bool active = pt0 < g.P;
  const int ntn = min(8, (g.N - n0) / 16);
  f32x4 acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = zero4();

  for (int s0 = 0; s0 < c.len; s0 += kSlab) {
    stage_slab(L, g, c, x, B, h, grp, p0, n0, s0);
    __syncthreads();
    if (active) {
      const auto a = frag_a(L, wave * 16 + r16, q);
#pragma unroll
      for (int t = 0; t < 8; ++t)
        if (t < ntn) mma(acc[t], a, frag_b(L, t * 16 + r16, q));
    }
    __syncthreads();
  }
  if (!active) return;
  ST* out = states + ((int64_t)j * g.H + h) * g.P * g.N;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    if (t >= ntn) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = pt0 + q * 4 + i;
      const int n = n0 + t * 16 + r16;
      out[(int64_t)p * g.N + n] = from_f32<ST>(acc[t][i]);
    }
  }
}

hipError_t launch_chunk_state(const Geo& g, TArg x, TArg B, int in_dtype, const float* cs,
                              void* states, int st_dtype, hipStream_t s) {
  if (g.K == 0) return hipSuccess;
  dim3 grid(g.K, g.H, ((g.P + 63) / 64) * ((g.N + 127) / 128));
  if (in_dtype == DT_BF16) {
    if (st_dtype == DT_BF16)
      hipLaunchKernelGGL((k_chunk_state<bf16, bf16>), grid, dim3(256), 0, s, g, x, B, cs,
                         (bf16*)states);
    else
      hipLaunchKernelGGL((k_chunk_state<bf16, float>), grid, dim3(256), 0, s, g, x, B, cs,
                         (float*)states);
  } else {
    if (st_dtype == DT_BF16)
      hipLaunchKernelGGL((k_chunk_state<float, bf16>), grid, dim3(256), 0, s, g, x, B, cs,
                         (bf16*)states);
    else
      hipLaunchKernelGGL((k_chunk_state<float, float>), grid, dim3(256), 0, s, g, x, B, cs,
                         (float*)states);
  }
  return hipGetLastError();
}

}  // namespace ssd
