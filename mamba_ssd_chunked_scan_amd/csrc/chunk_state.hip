// chunk_state.hip -- the standalone chunk-state kernels.  The bf16 body lives in
// stage_state.hpp; fp32 inputs use a simpler slab loop with fp32 matrix
// instructions.  With the step size on the input term (dtc != NULL) each
// token's decay weight is multiplied by its step size.
#include "kernels.hpp"
#include "stage_state.hpp"

namespace ssd {

template <typename ST, int C>
__global__ __launch_bounds__(256, 4) void k_chunk_state_bf16(Geo g, TArg x, TArg B,
                                                          const float* __restrict__ cs,
                                                          const float* __restrict__ dtc,
                                                          ST* __restrict__ states) {
  __shared__ __align__(16) char smem[chunk_state_lds_bytes<C>()];
  chunk_state_block<ST, C>(g, x, B, cs, dtc, states, blockIdx.x, blockIdx.y, blockIdx.z, smem);
}

// ------------------------------------------------------------------ fp32 path

constexpr int kSlabF = 32;
struct StateLdsF32 {
  static constexpr int LD = kSlabF + 4;  // 144-byte rows
  float x[64 * LD];
  float bt[128 * LD];
  float w[256];
};

__global__ __launch_bounds__(256) void k_chunk_state_f32(Geo g, TArg x, TArg B,
                                                         const float* __restrict__ cs,
                                                         const float* __restrict__ dtc,
                                                         float* __restrict__ states_f,
                                                         bf16* __restrict__ states_b) {
  __shared__ StateLdsF32 L;
  constexpr int LD = StateLdsF32::LD;
  const int j = blockIdx.x, h = blockIdx.y;
  Chunk c;
  if (!get_chunk(g, j, c)) return;
  const int nzn = (g.N + 127) / 128;
  const int p0 = (blockIdx.z / nzn) * 64, n0 = (blockIdx.z % nzn) * 128;
  const int grp = h / g.hpg;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int r16 = lane % 16, q = lane / 16;
  const float* csr = cs + ((int64_t)j * g.H + h) * g.C;
  const float* dtr = dtc ? dtc + ((int64_t)j * g.H + h) * g.C : nullptr;
  const float last = csr[c.len - 1];
  for (int s = tid; s < g.C; s += blockDim.x)
    L.w[s] = s < c.len ? fast_exp(last - csr[s]) * (dtr ? dtr[s] : 1.0f) : 0.0f;
  __syncthreads();
  const int pt0 = p0 + wave * 16;
  const bool active = pt0 < g.P;
  const int ntn = min(8, (g.N - n0) / 16);
  f32x4 acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = zero4();
  for (int s0 = 0; s0 < c.len; s0 += kSlabF) {
    {
      const int s = tid / 8, pp = (tid % 8) * 8, p = p0 + pp;
      f32x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
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
      const int s = v8 / 16, nn = (v8 % 16) * 8, n = n0 + nn;
      f32x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
      if (s0 + s < c.len && n < g.N) v = Vec8<float>::load(row_ptr<float>(B, c.b, c.t0 + s0 + s, grp) + n);
#pragma unroll
      for (int i = 0; i < 8; ++i) L.bt[(nn + i) * LD + s] = v[i];
    }
    __syncthreads();
    if (active) {
      FragF32 a;
      a.v = Vec8<float>::load(&L.x[(wave * 16 + r16) * LD + q * 8]);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        if (t < ntn) {
          FragF32 b;
          b.v = Vec8<float>::load(&L.bt[(t * 16 + r16) * LD + q * 8]);
          mma(acc[t], a, b);
        }
      }
    }
    __syncthreads();
  }
  if (!active) return;
  const int64_t base = ((int64_t)j * g.H + h) * g.P * g.N;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    if (t >= ntn) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t o = base + (int64_t)(pt0 + q * 4 + i) * g.N + n0 + t * 16 + r16;
      if (states_f) states_f[o] = acc[t][i];
      else states_b[o] = (bf16)acc[t][i];
    }
  }
}

template <typename ST>
static hipError_t launch_state_bf16(const Geo& g, TArg x, TArg B, const float* cs,
                                    const float* dtc, ST* st, hipStream_t s) {
  dim3 grid(g.K, g.H, ((g.P + 63) / 64) * ((g.N + 127) / 128));
  switch (g.C) {
    case 32: hipLaunchKernelGGL((k_chunk_state_bf16<ST, 32>), grid, dim3(256), 0, s, g, x, B, cs, dtc, st); break;
    case 64: hipLaunchKernelGGL((k_chunk_state_bf16<ST, 64>), grid, dim3(256), 0, s, g, x, B, cs, dtc, st); break;
    case 128: hipLaunchKernelGGL((k_chunk_state_bf16<ST, 128>), grid, dim3(256), 0, s, g, x, B, cs, dtc, st); break;
    default: hipLaunchKernelGGL((k_chunk_state_bf16<ST, 256>), grid, dim3(256), 0, s, g, x, B, cs, dtc, st); break;
  }
  return hipGetLastError();
}

hipError_t launch_chunk_state(const Geo& g, TArg x, TArg B, int in_dtype, const float* cs,
                              const float* dtc, void* states, int st_dtype, hipStream_t s) {
  if (g.K == 0) return hipSuccess;
  if (in_dtype == DT_BF16) {
    if (st_dtype == DT_BF16) return launch_state_bf16<bf16>(g, x, B, cs, dtc, (bf16*)states, s);
    return launch_state_bf16<float>(g, x, B, cs, dtc, (float*)states, s);
  }
  dim3 grid(g.K, g.H, ((g.P + 63) / 64) * ((g.N + 127) / 128));
  hipLaunchKernelGGL(k_chunk_state_f32, grid, dim3(256), 0, s, g, x, B, cs, dtc,
                     st_dtype == DT_BF16 ? nullptr : (float*)states,
                     st_dtype == DT_BF16 ? (bf16*)states : nullptr);
  return hipGetLastError();
}

}  // namespace ssd
