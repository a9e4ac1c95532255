// chunk_cumsum.hip -- the standalone chunk-cumsum kernel (body in stage_cumsum.hpp).
#include "kernels.hpp"
#include "stage_cumsum.hpp"

namespace ssd {

template <typename TDt>
__global__ __launch_bounds__(256) void k_chunk_cumsum(Geo g, TArg dt, const float* __restrict__ A,
                                                      const float* __restrict__ dt_bias,
                                                      int softplus, int clamp, float dt_min,
                                                      float dt_max, float* __restrict__ cs,
                                                      float* __restrict__ dt_out) {
  const int h = blockIdx.y * 4 + threadIdx.x / kWave;
  if (h >= g.H) return;
  cumsum_wave<TDt>(g, dt, A, dt_bias, softplus, clamp, dt_min, dt_max, cs, dt_out, blockIdx.x, h);
}

hipError_t launch_chunk_cumsum(const Geo& g, TArg dt, int dt_dtype, const float* A,
                               const float* dt_bias, int softplus, int clamp, float dt_min,
                               float dt_max, float* cs, float* dt_out, hipStream_t s) {
  if (g.K == 0) return hipSuccess;
  dim3 grid(g.K, (g.H + 3) / 4);
  if (dt_dtype == DT_BF16)
    hipLaunchKernelGGL(k_chunk_cumsum<bf16>, grid, dim3(256), 0, s, g, dt, A, dt_bias, softplus,
                       clamp, dt_min, dt_max, cs, dt_out);
  else
    hipLaunchKernelGGL(k_chunk_cumsum<float>, grid, dim3(256), 0, s, g, dt, A, dt_bias,
                       softplus, clamp, dt_min, dt_max, cs, dt_out);
  return hipGetLastError();
}

}  // namespace ssd
