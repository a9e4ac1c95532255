// bmm_chunk.hip -- the standalone BMM kernel (body in stage_bmm.hpp).
#include "kernels.hpp"
#include "stage_bmm.hpp"

namespace ssd {

template <typename T>
__global__ __launch_bounds__(256) void k_bmm_chunk(Geo g, TArg Cm, TArg Bm, float* __restrict__ CB) {
  bmm_wave<T>(g, Cm, Bm, CB, blockIdx.x, blockIdx.y, blockIdx.z * 4 + threadIdx.x / kWave);
}

template <int C>
__global__ __launch_bounds__(256, 2) void k_bmm_group_bf16(Geo g, TArg Cm, TArg Bm,
                                                         float* __restrict__ CB) {
  __shared__ __align__(16) bf16 s_b[C * (128 + 8)];
  bmm_group_bf16<C>(g, Cm, Bm, CB, blockIdx.x, blockIdx.y, s_b);
}

hipError_t launch_bmm_chunk(const Geo& g, TArg C, TArg B, int in_dtype, float* CB,
                            hipStream_t s) {
  if (g.K == 0) return hipSuccess;
  if (in_dtype == DT_BF16 && g.C <= 128) {
    dim3 grid(g.K, g.G);
    switch (g.C) {
      case 32: hipLaunchKernelGGL(k_bmm_group_bf16<32>, grid, dim3(256), 0, s, g, C, B, CB); break;
      case 64: hipLaunchKernelGGL(k_bmm_group_bf16<64>, grid, dim3(256), 0, s, g, C, B, CB); break;
      default: hipLaunchKernelGGL(k_bmm_group_bf16<128>, grid, dim3(256), 0, s, g, C, B, CB); break;
    }
    return hipGetLastError();
  }
  dim3 grid(g.K, g.G, (g.C / 16 + 3) / 4);
  if (in_dtype == DT_BF16)
    hipLaunchKernelGGL(k_bmm_chunk<bf16>, grid, dim3(256), 0, s, g, C, B, CB);
  else
    hipLaunchKernelGGL(k_bmm_chunk<float>, grid, dim3(256), 0, s, g, C, B, CB);
  return hipGetLastError();
}

}  // namespace ssd
