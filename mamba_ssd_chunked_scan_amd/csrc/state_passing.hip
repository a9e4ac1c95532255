// state_passing.hip -- the standalone state-passing kernel (body in stage_passing.hpp).
#include "kernels.hpp"
#include "stage_passing.hpp"

namespace ssd {

template <typename ST>
__global__ __launch_bounds__(256) void k_state_passing(Geo g, const ST* states,
                                                       const float* __restrict__ cs,
                                                       const float* __restrict__ h0,
                                                       ST* states_out,
                                                       float* __restrict__ hfinal) {
  const int64_t e0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  state_passing_thread<ST>(g, states, cs, h0, states_out, hfinal, e0, blockIdx.y, blockIdx.z);
}

hipError_t launch_state_passing(const Geo& g, const void* states, int st_dtype,
                                const float* cs, const float* h0, void* states_out,
                                float* hfinal, hipStream_t s) {
  const int64_t PN = (int64_t)g.P * g.N;
  const int threads = 256;
  dim3 grid((unsigned)((PN / 8 + threads - 1) / threads), g.H, g.nseq);
  if (g.nseq == 0) return hipSuccess;
  if (st_dtype == DT_BF16)
    hipLaunchKernelGGL(k_state_passing<bf16>, grid, dim3(threads), 0, s, g,
                       (const bf16*)states, cs, h0, (bf16*)states_out, hfinal);
  else
    hipLaunchKernelGGL(k_state_passing<float>, grid, dim3(threads), 0, s, g,
                       (const float*)states, cs, h0, (float*)states_out, hfinal);
  return hipGetLastError();
}

}  // namespace ssd
