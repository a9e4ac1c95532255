// varlen_meta.hip -- the standalone chunk-table kernel (body in stage_varlen.hpp).
#include "kernels.hpp"
#include "stage_varlen.hpp"

namespace ssd {

__global__ __launch_bounds__(256) void k_varlen_meta(const int32_t* __restrict__ cu, int nseq,
                                                     int T, int C, int K,
                                                     int32_t* __restrict__ meta) {
  __shared__ int lds_waves[4];
  varlen_meta_block(cu, nseq, T, C, K, meta, lds_waves);
}

hipError_t launch_varlen_meta(const Geo& g, const int32_t* cu_seqlens, int32_t* meta,
                              hipStream_t s) {
  hipLaunchKernelGGL(k_varlen_meta, dim3(1), dim3(256), 0, s, cu_seqlens, g.nseq, g.T, g.C,
                     g.K, meta);
  return hipGetLastError();
}

}  // namespace ssd
