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

// The adjoint of the scan above, per (sequence, head), 8 state elements per
// thread, chunks walked last to first: with U_j the gradient that chunk j's
// own tokens send to the state entering it,
//   dHout[last] = dfinal (or 0);  dHout[j - 1] = exp(Lambda_j) dHout[j] + U_j
// stores dHout[j] (the gradient of the state leaving chunk j through later
// tokens) over U_j in place, and the gradient of the initial state, dHin of the
// first chunk (dfinal itself for a sequence without tokens), into dh0.
__device__ __forceinline__ void state_passing_rev_thread(const Geo& g, float* adj,
                                                         const float* cs, const float* dfinal,
                                                         float* dh0, int64_t e0, int h, int seq) {
  const int64_t PN = (int64_t)g.P * g.N;
  if (e0 >= PN) return;
  int first, last;
  seq_chunks(g, seq, first, last);
  f32x8 cur;
  if (dfinal) {
    cur = Vec8<float>::load(dfinal + ((int64_t)seq * g.Hs + h) * PN + e0);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) cur[i] = 0.0f;
  }
  constexpr int D = 4;
  for (int j0 = last - 1; j0 >= first; j0 -= D) {
    f32x8 U[D];
    float dec[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int j = j0 - d;
      if (j >= first) {
        Chunk c;
        get_chunk(g, j, c);
        dec[d] = fast_exp(cs[((int64_t)j * g.H + h) * g.C + c.len - 1]);
        U[d] = Vec8<float>::load(adj + ((int64_t)j * g.H + h) * PN + e0);
      }
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int j = j0 - d;
      if (j >= first) {
        Vec8<float>::store(adj + ((int64_t)j * g.H + h) * PN + e0, cur);
#pragma unroll
        for (int i = 0; i < 8; ++i) cur[i] = dec[d] * cur[i] + U[d][i];
      }
    }
  }
  if (dh0) Vec8<float>::store(dh0 + ((int64_t)seq * g.Hs + h) * PN + e0, cur);
}

// Both scans of the per-chunk backward in one launch: sequences [0, nseq) of
// the grid's z axis run the forward scan (fp32 states, in place, from h0; no
// final state), [nseq, 2 nseq) the reverse one.  The two are independent and
// each is a walk over the chunks bound by the latency of its loads, so running
// them side by side overlaps the two walks.
__global__ __launch_bounds__(256) void k_state_passing_pair(Geo g, float* states,
                                                            const float* __restrict__ cs,
                                                            const float* __restrict__ h0,
                                                            float* adj,
                                                            const float* __restrict__ dfinal,
                                                            float* __restrict__ dh0) {
  const int64_t e0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  const int h = blockIdx.y, z = blockIdx.z;
  if (z < g.nseq)
    state_passing_thread<float>(g, states, cs, h0, states, nullptr, e0, h, z);
  else
    state_passing_rev_thread(g, adj, cs, dfinal, dh0, e0, h, z - g.nseq);
}

hipError_t launch_state_passing_pair(const Geo& g, float* states, const float* cs,
                                     const float* h0, float* adj, const float* dfinal, float* dh0,
                                     hipStream_t s) {
  const int64_t PN = (int64_t)g.P * g.N;
  dim3 grid((unsigned)((PN / 8 + 255) / 256), g.H, 2 * g.nseq);
  if (g.nseq == 0) return hipSuccess;
  hipLaunchKernelGGL(k_state_passing_pair, grid, dim3(256), 0, s, g, states, cs, h0, adj, dfinal,
                     dh0);
  return hipGetLastError();
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
