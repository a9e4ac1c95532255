// bmm_chunk.hip -- stage 2: CB[j, g, l, s] = sum_n C[t0 + l, g, n] B[t0 + s, g, n].
//
// SSD Reference, "Algorithm and tensor-shape contract" step 4 (Cb = Cc Bc^T),
// the BMM stage of vLLM PR 27299 "Purpose".  Only the causal half s <= l is
// ever consumed, so only 16x16 tiles on or below the diagonal are computed.
//
// One workgroup (4 waves) per (chunk, group).  Both operands are read with the
// reduction index n contiguous in memory, which is the layout the matrix-core
// fragments want, so fragments are loaded straight from global memory (16 B
// per lane for bf16); rows past the chunk's end read as zero.  Inputs are exact
// in their storage type, so the products need no hi/lo split.
#include "kernels.hpp"

namespace ssd {

template <typename T>
__global__ __launch_bounds__(256) void k_bmm_chunk(Geo g, TArg Cm, TArg Bm, float* __restrict__ CB) {
  using Pr = Prec<T>;
  const int j = blockIdx.x, grp = blockIdx.y;
  Chunk c;
  if (!get_chunk(g, j, c)) return;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int C = g.C, N = g.N;
  const int nlt = C / 16;
  const int ntiles = nlt * (nlt + 1) / 2;
  const int r16 = lane % 16, q = lane / 16;
  float* out = CB + ((int64_t)j * g.G + grp) * C * C;
  for (int idx = wave; idx < ntiles; idx += 4) {
    int lt = 0;
    while ((lt + 1) * (lt + 2) / 2 <= idx) ++lt;
    const int st = idx - lt * (lt + 1) / 2;
    const int lrow = lt * 16 + r16, srow = st * 16 + r16;
    const bool lok = lrow < c.len, sok = srow < c.len;
    const T* pc = row_ptr<T>(Cm, c.b, c.t0 + (lok ? lrow : 0), grp);
    const T* pb = row_ptr<T>(Bm, c.b, c.t0 + (sok ? srow : 0), grp);
    f32x4 acc = zero4();
    for (int k0 = 0; k0 < N; k0 += 32) {
      const int k = k0 + q * 8;
      const bool kok = k < N;
      typename Pr::Exact a = (lok && kok) ? Pr::load_exact(pc + k) : Pr::zero_exact();
      typename Pr::Exact b = (sok && kok) ? Pr::load_exact(pb + k) : Pr::zero_exact();
      mma(acc, a, b);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int l = lt * 16 + q * 4 + i;
      out[(int64_t)l * C + st * 16 + r16] = acc[i];
    }
  }
}

hipError_t launch_bmm_chunk(const Geo& g, TArg C, TArg B, int in_dtype, float* CB,
                            hipStream_t s) {
  if (g.K == 0) return hipSuccess;
  dim3 grid(g.K, g.G);
  if (in_dtype == DT_BF16)
    hipLaunchKernelGGL(k_bmm_chunk<bf16>, grid, dim3(256), 0, s, g, C, B, CB);
  else
    hipLaunchKernelGGL(k_bmm_chunk<float>, grid, dim3(256), 0, s, g, C, B, CB);
  return hipGetLastError();
}

}  // namespace ssd
