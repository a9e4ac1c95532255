// stage_bmm.hpp -- stage 2: CB[j, g, l, s] = sum_n C[t0 + l, g, n] B[t0 + s, g, n].
//
// SSD Reference, "Algorithm and tensor-shape contract" step 4 (Cb = Cc Bc^T),
// the BMM stage of vLLM PR 27299 "Purpose".  Only the causal half s <= l is
// ever consumed, so only 16x16 tiles on or below the diagonal are computed.
//
// Both operands are read with the reduction index n contiguous in memory, the
// layout the matrix-core fragments want, so fragments come straight from
// global memory (16 B per lane for bf16).  One wavefront per (chunk, group,
// 16-row l-tile) computes the l-tile's causal s-tiles four at a time: all
// fragment loads of a batch are issued together (one memory round trip per
// batch of up to 128 columns of N), rows past the chunk's end and columns past
// N are zeroed by select when used, and every matrix instruction runs outside
// data-dependent branches.
// Inputs are exact in their storage type, so the products need no hi/lo split.
#pragma once
#include <type_traits>

#include "common.hpp"

namespace ssd {

// One wavefront computes the causal tiles of l-tile lt of (chunk j, group grp).
template <typename T>
__device__ __forceinline__ void bmm_wave(const Geo& g, const TArg& Cm, const TArg& Bm, float* CB,
                                         int j, int grp, int lt) {
  using Pr = Prec<T>;
  using Ex = typename Pr::Exact;
  Chunk c;
  if (!get_chunk(g, j, c)) return;
  const int lane = threadIdx.x % kWave;
  const int C = g.C, N = g.N;
  if (lt >= C / 16) return;
  const int r16 = lane % 16, q = lane / 16;
  const int lrow = lt * 16 + r16;
  const T* crow = row_ptr<T>(Cm, c.b, c.t0 + min(lrow, c.len - 1), grp);
  const bool lok = lrow < c.len;
  float* out = CB + ((int64_t)j * g.G + grp) * C * C;

  for (int st0 = 0; st0 <= lt; st0 += 4) {
    f32x4 acc[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[b] = zero4();
    // NB k-blocks of 32 starting at n0: every load first (addresses clamped
    // into the rows and into N), then the matrix instructions, with rows past
    // the chunk's end and k past N zeroed by select
    auto batch = [&](auto nb, int n0) {
      constexpr int NB = decltype(nb)::value;
      Ex a[NB], bf[4][NB];
#pragma unroll
      for (int kk = 0; kk < NB; ++kk) {
        const int k = min(n0 + kk * 32 + q * 8, N - 8);
        a[kk] = Pr::load_exact(crow + k);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int srow = min((st0 + b) * 16 + r16, c.len - 1);
          bf[b][kk] = Pr::load_exact(row_ptr<T>(Bm, c.b, c.t0 + srow, grp) + k);
        }
      }
#pragma unroll
      for (int kk = 0; kk < NB; ++kk) {
        const bool kok = n0 + kk * 32 + q * 8 < N;
        const Ex av = lok && kok ? a[kk] : Pr::zero_exact();
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const bool sok = (st0 + b) * 16 + r16 < c.len && kok;
          mma(acc[b], av, sok ? bf[b][kk] : Pr::zero_exact());
        }
      }
    };
    // 128-wide blocks, then the tail of N (a multiple of 16) in blocks of 64
    // and 32; all branches are uniform, so no matrix instruction sits under a
    // data-dependent one
    int n0 = 0;
    for (; n0 + 128 <= N; n0 += 128) batch(std::integral_constant<int, 4>(), n0);
    if (n0 + 64 <= N) {
      batch(std::integral_constant<int, 2>(), n0);
      n0 += 64;
    }
    for (; n0 < N; n0 += 32) batch(std::integral_constant<int, 1>(), n0);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if (st0 + b > lt) break;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        out[(int64_t)(lt * 16 + q * 4 + i) * C + (st0 + b) * 16 + r16] = acc[b][i];
    }
  }
}

// bf16 inputs, C <= 128: one workgroup of four waves per (chunk, group), the
// whole causal half in one round.  Wave w owns l-tile w and, at C = 128, also
// l-tile 7 - w, so every wave computes nine causal tiles (the causal triangle
// split evenly).  s-tiles come in batches of four; the l-tile of slot u needs
// batches 0..u, and batch 0 serves both slots, so each B fragment a wave needs
// is loaded once.  Every load of a 128-wide block of N (the C fragments of
// both l-tiles and the B fragments of both batches, 40 x 16 B per lane) is
// issued before the first matrix instruction.  The k-blocks accumulate in the
// same order as in bmm_wave, so both give the same bits.
template <int C>
__device__ __forceinline__ void bmm_group_bf16(const Geo& g, const TArg& Cm, const TArg& Bm,
                                               float* CB, int j, int grp) {
  constexpr int NLT = C / 16;
  constexpr int LTW = NLT >= 8 ? 2 : 1;  // l-tile slots per wave
  static_assert(C <= 128, "one workgroup covers at most eight l-tiles");
  Chunk c;
  if (!get_chunk(g, j, c)) return;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  if (wave >= NLT) return;  // C = 32: two l-tiles
  const int r16 = lane % 16, q = lane / 16;
  const int N = g.N;
  float* out = CB + ((int64_t)j * g.G + grp) * C * C;
  int lt[LTW];
  lt[0] = wave;
  if (LTW == 2) lt[LTW - 1] = NLT - 1 - wave;

  f32x4 acc[LTW][LTW][4];  // [slot][s-batch][s-tile of the batch]; slot u uses batches 0..u
#pragma unroll
  for (int u = 0; u < LTW; ++u)
#pragma unroll
    for (int sb = 0; sb < LTW; ++sb)
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) acc[u][sb][bi] = zero4();

  for (int n0 = 0; n0 < N; n0 += 128) {
    FragBF a[LTW][4], b[LTW][4][4];
#pragma unroll
    for (int u = 0; u < LTW; ++u) {
      const bf16* crow = row_ptr<bf16>(Cm, c.b, c.t0 + min(lt[u] * 16 + r16, c.len - 1), grp);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) a[u][kb].v = *reinterpret_cast<const bf16x8*>(crow + min(n0 + kb * 32 + q * 8, N - 8));
    }
#pragma unroll
    for (int sb = 0; sb < LTW; ++sb)
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) {
        const bf16* brow =
            row_ptr<bf16>(Bm, c.b, c.t0 + min((4 * sb + bi) * 16 + r16, c.len - 1), grp);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          b[sb][bi][kb].v = *reinterpret_cast<const bf16x8*>(brow + min(n0 + kb * 32 + q * 8, N - 8));
      }
    const FragBF zf = Prec<bf16>::zero_exact();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const bool kok = n0 + kb * 32 + q * 8 < N;
#pragma unroll
      for (int u = 0; u < LTW; ++u) {
        const FragBF av = kok && lt[u] * 16 + r16 < c.len ? a[u][kb] : zf;
#pragma unroll
        for (int sb = 0; sb <= u; ++sb)
#pragma unroll
          for (int bi = 0; bi < 4; ++bi) {
            const bool sok = kok && (4 * sb + bi) * 16 + r16 < c.len;
            mma(acc[u][sb][bi], av, sok ? b[sb][bi][kb] : zf);
          }
      }
    }
  }
#pragma unroll
  for (int u = 0; u < LTW; ++u)
#pragma unroll
    for (int sb = 0; sb <= u; ++sb)
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) {
        const int st = 4 * sb + bi;
        if (st > lt[u]) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          out[(int64_t)(lt[u] * 16 + q * 4 + i) * C + st * 16 + r16] = acc[u][sb][bi][i];
      }
}

}  // namespace ssd
