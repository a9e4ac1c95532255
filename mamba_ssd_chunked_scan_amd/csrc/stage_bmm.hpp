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

// C.B^T of one (chunk, group) for chunks of at most 128 tokens (bf16): one
// workgroup of four waves covers the whole causal half in one round.  Wave w
// owns l-tile w and, at C = 128, also l-tile 7 - w, so every wave computes nine
// causal tiles (the causal triangle split evenly).  The chunk's B rows are
// staged in LDS once per 128-wide block of N (rows past the chunk and columns
// past N zeroed there) and each wave loads only its C fragments: a workgroup
// moves 64 KB through L2 per block, where loading every B fragment a wave needs
// from memory moved 160 KB (20.2 -> 16.1 us at the Nemotron-Nano size).  Per
// k-block, every B fragment (natural layout: one row s, eight consecutive n)
// is read before the products; each serves both of the wave's l-tiles.  The
// k-blocks accumulate in the same order as in bmm_wave, so both give the same
// bits.
template <int C>
__device__ __forceinline__ void bmm_group_bf16(const Geo& g, const TArg& Cm, const TArg& Bm,
                                              float* CB, int j, int grp, bf16* s_b) {
  constexpr int NLT = C / 16;
  constexpr int LTW = NLT >= 8 ? 2 : 1;  // l-tile slots per wave
  constexpr int BLD = 128 + 8;           // bf16 per staged B row
  static_assert(C <= 128, "one workgroup covers at most eight l-tiles");
  Chunk c;
  if (!get_chunk(g, j, c)) return;  // (uniform: the whole workgroup leaves)
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int r16 = lane % 16, q = lane / 16;
  const int N = g.N;
  const bool active = wave < NLT;  // C = 32: two l-tiles, waves 2 and 3 only stage
  float* out = CB + ((int64_t)j * g.G + grp) * C * C;
  int lt[LTW];
  lt[0] = wave;
  if (LTW == 2) lt[LTW - 1] = NLT - 1 - wave;

  f32x4 acc[LTW][NLT];
#pragma unroll
  for (int u = 0; u < LTW; ++u)
#pragma unroll
    for (int st = 0; st < NLT; ++st) acc[u][st] = zero4();
  const FragBF zf = Prec<bf16>::zero_exact();
  for (int n0 = 0; n0 < N; n0 += 128) {
    __syncthreads();  // every wave is done with the previous block's B rows
    {
      const int row0 = tid / 16, col = (tid % 16) * 8;
      const bool cok = n0 + col < N;
      const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int k = 0; k < C / 16; ++k) {
        const int row = row0 + 16 * k;
        const bf16* brow = row_ptr<bf16>(Bm, c.b, c.t0 + min(row, c.len - 1), grp);
        const u32x4 v = *reinterpret_cast<const u32x4*>(brow + min(n0 + col, N - 8));
        *reinterpret_cast<u32x4*>(&s_b[row * BLD + col]) = (row < c.len && cok) ? v : zero;
      }
    }
    FragBF a[LTW][4];
#pragma unroll
    for (int u = 0; u < LTW; ++u) {
      const int l = min(lt[u], NLT - 1) * 16 + r16;
      const bf16* crow = row_ptr<bf16>(Cm, c.b, c.t0 + min(l, c.len - 1), grp);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int n = n0 + kb * 32 + q * 8;
        FragBF v;
        v.v = *reinterpret_cast<const bf16x8*>(crow + min(n, N - 8));
        a[u][kb] = (l < c.len && n < N) ? v : zf;
      }
    }
    __syncthreads();
    if (active) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        FragBF bt[NLT];
#pragma unroll
        for (int st = 0; st < NLT; ++st)
          bt[st].v = *reinterpret_cast<const bf16x8*>(&s_b[(st * 16 + r16) * BLD + kb * 32 + q * 8]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int st = 0; st < NLT; ++st)
#pragma unroll
          for (int u = 0; u < LTW; ++u)
            if (st <= lt[u]) mma(acc[u][st], a[u][kb], bt[st]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  if (!active) return;
#pragma unroll
  for (int u = 0; u < LTW; ++u)
#pragma unroll
    for (int st = 0; st < NLT; ++st) {
      if (st > lt[u]) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        out[(int64_t)(lt[u] * 16 + q * 4 + i) * C + st * 16 + r16] = acc[u][st][i];
    }
}

}  // namespace ssd
