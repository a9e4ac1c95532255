// stage_varlen.hpp -- the packed-batch chunk table, built on the device.
//
// Sequence i (tokens [cu[i], cu[i+1])) is cut into ceil(L_i / C) chunks counted
// from its own first token, so every chunk lies inside one sequence and the
// state can restart at a sequence boundary (continuous batching, vLLM PR 27299
// "Test Plan"; the SSD Reference's chunk grid of "Padding rule" applied per
// sequence).  Table layout is documented in ssd.h (ssd_varlen_meta_len).
//
// One workgroup: pass 1 scans the per-sequence chunk counts (block-wide
// exclusive prefix, 256 sequences per step) into first_chunk[]; pass 2 lets
// every chunk slot j find its sequence by binary search over first_chunk[] and
// write (sequence, first token, length).  Integer-only, bit-exact.
//
// cu_seqlens is read only here, on the device.  For a valid array the table is
// exact.  An invalid one (negative, past T, decreasing) cannot make any later
// kernel touch memory outside the tensors: offsets are clamped to [0, T], each
// sequence's span to [cu[i], T], and chunk ids to the K slots.
#pragma once
#include "common.hpp"

namespace ssd {

__device__ __forceinline__ int block_exclusive_scan(int v, int* lds_waves, int& total) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  int x = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int o = __shfl_up(x, d, kWave);
    if (lane >= d) x += o;
  }
  if (lane == kWave - 1) lds_waves[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
  const int nw = blockDim.x / kWave;
  for (int w = 0; w < nw; ++w) {
    const int t = lds_waves[w];
    if (w < wave) before += t;
    all += t;
  }
  __syncthreads();
  total = all;
  return before + x - v;
}

__device__ __forceinline__ int clamp_tok(int v, int T) { return min(max(v, 0), T); }

__device__ __forceinline__ void seq_span(const int32_t* cu, int i, int T, int& start, int& len) {
  start = clamp_tok(cu[i], T);
  len = max(clamp_tok(cu[i + 1], T) - start, 0);
}

// One workgroup of 256 threads builds the whole table; lds_waves holds 4 ints.
__device__ __forceinline__ void varlen_meta_block(const int32_t* cu, int nseq, int T, int C,
                                                  int K, int32_t* meta, int* lds_waves) {
  int32_t* first = meta + kMetaHeader + 3 * K;
  int base = 0;
  for (int i0 = 0; i0 < nseq; i0 += blockDim.x) {
    const int i = i0 + threadIdx.x;
    int n = 0;
    if (i < nseq) {
      int st, L;
      seq_span(cu, i, T, st, L);
      n = (L + C - 1) / C;
    }
    int tot;
    const int ex = block_exclusive_scan(n, lds_waves, tot);
    if (i < nseq) first[i] = min(base + ex, K);
    base = min(base + tot, K);
  }
  if (threadIdx.x == 0) {
    first[nseq] = base;
    meta[0] = base;
    meta[1] = nseq;
    meta[2] = C;
    meta[3] = K;
  }
  __syncthreads();
  const int Kr = base;
  for (int j = threadIdx.x; j < K; j += blockDim.x) {
    int32_t* e = meta + kMetaHeader + 3 * j;
    if (j >= Kr) {
      e[0] = -1; e[1] = 0; e[2] = 0;
      continue;
    }
    // last sequence i with first[i] <= j; empty sequences share their first
    // value with the next one, and the search skips them.
    int lo = 0, hi = nseq - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (first[mid] <= j) lo = mid; else hi = mid - 1;
    }
    const int k = j - first[lo];
    int st, L;
    seq_span(cu, lo, T, st, L);
    e[0] = lo;
    e[1] = st + k * C;
    e[2] = min(C, L - k * C);
  }
}

}  // namespace ssd
