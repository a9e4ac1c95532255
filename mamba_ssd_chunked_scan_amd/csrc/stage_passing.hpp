// stage_passing.hpp -- stage 4: the sequential scan over the chunks of each sequence.
//
//   Hin[first] = h_init (or 0);   Hin[j + 1] = exp(Lambda_j) Hin[j] + S_j
//   final      = exp(Lambda_last) Hin[last] + S_last
//
// with Lambda_j the chunk's total log-decay (dA_cumsum at its last token).  This
// is the SSD Reference's inter-chunk propagation ("Inter-chunk propagation":
// decay_chunk[z, c] = exp(CD[z-1] - CD[c]) 1[z > c] plus the init term
// exp(CD[z-1]) H_-1) evaluated as a recurrence instead of a (z, c) matrix:
// O(chunks) instead of O(chunks^2) traffic.  It is the "State Passing" stage of
// vLLM PR 27299 and state_passing_fwd of mamba PR 1012.
//
// A pure HBM stream: each thread owns 8 consecutive state elements of one
// (sequence, head) and walks the chunks in order, keeping the running state in
// fp32 registers and reading four chunks ahead.  Hin[j] may overwrite S[j] in
// place: a thread loads S[j] before it stores Hin[j] at the same address and no
// other thread touches those elements.
#pragma once
#include "common.hpp"

namespace ssd {

template <typename ST> struct St8;
template <> struct St8<float> {
  static __device__ __forceinline__ f32x8 load(const float* p) { return Vec8<float>::load(p); }
  static __device__ __forceinline__ void store(float* p, f32x8 v) { Vec8<float>::store(p, v); }
};
template <> struct St8<bf16> {
  static __device__ __forceinline__ f32x8 load(const bf16* p) { return Vec8<bf16>::load(p); }
  static __device__ __forceinline__ void store(bf16* p, f32x8 v) { Vec8<bf16>::store(p, v); }
};

// One thread carries 8 consecutive state elements (starting at e0) of (seq, h).
template <typename ST>
__device__ __forceinline__ void state_passing_thread(const Geo& g, const ST* states,
                                                     const float* cs, const float* h0,
                                                     ST* states_out, float* hfinal, int64_t e0,
                                                     int h, int seq) {
  const int64_t PN = (int64_t)g.P * g.N;
  if (e0 >= PN) return;
  int first, last;
  seq_chunks(g, seq, first, last);

  f32x8 cur;
  if (h0) {
    cur = Vec8<float>::load(h0 + ((int64_t)seq * g.Hs + h) * PN + e0);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) cur[i] = 0.0f;
  }
  constexpr int D = 4;
  for (int j0 = first; j0 < last; j0 += D) {
    f32x8 S[D];
    float dec[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int j = j0 + d;
      if (j < last) {
        Chunk c;
        get_chunk(g, j, c);
        dec[d] = fast_exp(cs[((int64_t)j * g.H + h) * g.C + c.len - 1]);
        S[d] = St8<ST>::load(states + ((int64_t)j * g.H + h) * PN + e0);
      }
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int j = j0 + d;
      if (j < last) {
        St8<ST>::store(states_out + ((int64_t)j * g.H + h) * PN + e0, cur);
#pragma unroll
        for (int i = 0; i < 8; ++i) cur[i] = dec[d] * cur[i] + S[d][i];
      }
    }
  }
  if (hfinal) Vec8<float>::store(hfinal + ((int64_t)seq * g.Hs + h) * PN + e0, cur);
}

}  // namespace ssd
