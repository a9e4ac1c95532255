// state_scan.hip -- chunk states and the inter-chunk scan in one pass.
//
// For every sequence, head h and chunk j in order:
//   S_j   = sum_{s < len} exp(cs[len-1] - cs[s]) x_s (outer) B_s      (chunk state)
//   Hin_j = carry;   carry = exp(Lambda_j) carry + S_j                  (state passing)
// i.e. the SSD Reference's per-chunk states ("Intra-chunk outputs and
// per-chunk states") fed straight into its inter-chunk propagation
// ("Inter-chunk propagation", the decay_chunk / init-state recurrence).  The
// per-chunk states S_j never leave registers: only the carry-in states Hin_j
// (what the chunk scan consumes) and the final states are written.  Compared
// with running the chunk-state and state-passing stages back to back this
// removes one write and one read of every S_j.
//
// Work split: one workgroup per (sequence, head, 16 rows of P, 64 columns of
// N); it walks its sequence's chunks serially.  Wave w owns the 16x16 block of
// columns [16w, 16w+16), so the carried state is four fp32 per lane, held in
// the matrix-core accumulator layout.  Loads for a chunk depend on nothing
// computed before, so they are issued three chunks ahead (register ring);
// per chunk a workgroup then only does the LDS transpose (packed token pairs,
// decay-weighted x split into bf16 hi + lo), 4 k-blocks x 2 matrix
// instructions per wave, the carry update and the store of Hin_j.
#include "kernels.hpp"

namespace ssd {

template <int C> struct ChainCfg {
  static constexpr int NPAIR = C / 2;
  static constexpr int LDW = (C + 8) / 2;     // dwords per transposed row
  static constexpr int XU = (2 * NPAIR + 255) / 256;   // x units: 2 tokens x 8 p (16 p = 2 groups)
  static constexpr int BU = (8 * NPAIR + 255) / 256;   // B units: 2 tokens x 8 n (64 n = 8 groups)
  static constexpr int DEPTH = 3;                      // chunks in flight
};

template <int C> struct ChainStage {
  u32x4 x[ChainCfg<C>::XU][2];
  u32x4 b[ChainCfg<C>::BU][2];
  float cs0[ChainCfg<C>::XU], cs1[ChainCfg<C>::XU];  // cumsum at this thread's x tokens
  float last;                                        // cumsum at the chunk's last token
  int len;
};

template <typename ST, int C>
__global__ __launch_bounds__(256) void k_state_scan_bf16(Geo g, TArg x, TArg B,
                                                         const float* __restrict__ cs,
                                                         const float* __restrict__ h0,
                                                         ST* __restrict__ hin,
                                                         float* __restrict__ hfinal) {
  using Cfg = ChainCfg<C>;
  constexpr int NPAIR = Cfg::NPAIR, LDW = Cfg::LDW, XU = Cfg::XU, BU = Cfg::BU, DEPTH = Cfg::DEPTH;
  __shared__ __align__(16) uint32_t xh[16 * LDW];
  __shared__ __align__(16) uint32_t xl[16 * LDW];
  __shared__ __align__(16) uint32_t bt[64 * LDW];

  // logical item = ((seq * H + h) * slices + slice): the slices of one head,
  // and the heads of one group, are consecutive -> placed on one XCD, where
  // they share the L2 lines of x and B
  const int nns = (g.N + 63) / 64;
  const int slices = (g.P / 16) * nns;
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  const int slice = item % slices;
  const int h = (item / slices) % g.H, seq = item / (slices * g.H);
  const int ps = slice / nns, ns = slice % nns;
  const int p0 = ps * 16, n0 = ns * 64;
  const int grp = h / g.hpg;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int r16 = lane % 16, q = lane / 16;
  int first, last;
  seq_chunks(g, seq, first, last);
  const int64_t PN = (int64_t)g.P * g.N;

  // carry: rows p0 + q*4 + i, column n0 + 16*wave + r16
  const bool wave_on = n0 + wave * 16 < g.N;
  f32x4 carry = zero4();
  if (h0 && wave_on) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      carry[i] = h0[((int64_t)seq * g.H + h) * PN + (int64_t)(p0 + q * 4 + i) * g.N + n0 +
                    wave * 16 + r16];
  }

  if (first >= last) {  // empty sequence: the final state is the initial one
    if (hfinal && wave_on) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        hfinal[((int64_t)seq * g.H + h) * PN + (int64_t)(p0 + q * 4 + i) * g.N + n0 + wave * 16 +
               r16] = carry[i];
    }
    return;
  }

  // Loads are unconditional (addresses clamped into the sequence's last real
  // chunk): with no branch around a memory instruction the loop body is
  // straight-line code, and the compiler can wait for exactly the chunk being
  // consumed while later prefetches stay in flight.  Data past the chunk's end
  // is zeroed where it is consumed, not where it is loaded -- a select right
  // after the load would make the load's result needed (and waited for)
  // immediately.
  ChainStage<C> ring[DEPTH];
  auto load = [&](ChainStage<C>& st, int j) {
    const bool ok = j < last;
    Chunk c;
    get_chunk(g, ok ? j : last - 1, c);
    st.len = ok ? c.len : 0;
    const float* csr = cs + ((int64_t)(ok ? j : last - 1) * g.H + h) * C;
    st.last = csr[c.len - 1];
#pragma unroll
    for (int k = 0; k < XU; ++k) {
      const int u = min(tid + 256 * k, 2 * NPAIR - 1);
      const int grp8 = u / NPAIR, pr = u % NPAIR;
      st.cs0[k] = csr[2 * pr];
      st.cs1[k] = csr[2 * pr + 1];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int s = 2 * pr + t;
        st.x[k][t] = *reinterpret_cast<const u32x4*>(
            row_ptr<bf16>(x, c.b, c.t0 + min(s, c.len - 1), h) + p0 + grp8 * 8);
      }
    }
#pragma unroll
    for (int k = 0; k < BU; ++k) {
      const int u = min(tid + 256 * k, 8 * NPAIR - 1);
      const int grp8 = u / NPAIR, pr = u % NPAIR;
      const int n = n0 + grp8 * 8;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int s = 2 * pr + t;
        st.b[k][t] = *reinterpret_cast<const u32x4*>(
            row_ptr<bf16>(B, c.b, c.t0 + min(s, c.len - 1), grp) + min(n, g.N - 8));
      }
    }
  };

#pragma unroll
  for (int d = 0; d < DEPTH; ++d) load(ring[d], first + d);

  for (int j0 = first; j0 < last; j0 += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int j = j0 + d;
      if (j >= last) break;
      ChainStage<C>& st = ring[d];
      // transposed, decay-weighted x (hi/lo) and B into LDS
#pragma unroll
      for (int k = 0; k < XU; ++k) {
        const int u = tid + 256 * k;
        if (u >= 2 * NPAIR) continue;
        const int grp8 = u / NPAIR, pr = u % NPAIR;
        const float wa = 2 * pr < st.len ? fast_exp(st.last - st.cs0[k]) : 0.0f;
        const float wb = 2 * pr + 1 < st.len ? fast_exp(st.last - st.cs1[k]) : 0.0f;
#pragma unroll
        for (int dd = 0; dd < 4; ++dd) {
          // tokens past the chunk's end hold a copy of its last token: weight 0
          const uint32_t ua = st.x[k][0][dd], ub = st.x[k][1][dd];
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const float fa = (half ? bf16_hi_f32(ua) : bf16_lo_f32(ua)) * wa;
            const float fb = (half ? bf16_hi_f32(ub) : bf16_lo_f32(ub)) * wb;
            const bf16 ha = (bf16)fa, hb = (bf16)fb;
            const int row = grp8 * 8 + 2 * dd + half;
            xh[row * LDW + pr] = pack2(ha, hb);
            xl[row * LDW + pr] = pack2((bf16)(fa - (float)ha), (bf16)(fb - (float)hb));
          }
        }
      }
#pragma unroll
      for (int k = 0; k < BU; ++k) {
        const int u = tid + 256 * k;
        if (u >= 8 * NPAIR) continue;
        const int grp8 = u / NPAIR, pr = u % NPAIR;
        const bool n_ok = n0 + grp8 * 8 < g.N;
        const bool k0 = n_ok && 2 * pr < st.len, k1 = n_ok && 2 * pr + 1 < st.len;
#pragma unroll
        for (int dd = 0; dd < 4; ++dd) {
          const int row = grp8 * 8 + 2 * dd;
          const uint32_t ba = k0 ? st.b[k][0][dd] : 0u, bb = k1 ? st.b[k][1][dd] : 0u;
          bt[row * LDW + pr] = pack_lo(ba, bb);
          bt[(row + 1) * LDW + pr] = pack_hi(ba, bb);
        }
      }
      const float lam = st.last;
      __syncthreads();
      // the slot is consumed: refill it with the chunk DEPTH ahead
      load(st, j + DEPTH);
      // S_j block for this wave
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < C / 32; ++kb) {
        const int off = kb * 16 + q * 4;
        FragSplit a;
        a.hi = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&xh[r16 * LDW + off]));
        a.lo = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&xl[r16 * LDW + off]));
        FragBF b;
        b.v = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                             &bt[(wave * 16 + r16) * LDW + off]));
        mma(acc, a, b);
      }
      // Hin_j = carry, then carry = exp(Lambda_j) carry + S_j
      if (wave_on) {
        ST* out = hin + ((int64_t)j * g.H + h) * PN + n0 + wave * 16 + r16;
        const float e = fast_exp(lam);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          out[(int64_t)(p0 + q * 4 + i) * g.N] = from_f32<ST>(carry[i]);
          carry[i] = e * carry[i] + acc[i];
        }
      }
      __syncthreads();
    }
  }
  if (hfinal && wave_on) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      hfinal[((int64_t)seq * g.H + h) * PN + (int64_t)(p0 + q * 4 + i) * g.N + n0 + wave * 16 +
             r16] = carry[i];
  }
}

hipError_t launch_state_scan(const Geo& g, TArg x, TArg B, const float* cs, const float* h0,
                             void* hin, int st_dtype, float* hfinal, hipStream_t s) {
  if (g.nseq == 0) return hipSuccess;
  dim3 grid((g.P / 16) * ((g.N + 63) / 64) * g.H * g.nseq);
#define SSD_CHAIN(ST, CC)                                                                  \
  hipLaunchKernelGGL((k_state_scan_bf16<ST, CC>), grid, dim3(256), 0, s, g, x, B, cs, h0, \
                     (ST*)hin, hfinal)
  const bool sb = st_dtype == DT_BF16;
  switch (g.C) {
    case 32: if (sb) SSD_CHAIN(bf16, 32); else SSD_CHAIN(float, 32); break;
    case 64: if (sb) SSD_CHAIN(bf16, 64); else SSD_CHAIN(float, 64); break;
    case 128: if (sb) SSD_CHAIN(bf16, 128); else SSD_CHAIN(float, 128); break;
    default: if (sb) SSD_CHAIN(bf16, 256); else SSD_CHAIN(float, 256); break;
  }
#undef SSD_CHAIN
  return hipGetLastError();
}

}  // namespace ssd
