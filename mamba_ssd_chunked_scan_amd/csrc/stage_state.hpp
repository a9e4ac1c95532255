// stage_state.hpp -- stage 3: every chunk's end state from a zero start,
//
//   S[j, h, p, n] = sum_{s < len} w_s x[t0 + s, h, p] B[t0 + s, g, n],
//   w_s = exp(cs[len - 1] - cs[s])
//
// SSD Reference, "Intra-chunk outputs and per-chunk states" (the states einsum
// with decay_states = exp(A_cumsum[-1] - A_cumsum)) and "Algorithm and
// tensor-shape contract" step 6 (state = Xc^T (decay_states * Bc)).  Unlike the
// page, the decay weight is folded into x rather than B: x is the per-head
// operand, B is shared by the heads of a group.
//
// Matrix-core formulation: S (P x N) = Xw^T (P x s) * B (s x N), reducing over
// tokens s.  Tokens are the strided axis in memory while the 16x16x32 MFMA
// wants eight consecutive tokens per lane, so x and B pass through LDS
// transposed ([p][s], [n][s]).
//
// bf16 inputs (the fast path).  One workgroup covers 64 (p) x 128 (n) of one
// (chunk, head); wave w owns p-tile w and all eight n-tiles (8 fp32 16x16
// accumulators).  Tokens are processed in slabs of up to 64 (~38 KB of LDS,
// four workgroups per CU):
//   * every load of a slab is issued at once into registers (2 x 16 B of x and
//     4 x 16 B of B per thread), and the next slab's loads are issued before the
//     current slab's MFMAs, so a workgroup waits on memory about once per slab;
//   * the transpose is written as packed token pairs: a thread holds tokens
//     (s, s+1) for 8 columns and writes 8 dwords (x[s][c], x[s+1][c]); half a
//     wave covers one 8-column group's 32 token pairs, so each LDS write
//     instruction touches two runs of 32 consecutive dwords;
//   * the weighted x is split into bf16 hi + lo on the way in;
//   * the finished tile goes through LDS so the state is stored in coalesced
//     16-byte rows.
// fp32 inputs use a simpler slab loop with fp32 MFMA (small problems only).
#pragma once
#include "common.hpp"

namespace ssd {

// ------------------------------------------------------------------ bf16 path

template <int C> struct StateCfg {
  static constexpr int SL = C < 64 ? C : 64;       // tokens per slab
  static constexpr int NSL = C / SL;
  static constexpr int NPAIR = SL / 2;
  static constexpr int LD = SL + 8;                // bf16 elements per transposed row
  static constexpr int LDW = LD / 2;               // the same in dwords
  static constexpr int XU = (8 * NPAIR + 255) / 256;   // x units (2 tokens x 8 p) per thread
  static constexpr int BU = (16 * NPAIR + 255) / 256;  // B units (2 tokens x 8 n) per thread
  static constexpr int LDS_T = (2 * 64 + 128) * LDW;   // dwords: x hi, x lo, B
  static constexpr int LDS_S = 64 * (128 + 4);         // floats: output tile
  static constexpr int LDS = LDS_T > LDS_S ? LDS_T : LDS_S;
};

// LDS bytes one workgroup of the bf16 chunk-state body needs.
template <int C> __host__ __device__ constexpr size_t chunk_state_lds_bytes() {
  return (size_t)StateCfg<C>::LDS * 4 + (size_t)C * 4;
}

// One workgroup computes the 64 (p) x 128 (n) block z of the state of
// (chunk j, head h); smem holds chunk_state_lds_bytes<C>() bytes.
template <typename ST, int C>
__device__ __forceinline__ void chunk_state_block(const Geo& g, const TArg& x, const TArg& B,
                                                  const float* cs, const float* dtc, ST* states,
                                                  int j, int h, int z, char* smem) {
  using Cfg = StateCfg<C>;
  constexpr int SL = Cfg::SL, NPAIR = Cfg::NPAIR, LDW = Cfg::LDW, XU = Cfg::XU, BU = Cfg::BU;
  uint32_t* lds = reinterpret_cast<uint32_t*>(smem);
  float* w = reinterpret_cast<float*>(smem + (size_t)Cfg::LDS * 4);
  uint32_t* xh = lds;
  uint32_t* xl = lds + 64 * LDW;
  uint32_t* bt = lds + 128 * LDW;

  Chunk c;
  if (!get_chunk(g, j, c)) return;
  const int nzn = (g.N + 127) / 128;
  const int p0 = (z / nzn) * 64, n0 = (z % nzn) * 128;
  const int grp = h / g.hpg;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int r16 = lane % 16, q = lane / 16;

  u32x4 xr[XU][2], br[BU][2];
  auto load_slab = [&](int sl) {
#pragma unroll
    for (int k = 0; k < XU; ++k) {
      const int u = tid + 256 * k;
      const int grp8 = u / NPAIR, pr = u % NPAIR;
      const int s = sl * SL + 2 * pr, p = p0 + grp8 * 8;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (u < 8 * NPAIR && s + t < c.len && p < g.P)
          v = *reinterpret_cast<const u32x4*>(row_ptr<bf16>(x, c.b, c.t0 + s + t, h) + p);
        xr[k][t] = v;
      }
    }
#pragma unroll
    for (int k = 0; k < BU; ++k) {
      const int u = tid + 256 * k;
      const int grp8 = u / NPAIR, pr = u % NPAIR;
      const int s = sl * SL + 2 * pr, n = n0 + grp8 * 8;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (u < 16 * NPAIR && s + t < c.len && n < g.N)
          v = *reinterpret_cast<const u32x4*>(row_ptr<bf16>(B, c.b, c.t0 + s + t, grp) + n);
        br[k][t] = v;
      }
    }
  };
  auto write_slab = [&](int sl) {
#pragma unroll
    for (int k = 0; k < XU; ++k) {
      const int u = tid + 256 * k;
      if (u >= 8 * NPAIR) continue;
      const int grp8 = u / NPAIR, pr = u % NPAIR;
      const float wa = w[sl * SL + 2 * pr], wb = w[sl * SL + 2 * pr + 1];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const uint32_t ua = xr[k][0][d], ub = xr[k][1][d];
          const float fa = __uint_as_float(half ? (ua & 0xffff0000u) : (ua << 16)) * wa;
          const float fb = __uint_as_float(half ? (ub & 0xffff0000u) : (ub << 16)) * wb;
          const bf16 ha = (bf16)fa, hb = (bf16)fb;
          const bf16 la = (bf16)(fa - (float)ha), lb = (bf16)(fb - (float)hb);
          const int row = grp8 * 8 + 2 * d + half;
          xh[row * LDW + pr] = pack2(ha, hb);
          xl[row * LDW + pr] = pack2(la, lb);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < BU; ++k) {
      const int u = tid + 256 * k;
      if (u >= 16 * NPAIR) continue;
      const int grp8 = u / NPAIR, pr = u % NPAIR;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int row = grp8 * 8 + 2 * d;
        bt[row * LDW + pr] = pack_lo(br[k][0][d], br[k][1][d]);
        bt[(row + 1) * LDW + pr] = pack_hi(br[k][0][d], br[k][1][d]);
      }
    }
  };

  load_slab(0);
  {
    const float* csr = cs + ((int64_t)j * g.H + h) * g.C;
    const float* dtr = dtc ? dtc + ((int64_t)j * g.H + h) * g.C : nullptr;
    const float last = csr[c.len - 1];
    for (int s = tid; s < C; s += 256)
      w[s] = s < c.len ? fast_exp(last - csr[s]) * (dtr ? dtr[s] : 1.0f) : 0.0f;
  }
  __syncthreads();

  const int pt0 = p0 + wave * 16;
  const bool active = pt0 < g.P;
  const int ntn = min(8, (g.N - n0) / 16);
  f32x4 acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = zero4();

#pragma unroll
  for (int sl = 0; sl < Cfg::NSL; ++sl) {
    if (sl * SL >= c.len) break;
    write_slab(sl);
    __syncthreads();
    if (sl + 1 < Cfg::NSL && (sl + 1) * SL < c.len) load_slab(sl + 1);
    if (active) {
#pragma unroll
      for (int kb = 0; kb < SL / 32; ++kb) {
        const int off = kb * 16 + q * 4;  // dword offset of this lane's 8 tokens
        FragSplit a;
        a.hi = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                              &xh[(wave * 16 + r16) * LDW + off]));
        a.lo = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                              &xl[(wave * 16 + r16) * LDW + off]));
        // all eight n-tiles run unconditionally: LDS rows past N hold zeros,
        // and a data-dependent guard around the matrix instructions would make
        // the compiler keep conditional copies of every accumulator
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          FragBF b;
          b.v = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                               &bt[(t * 16 + r16) * LDW + off]));
          mma(acc[t], a, b);
        }
      }
    }
    __syncthreads();
  }

  // stage the 64 x 128 tile through LDS, then coalesced 16-byte stores
  float* so = reinterpret_cast<float*>(lds);
  constexpr int LDO = 128 + 4;
  if (active) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if (t >= ntn) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) so[(wave * 16 + q * 4 + i) * LDO + t * 16 + r16] = acc[t][i];
    }
  }
  __syncthreads();
  const int prows = min(64, g.P - p0), ncols = ntn * 16;
  const int vpr = ncols / 8;
  ST* out = states + ((int64_t)j * g.H + h) * g.P * g.N;
  for (int v = tid; v < prows * vpr; v += 256) {
    const int pr = v / vpr, nn = (v % vpr) * 8;
    const f32x8 val = Vec8<float>::load(so + pr * LDO + nn);
    Vec8<ST>::store(out + (int64_t)(p0 + pr) * g.N + n0 + nn, val);
  }
}

}  // namespace ssd
