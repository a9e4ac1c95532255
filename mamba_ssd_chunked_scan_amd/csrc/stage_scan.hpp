// stage_scan.hpp -- stage 5: the output of every position of every chunk,
//
//   y[l] = exp(cs[l]) * C_l . Hin[j]                              (Y_off)
//        + sum_{s <= l} exp(cs[l] - cs[s]) CB[l, s] f_s x_s        (Y_diag)
//        + D_h x_l;            out = y * silu(z)   when z is given
//
// SSD Reference: "Intra-chunk outputs and per-chunk states" (segment matrix
// L[l, s] = exp(A_cumsum[l] - A_cumsum[s]) 1[l >= s], Y_diag = (L o CB) X) and
// "Readout" (Y_off = C . state . exp(A_cumsum), Y = Y_diag + Y_off); the skip
// and SiLU gate of cudnn-frontend PR 1133.  f_s is the step size of token s
// when it scales the input term (dtc != NULL), else 1.  The mask is applied by selecting
// before exponentiating, so exp never sees the positive exponents above the
// diagonal (exp(large) * 0 would be inf * 0).
//
// One workgroup per (chunk, head, 64-wide slice of P).  LDS holds the chunk's
// cumsum and f, x transposed ([p][s], the reduction axis contiguous for the Y_diag
// B operand) and the carry-in state ([p][n], split into bf16 hi + lo when it is
// stored in fp32).  Wave w owns the 16-row l-tiles w and 7 - w of every group
// of 8 (balancing the causal triangle) and all four p-tiles.  The decay-weighted
// CB fragment and the C fragment are built once per (l-tile, k-block) and reused
// across p-tiles.  The epilogue goes through LDS so that x, z and out move in
// coalesced 16-byte rows.
#pragma once
#include "common.hpp"

namespace ssd {

// Carry-in state in LDS, per (input type, state type).
template <typename T, typename ST> struct HinLds;
template <> struct HinLds<bf16, float> {  // fp32 state -> bf16 hi + lo
  static __host__ __device__ int ld(int N) { return N + 8; }
  static __host__ __device__ size_t bytes(int N) { return 2ull * 64 * ld(N) * sizeof(bf16); }
  static __device__ void stage(char* base, const float* src, int N, int prow, int n, f32x8 v) {
    bf16* hi = reinterpret_cast<bf16*>(base);
    bf16* lo = hi + 64 * ld(N);
    FragSplit f = split_f32x8(v);
    *reinterpret_cast<bf16x8*>(&hi[prow * ld(N) + n]) = f.hi;
    *reinterpret_cast<bf16x8*>(&lo[prow * ld(N) + n]) = f.lo;
  }
  static __device__ FragSplit frag(const char* base, int N, int prow, int k) {
    const bf16* hi = reinterpret_cast<const bf16*>(base);
    const bf16* lo = hi + 64 * ld(N);
    FragSplit f;
    f.hi = *reinterpret_cast<const bf16x8*>(&hi[prow * ld(N) + k]);
    f.lo = *reinterpret_cast<const bf16x8*>(&lo[prow * ld(N) + k]);
    return f;
  }
  static __device__ void stage1(char* base, int N, int prow, int n, float v) {
    bf16* hi = reinterpret_cast<bf16*>(base);
    bf16* lo = hi + 64 * ld(N);
    const bf16 h = (bf16)v;
    hi[prow * ld(N) + n] = h;
    lo[prow * ld(N) + n] = (bf16)(v - (float)h);
  }
};
template <> struct HinLds<bf16, bf16> {  // bf16 state is exact
  static __host__ __device__ int ld(int N) { return N + 8; }
  static __host__ __device__ size_t bytes(int N) { return 64ull * ld(N) * sizeof(bf16); }
  static __device__ void stage(char* base, const bf16*, int N, int prow, int n, f32x8 v) {
    bf16* hi = reinterpret_cast<bf16*>(base);
    bf16x8 o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (bf16)v[i];
    *reinterpret_cast<bf16x8*>(&hi[prow * ld(N) + n]) = o;
  }
  static __device__ FragBF frag(const char* base, int N, int prow, int k) {
    const bf16* hi = reinterpret_cast<const bf16*>(base);
    FragBF f;
    f.v = *reinterpret_cast<const bf16x8*>(&hi[prow * ld(N) + k]);
    return f;
  }
  static __device__ void stage1(char* base, int N, int prow, int n, float v) {
    reinterpret_cast<bf16*>(base)[prow * ld(N) + n] = (bf16)v;
  }
};
template <typename ST> struct HinLdsF32 {  // fp32 inputs: fp32 operands throughout
  static __host__ __device__ int ld(int N) { return N + 4; }
  static __host__ __device__ size_t bytes(int N) { return 64ull * ld(N) * sizeof(float); }
  static __device__ void stage(char* base, const ST*, int N, int prow, int n, f32x8 v) {
    Vec8<float>::store(reinterpret_cast<float*>(base) + prow * ld(N) + n, v);
  }
  static __device__ void stage1(char* base, int N, int prow, int n, float v) {
    reinterpret_cast<float*>(base)[prow * ld(N) + n] = v;
  }
  static __device__ FragF32 frag(const char* base, int N, int prow, int k) {
    FragF32 f;
    f.v = Vec8<float>::load(reinterpret_cast<const float*>(base) + prow * ld(N) + k);
    return f;
  }
};
template <> struct HinLds<float, float> : HinLdsF32<float> {};
template <> struct HinLds<float, bf16> : HinLdsF32<bf16> {};

template <typename ST> struct StLoad;
template <> struct StLoad<float> {
  static __device__ f32x8 load(const float* p) { return Vec8<float>::load(p); }
};
template <> struct StLoad<bf16> {
  static __device__ f32x8 load(const bf16* p) { return Vec8<bf16>::load(p); }
};

template <typename T> __host__ __device__ constexpr int xt_pad() { return sizeof(T) == 2 ? 8 : 4; }

struct ScanLayout {
  size_t off_x, off_h, bytes;
  int ldx, ldy;
};

template <typename T, typename ST>
__host__ __device__ inline ScanLayout scan_layout(int C, int N) {
  ScanLayout L;
  L.ldx = C + xt_pad<T>();
  L.ldy = 64 + 4;
  L.off_x = 8 * C;  // cs, then f: C floats each
  const size_t xbytes = 64ull * L.ldx * sizeof(T);
  L.off_h = (L.off_x + xbytes + 15) & ~size_t(15);
  const size_t hb = HinLds<T, ST>::bytes(N);
  const size_t yb = (size_t)C * L.ldy * sizeof(float);
  L.bytes = L.off_h + (hb > yb ? hb : yb);
  return L;
}

// fp32 inputs with every operand split into bf16 hi + lo (three bf16 matrix
// instructions per product instead of eight fp32 ones): x^T is held as a hi
// and a lo plane, the carry-in state as HinLds<bf16, ST>.
template <typename ST>
__host__ __device__ inline ScanLayout scan_layout_split(int C, int N) {
  ScanLayout L;
  L.ldx = C + 8;  // bf16 per x^T row, per plane
  L.ldy = 64 + 4;
  L.off_x = 8 * C;
  const size_t xbytes = 2ull * 64 * L.ldx * sizeof(bf16);
  L.off_h = (L.off_x + xbytes + 15) & ~size_t(15);
  const size_t hb = HinLds<bf16, ST>::bytes(N);
  const size_t yb = (size_t)C * L.ldy * sizeof(float);
  L.bytes = L.off_h + (hb > yb ? hb : yb);
  return L;
}

// ------------------------------------------------------------------ bf16 fast path
//
// Same math, organised to keep many loads in flight and LDS traffic free of
// bank conflicts:
//   * prologue: every thread issues all of its x and carry-in-state loads at
//     once; x is written transposed as packed token pairs (a wave covers one
//     8-column group and the chunk's token pairs, so every LDS write hits one
//     row's consecutive dwords), the state as bf16 hi + lo;
//   * the z tile for the epilogue is prefetched into registers before the
//     matrix-core phase and consumed after it;
//   * per 16-row l-tile, all C and CB fragment loads are issued before the
//     matrix instructions that use them;
//   * the D skip is added in the accumulator layout from x^T in LDS (no second
//     read of x from memory), then y goes through LDS once for a coalesced,
//     gated, 16-byte-row store.

template <int C> struct ScanCfg {
  static constexpr int NPAIR = C / 2;
  static constexpr int LDW = (C + 8) / 2;                  // dwords per x^T row
  static constexpr int XU = (8 * NPAIR + 255) / 256;       // x units (2 tokens x 8 p) / thread
  static constexpr int ZV = (C * 8 + 255) / 256;           // epilogue 8-vectors / thread
  static constexpr int NLT = C / 16;                       // l-tiles
  static constexpr int LTW = NLT >= 8 ? NLT / 4 : 1;       // l-tiles per wave
};

template <typename ST>
__host__ __device__ inline ScanLayout scan_layout_bf16(int C, int N) {
  ScanLayout L;
  L.ldx = (C + 8) / 2;  // dwords
  L.ldy = 64 + 4;
  // cs, then f: C floats each (at C = 128 this keeps three workgroups' LDS
  // within a CU's 160 KB)
  L.off_x = 8 * C;
  const size_t xbytes = 64ull * L.ldx * 4;
  L.off_h = (L.off_x + xbytes + 15) & ~size_t(15);
  const size_t hb = HinLds<bf16, ST>::bytes(N);
  const size_t yb = (size_t)C * L.ldy * sizeof(float);
  L.bytes = L.off_h + (hb > yb ? hb : yb);
  return L;
}

// Fragments one wave needs for one 16-row l-tile: the first four k-blocks of
// C (Y_off A operand) and of the CB row block (Y_diag).  Loaded ahead of use.
struct ScanFrags {
  u32x4 cf[4];
  f32x8 cb[4];
};

// One workgroup computes the outputs of (chunk j, head h, columns [64 pz,
// 64 pz + 64) of P); smem holds scan_layout_bf16<ST>(C, N).bytes bytes.
// F: the step size scales the input term (dtc is read), compiled in only then.
template <typename ST, typename TO, int C, bool F>
__device__ __forceinline__ void chunk_scan_block(const Geo& g, const float* CB, const TArg& x,
                                                 const TArg& Cm, const float* cs,
                                                 const float* dtc, const ST* states,
                                                 const float* D, const TArg& z,
                                                 const TArg& out, float* yoff, int j, int h,
                                                 int pz, char* smem) {
  using Cfg = ScanCfg<C>;
  using HL = HinLds<bf16, ST>;
  constexpr int NPAIR = Cfg::NPAIR, LDW = Cfg::LDW;
  const int p0 = pz * 64;
  Chunk c;
  if (!get_chunk(g, j, c)) return;
  const int N = g.N, P = g.P;
  const int grp = h / g.hpg;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int r16 = lane % 16, q = lane / 16;
  const ScanLayout lay = scan_layout_bf16<ST>(C, N);
  float* s_cs = reinterpret_cast<float*>(smem);
  float* s_f = s_cs + C;
  uint32_t* s_xt = reinterpret_cast<uint32_t*>(smem + lay.off_x);
  char* s_h = smem + lay.off_h;
  float* s_y = reinterpret_cast<float*>(smem + lay.off_h);
  const int pw = min(64, P - p0);
  const float* cbm = CB + ((int64_t)j * g.G + grp) * C * C;
  const int nkb = (N + 31) / 32;

  // l-tile of the wave's u-th slot: w and 7 - w of every group of eight
  auto lt_of = [&](int u) { return (u / 2) * 8 + ((u & 1) ? 7 - wave : wave); };
  // Loads for one l-tile, issued before they are needed.  Addresses are always
  // inside the tensors (rows clamped into the chunk, columns into N, the CB tile
  // covers every (l, s) of the chunk); values that must not count are zeroed
  // where they are consumed.
  auto load_frags = [&](int u, ScanFrags& f) {
    const int lt = lt_of(u);
    const int lrow = lt * 16 + r16;
    const int nkd = (lt * 16 + 16 + 31) / 32;  // k-blocks the causal row block needs
    const bf16* crow = row_ptr<bf16>(Cm, c.b, c.t0 + min(lrow, c.len - 1), grp);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int k = min(kk * 32 + q * 8, N - 8);
      f.cf[kk] = *reinterpret_cast<const u32x4*>(crow + k);
      // past the causal block: repeat the last needed address (a cache hit)
      f.cb[kk] = Vec8<float>::load(cbm + (int64_t)lrow * C + min(kk, nkd - 1) * 32 + q * 8);
    }
  };

  // ---- prologue: every load of the tile's first phase at once
  u32x4 xr[Cfg::XU][2];
#pragma unroll
  for (int k = 0; k < Cfg::XU; ++k) {
    const int u = min(tid + 256 * k, 8 * NPAIR - 1);
    const int grp8 = u / NPAIR, pr = u % NPAIR;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int s = 2 * pr + t;
      xr[k][t] = *reinterpret_cast<const u32x4*>(
          row_ptr<bf16>(x, c.b, c.t0 + min(s, c.len - 1), h) + p0 + min(grp8 * 8, pw - 8));
    }
  }
  ScanFrags fr;
  if (lt_of(0) < Cfg::NLT) load_frags(0, fr);
  const ST* hsrc = states + ((int64_t)j * g.H + h) * P * N;
  const int nvec_h = 64 * (N / 8);
  constexpr int HB = 8;  // state 8-vectors per thread per batch
  for (int v0 = 0; v0 < nvec_h; v0 += 256 * HB) {
    f32x8 hv[HB];
#pragma unroll
    for (int b = 0; b < HB; ++b) {
      const int v = min(v0 + tid + 256 * b, nvec_h - 1);
      const int pr = min(v / (N / 8), pw - 1), n = (v % (N / 8)) * 8;
      hv[b] = StLoad<ST>::load(hsrc + (int64_t)(p0 + pr) * N + n);
    }
#pragma unroll
    for (int b = 0; b < HB; ++b) {
      const int v = v0 + tid + 256 * b;
      if (v < nvec_h) {
        const int pr = v / (N / 8);
        f32x8 val = hv[b];
        if (pr >= pw) {
#pragma unroll
          for (int e = 0; e < 8; ++e) val[e] = 0.0f;
        }
        HL::stage(s_h, hsrc, N, pr, (v % (N / 8)) * 8, val);
      }
    }
  }
  const float* csr = cs + ((int64_t)j * g.H + h) * C;
  const float* dtr = dtc ? dtc + ((int64_t)j * g.H + h) * C : nullptr;
  for (int l = tid; l < C; l += 256) {
    s_cs[l] = csr[l] * 1.4426950408889634f;  // base 2: every decay is one 2^x
    s_f[l] = dtr ? dtr[l] : 1.0f;
  }
#pragma unroll
  for (int k = 0; k < Cfg::XU; ++k) {
    const int u = tid + 256 * k;
    if (u >= 8 * NPAIR) continue;
    const int grp8 = u / NPAIR, pr = u % NPAIR;
    const bool col_ok = grp8 * 8 < pw;
    const bool k0 = col_ok && 2 * pr < c.len, k1 = col_ok && 2 * pr + 1 < c.len;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int row = grp8 * 8 + 2 * d;
      const uint32_t a = k0 ? xr[k][0][d] : 0u, b = k1 ? xr[k][1][d] : 0u;
      s_xt[row * LDW + pr] = pack_lo(a, b);
      s_xt[(row + 1) * LDW + pr] = pack_hi(a, b);
    }
  }
  __syncthreads();

  // ---- prefetch z for the epilogue (row-major 8-vectors)
  const int vpr = pw / 8;
  u32x4 zr[Cfg::ZV];
  if (z.p) {
#pragma unroll
    for (int k = 0; k < Cfg::ZV; ++k) {
      const int v = tid + 256 * k;
      const int l = min(v / vpr, c.len - 1), pp = (v % vpr) * 8;
      zr[k] = *reinterpret_cast<const u32x4*>(row_ptr<bf16>(z, c.b, c.t0 + l, h) + p0 + pp);
    }
  }

  // ---- matrix-core phase.  All four p-tiles run even when fewer than 64
  // columns are in range: x^T and state rows past P were staged as zeros.
  f32x4 acc[Cfg::LTW][4];
#pragma unroll
  for (int a = 0; a < Cfg::LTW; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = zero4();

#pragma unroll
  for (int u = 0; u < Cfg::LTW; ++u) {
    const int lt = lt_of(u);
    if (lt >= Cfg::NLT) continue;
    const int lrow = lt * 16 + r16;
    const bool lok = lrow < c.len;
    const bf16* crow = row_ptr<bf16>(Cm, c.b, c.t0 + min(lrow, c.len - 1), grp);
    // Y_off: C_l . Hin^T.  The first four k-blocks come from the prefetch.
    for (int k0 = 0; k0 < nkb; k0 += 4) {
      FragBF cf[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int k = (k0 + kk) * 32 + q * 8;
        const u32x4 raw = k0 == 0 ? fr.cf[kk]
                                  : *reinterpret_cast<const u32x4*>(crow + min(k, N - 8));
        const u32x4 zero = {0u, 0u, 0u, 0u};
        cf[kk].v = __builtin_bit_cast(bf16x8, (lok && k < N) ? raw : zero);
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int k = (k0 + kk) * 32 + q * 8;
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          auto b = HL::frag(s_h, N, pt * 16 + r16, k < N ? k : 0);
          mma(acc[u][pt], cf[kk], b);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = fast_exp2(s_cs[lt * 16 + q * 4 + i]);
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) acc[u][pt][i] *= e;
    }
    // optionally keep Y_off on its own, (tokens, H, P) fp32 on the packed axis
    if (yoff) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int l = lt * 16 + q * 4 + i;
        if (l >= c.len) continue;
        float* yr = yoff + ((int64_t)(c.b * g.T + c.t0 + l) * g.H + h) * P + p0;
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
          if (pt * 16 + r16 < pw) yr[pt * 16 + r16] = acc[u][pt][i];
      }
    }
    // Y_diag: (L o CB) x over s <= l.  The first four k-blocks come from the
    // prefetch; the mask is a select after the exponential (whose argument is
    // zeroed where masked, so it never overflows).
    const float csl = s_cs[lrow];
    const int nkd = (lt * 16 + 16 + 31) / 32;
    f32x8 cbv[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) cbv[kk] = fr.cb[kk];
    // the prefetch buffer is free again: start loading the next l-tile
    if (u + 1 < Cfg::LTW && lt_of(u + 1) < Cfg::NLT) load_frags(u + 1, fr);
    for (int k0 = 0; k0 < nkd; k0 += 4) {
      if (k0 > 0) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          cbv[kk] = Vec8<float>::load(cbm + (int64_t)lrow * C + min(k0 + kk, nkd - 1) * 32 + q * 8);
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        if (k0 + kk >= nkd) break;
        const int s0 = (k0 + kk) * 32 + q * 8;
        // the cumsum, then the x^T fragments, whose LDS latency runs under the
        // decay weights below (LDS reads complete in order: waiting for the
        // cumsum does not wait for them)
        const f32x8 csv = Vec8<float>::load(s_cs + s0);
        FragBF xb[4];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
          xb[pt].v = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                                    &s_xt[(pt * 16 + r16) * LDW + s0 / 2]));
        f32x8 m;
        if (k0 + kk < nkd - 1 && c.len == C) {
          // a k-block wholly below the diagonal of a full chunk: every
          // (l, s) is kept, the exponent is <= 0 (or small for growth)
#pragma unroll
          for (int e = 0; e < 8; ++e) m[e] = fast_exp2(csl - csv[e]) * cbv[kk][e];
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int s = s0 + e;
            const bool keep = lok && (s <= lrow) && (s < c.len);
            const float ex = fast_exp2(keep ? csl - csv[e] : 0.0f);
            m[e] = keep ? ex * cbv[kk][e] : 0.0f;
          }
        }
        if constexpr (F) {
          const f32x8 fv = Vec8<float>::load(s_f + s0);
#pragma unroll
          for (int e = 0; e < 8; ++e) m[e] *= fv[e];
        }
        const FragSplit mf = split_f32x8(m);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) mma(acc[u][pt], mf, xb[pt]);
      }
    }
  }

  // ---- D skip in the accumulator layout, from x^T in LDS
  if (D) {
    const float Dh = D[h];
#pragma unroll
    for (int u = 0; u < Cfg::LTW; ++u) {
      const int lt = lt_of(u);
      if (lt >= Cfg::NLT) continue;
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const u32x2 xv = *reinterpret_cast<const u32x2*>(
            &s_xt[(pt * 16 + r16) * LDW + (lt * 16 + q * 4) / 2]);
        acc[u][pt][0] += Dh * bf16_lo_f32(xv[0]);
        acc[u][pt][1] += Dh * bf16_hi_f32(xv[0]);
        acc[u][pt][2] += Dh * bf16_lo_f32(xv[1]);
        acc[u][pt][3] += Dh * bf16_hi_f32(xv[1]);
      }
    }
  }
  __syncthreads();  // all waves are done with the state; reuse its area for y
#pragma unroll
  for (int u = 0; u < Cfg::LTW; ++u) {
    const int lt = lt_of(u);
    if (lt >= Cfg::NLT) continue;
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) s_y[(lt * 16 + q * 4 + i) * lay.ldy + pt * 16 + r16] = acc[u][pt][i];
    }
  }
  __syncthreads();

  // ---- epilogue: gate and store, coalesced 8-element rows
#pragma unroll
  for (int k = 0; k < Cfg::ZV; ++k) {
    const int v = tid + 256 * k;
    const int l = v / vpr, pp = (v % vpr) * 8;
    if (l >= c.len) continue;
    f32x8 y = Vec8<float>::load(s_y + l * lay.ldy + pp);
    if (z.p) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        y[2 * d] *= silu(bf16_lo_f32(zr[k][d]));
        y[2 * d + 1] *= silu(bf16_hi_f32(zr[k][d]));
      }
    }
    Vec8<TO>::store(row_ptr_mut<TO>(out, c.b, c.t0 + l, h) + p0 + pp, y);
  }
}

}  // namespace ssd
