// fused_fwd.hip -- the whole SSD forward pass (stages 1-5) as one pass over the
// inputs: x, B, C, dt and z are read, out and the final states are written,
// and nothing chunk-sized goes through HBM in between.
//
// The math is the chunked algorithm of the SSD Reference ("Chunking and the
// discretized log-decay", "Intra-chunk outputs and per-chunk states",
// "Inter-chunk propagation", "Readout") with the D skip and SiLU gate of
// cudnn-frontend PR 1133, organised the way vLLM PR 27299 ("Purpose")
// describes its fused kernel: the log-decay cumsum and C.B^T are recomputed
// where they are consumed instead of being stored, and the chunk-to-chunk state
// is handed between workgroups through memory with inter-workgroup
// synchronisation.
//
// Work split.  The internal chunk is 128 tokens (the chunked result does not
// depend on the chunk length, so the problem's chunk_size only matters to the
// staged path).  A unit is (head h, 64-row slab of P); its chunks are cut into
// `nr` ranges of R consecutive chunks, and one workgroup owns one (unit,
// range).  A workgroup
//   1. (pass 1, only if a later range continues its last sequence) runs the
//      chunk-state recurrence over its range from a zero state -- or from the
//      sequence's initial state when the sequence starts inside the range --
//      and publishes that aggregate with the range's total decay E;
//   2. if its first chunk continues a sequence, waits for the aggregates of
//      the preceding ranges back to the one where the sequence starts and sums
//      them, decayed, in a fixed order: the carry-in state (a decoupled
//      look-back that never depends on timing, so results are bit-identical
//      run to run);
//   3. (pass 2) walks its chunks: cumsum from dt, chunk state S_j, the carry-in
//      H_j of the chunk staged in LDS as bf16 hi + lo, C.B^T tile by tile,
//      Y_off + Y_diag + D x, SiLU gate, store; then H_{j+1} = exp(Lambda_j)
//      H_j + S_j in registers, and the final state at a sequence's last chunk.
// Workgroups take (unit, range) in order from an atomic ticket counter, so a
// workgroup only ever waits for work that a running or finished workgroup
// owns: no residency assumption, no deadlock.  Every wait is bounded; on
// timeout an error bit is set in the workspace and the kernel still finishes.
//
// Per chunk, per workgroup (4 waves, wave w):
//   * S_j^T (n x p) = B^T (n x s) . (w_s x_s) (s x p): wave w owns p-tile w
//     and all n-tiles; the carried state uses this accumulator layout (lane:
//     one p, four consecutive n per n-tile), which is also the layout of the
//     carry-in rows the Y_off operand reads from LDS;
//   * C.B^T: wave w computes the tiles (s-tile, l-tile) of its l-tiles w and
//     7 - w (balanced causal work) with B and C fragments read straight from
//     global memory (n contiguous).  The accumulator layout of a C.B^T tile
//     (lane: one l, four consecutive s) is used directly as the A operand of
//     Y_diag = M . x with the k (token) order permuted to match; the x operand
//     is read from x^T in LDS in the same permuted order, so M never goes
//     through LDS.
// Precision is that of the staged path: exact bf16 inputs, fp32-derived
// operands (decay-weighted x, M = L o CB, the carried state) split into bf16
// hi + lo, fp32 accumulation, fp64 within-chunk cumsum rounded once.
#include "kernels.hpp"
#include "stage_varlen.hpp"

namespace ssd {

namespace {

constexpr int FC = 128;                 // internal chunk length
constexpr int FNP = FC / 2;             // token pairs per chunk
constexpr int FLDW = (FC + 8) / 2;      // dwords per transposed (token-pair) row
constexpr int FXU = (8 * FNP) / 256;    // x staging units per thread (token pair x 8 p)
constexpr int FZV = (FC * 8) / 256;     // epilogue 8-vectors per thread
constexpr int FYLD = 64 + 4;            // floats per staged output row
constexpr uint32_t kFlagAgg = 1;        // aggregate of a range that continues a sequence
constexpr uint32_t kFlagReset = 2;      // aggregate of a range where the sequence starts
constexpr int kSpinLimit = 1 << 18;     // polls (~1 us each) before giving up

template <int NT> struct FCfg {
  static constexpr int NMAX = 16 * NT;         // d_state capacity
  static constexpr int NKB = NT / 2;           // 32-wide k-blocks over n
  static constexpr int BU = NT / 2;            // B staging units per thread
  static constexpr int HLD = NMAX + 8;         // bf16 per carry-in row in LDS
  static constexpr int OFF_CS = 0;             // cs[128]
  static constexpr int OFF_W = 512;            // w[128] = exp(Lambda - cs)
  static constexpr int OFF_MISC = 1024;        // broadcast words
  static constexpr int OFF_XT = 1088;          // x^T [64 p][FLDW]
  static constexpr int XT_BYTES = 64 * FLDW * 4;
  static constexpr int OFF_R = OFF_XT + XT_BYTES;   // B^T, then carry-in, then y
  static constexpr int BT_BYTES = NMAX * FLDW * 4;
  static constexpr int H_BYTES = 2 * 64 * HLD * 2;
  static constexpr int Y_BYTES = FC * FYLD * 4;
  static constexpr int R_BYTES = BT_BYTES > H_BYTES ? (BT_BYTES > Y_BYTES ? BT_BYTES : Y_BYTES)
                                                    : (H_BYTES > Y_BYTES ? H_BYTES : Y_BYTES);
  static constexpr int LDS = OFF_R + R_BYTES;
};

}  // namespace

struct FusedArgs {
  Geo g;                  // 128-token chunk geometry; meta = the fused chunk table
  TArg x, B, C, dt, z, out;
  int dt_bf16;
  const float* A;
  const float* dt_bias;
  const float* D;
  const float* h0;
  float* hfinal;
  int softplus, clamp;
  float dt_min, dt_max;
  int U, PS, R;           // units, P slabs per head, chunks per range
  uint32_t* sync;         // [0] ticket counter, [1] error bits, [2 + r * U + u] flags
  float* edec;            // [r * U + u] total decay of the range's aggregate
  float* agg;             // [r * U + u][64][NMAX] aggregates
};

template <typename TO, int NT>
__global__ __launch_bounds__(256, 2) void k_fused_fwd(FusedArgs a) {
  using Cfg = FCfg<NT>;
  constexpr int NMAX = Cfg::NMAX, NKB = Cfg::NKB, BU = Cfg::BU, HLD = Cfg::HLD;
  __shared__ __align__(16) char smem[Cfg::LDS];
  float* s_cs = reinterpret_cast<float*>(smem + Cfg::OFF_CS);
  float* s_w = reinterpret_cast<float*>(smem + Cfg::OFF_W);
  uint32_t* s_misc = reinterpret_cast<uint32_t*>(smem + Cfg::OFF_MISC);
  uint32_t* s_xt = reinterpret_cast<uint32_t*>(smem + Cfg::OFF_XT);
  uint32_t* s_bt = reinterpret_cast<uint32_t*>(smem + Cfg::OFF_R);
  bf16* s_hh = reinterpret_cast<bf16*>(smem + Cfg::OFF_R);
  bf16* s_hl = s_hh + 64 * HLD;
  float* s_y = reinterpret_cast<float*>(smem + Cfg::OFF_R);

  const Geo& g = a.g;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int r16 = lane % 16, q = lane / 16;

  if (tid == 0)
    s_misc[0] = __hip_atomic_fetch_add(a.sync, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int ticket = (int)s_misc[0];
  const int r = ticket / a.U, u = ticket % a.U;
  const int h = u / a.PS, p0 = (u % a.PS) * 64;
  const int grp = h / g.hpg;
  const int pw = min(64, g.P - p0);
  const int Kr = g.meta ? g.meta[0] : g.K;
  const int j0 = r * a.R, j1 = min(j0 + a.R, Kr);
  if (j0 >= j1) return;

  // this lane's column of the carried state: p = p0 + pl, n = 16 nt + 4 q + i
  const int pl = wave * 16 + r16;
  const bool p_ok = pl < pw;
  const int64_t PN = (int64_t)g.P * g.N;
  auto state_row = [&](int seq) { return ((int64_t)seq * g.H + h) * PN + (int64_t)(p0 + pl) * g.N; };
  auto slot = [&](int rr) { return ((int64_t)rr * a.U + u) * 64 * NMAX + pl * NMAX + q * 4; };
  auto load_h0 = [&](f32x4 (&v)[NT], int seq) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      v[nt] = zero4();
      if (a.h0 && p_ok && nt * 16 < g.N)
        v[nt] = *reinterpret_cast<const f32x4*>(a.h0 + state_row(seq) + nt * 16 + q * 4);
    }
  };

  const float Ah = a.A[h];
  const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
  u32x4 xr[FXU][2], br[BU][2], zr[FZV];
  float dtv[2];

  // ---- issue every global load of chunk c (x, B, dt; z when gating)
  auto load_chunk = [&](const Chunk& c, bool with_z) {
#pragma unroll
    for (int k = 0; k < FXU; ++k) {
      const int uu = tid + 256 * k, grp8 = uu / FNP, pr = uu % FNP;
#pragma unroll
      for (int t = 0; t < 2; ++t)
        xr[k][t] = *reinterpret_cast<const u32x4*>(
            row_ptr<bf16>(a.x, c.b, c.t0 + min(2 * pr + t, c.len - 1), h) + p0 +
            min(grp8 * 8, pw - 8));
    }
#pragma unroll
    for (int k = 0; k < BU; ++k) {
      const int uu = tid + 256 * k, grp8 = uu / FNP, pr = uu % FNP;
#pragma unroll
      for (int t = 0; t < 2; ++t)
        br[k][t] = *reinterpret_cast<const u32x4*>(
            row_ptr<bf16>(a.B, c.b, c.t0 + min(2 * pr + t, c.len - 1), grp) +
            min(grp8 * 8, g.N - 8));
    }
    if (wave == 0) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int t = c.t0 + min(2 * lane + e, c.len - 1);
        dtv[e] = a.dt_bf16 ? to_f32<bf16>(*row_ptr<bf16>(a.dt, c.b, t, h))
                           : *row_ptr<float>(a.dt, c.b, t, h);
      }
    }
    if (with_z && a.z.p) {
#pragma unroll
      for (int k = 0; k < FZV; ++k) {
        const int v = tid + 256 * k, l = v / 8, pp = (v % 8) * 8;
        zr[k] = *reinterpret_cast<const u32x4*>(
            row_ptr<bf16>(a.z, c.b, c.t0 + min(l, c.len - 1), h) + p0 + min(pp, pw - 8));
      }
    }
  };

  // ---- LDS: cumsum, decay weights, x^T and B^T as packed token pairs.
  // Tokens past the chunk's end (loaded as copies of its last token), columns
  // past P and rows past N are zeroed here.
  auto stage_chunk = [&](const Chunk& c) {
    if (wave == 0) {
      double av[2], run = 0.0;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int l = 2 * lane + e;
        float aa = 0.0f;
        if (l < c.len) {
          const float uu = dtv[e] + bias;
          float d = a.softplus ? softplus_f32(uu) : uu;
          if (a.clamp) d = fminf(fmaxf(d, a.dt_min), a.dt_max);
          aa = d * Ah;
        }
        run += (double)aa;
        av[e] = run;
      }
      const double incl = wave_inclusive_sum_f64(run);
      const double excl = incl - run;
      const float c0 = (float)(excl + av[0]), c1 = (float)(excl + av[1]);
      s_cs[2 * lane] = c0;
      s_cs[2 * lane + 1] = c1;
      const int ll = c.len - 1;
      const float lam = __shfl((ll & 1) ? c1 : c0, ll >> 1, kWave);
      s_w[2 * lane] = 2 * lane < c.len ? fast_exp(lam - c0) : 0.0f;
      s_w[2 * lane + 1] = 2 * lane + 1 < c.len ? fast_exp(lam - c1) : 0.0f;
      if (lane == 0) s_misc[1] = __float_as_uint(lam);
    }
#pragma unroll
    for (int k = 0; k < FXU; ++k) {
      const int uu = tid + 256 * k, grp8 = uu / FNP, pr = uu % FNP;
      const bool col_ok = grp8 * 8 < pw;
      const bool k0 = col_ok && 2 * pr < c.len, k1 = col_ok && 2 * pr + 1 < c.len;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int row = grp8 * 8 + 2 * d;
        const uint32_t va = k0 ? xr[k][0][d] : 0u, vb = k1 ? xr[k][1][d] : 0u;
        s_xt[row * FLDW + pr] = pack_lo(va, vb);
        s_xt[(row + 1) * FLDW + pr] = pack_hi(va, vb);
      }
    }
#pragma unroll
    for (int k = 0; k < BU; ++k) {
      const int uu = tid + 256 * k, grp8 = uu / FNP, pr = uu % FNP;
      const bool n_ok = grp8 * 8 < g.N;
      const bool k0 = n_ok && 2 * pr < c.len, k1 = n_ok && 2 * pr + 1 < c.len;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int row = grp8 * 8 + 2 * d;
        const uint32_t va = k0 ? br[k][0][d] : 0u, vb = k1 ? br[k][1][d] : 0u;
        s_bt[row * FLDW + pr] = pack_lo(va, vb);
        s_bt[(row + 1) * FLDW + pr] = pack_hi(va, vb);
      }
    }
  };

  // ---- S_j^T = B^T (w x): wave w owns p-tile w, all n-tiles
  auto state_mma = [&](f32x4 (&acc)[NT]) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = zero4();
#pragma unroll
    for (int kb = 0; kb < FC / 32; ++kb) {
      const int off = kb * 16 + q * 4;  // dwords of tokens 32 kb + 8 q .. + 7
      const u32x4 xv = *reinterpret_cast<const u32x4*>(&s_xt[pl * FLDW + off]);
      const f32x4 w0 = *reinterpret_cast<const f32x4*>(&s_w[kb * 32 + q * 8]);
      const f32x4 w1 = *reinterpret_cast<const f32x4*>(&s_w[kb * 32 + q * 8 + 4]);
      f32x8 xw;
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        xw[2 * d] = bf16_lo_f32(xv[d]) * w0[2 * d];
        xw[2 * d + 1] = bf16_hi_f32(xv[d]) * w0[2 * d + 1];
        xw[4 + 2 * d] = bf16_lo_f32(xv[2 + d]) * w1[2 * d];
        xw[4 + 2 * d + 1] = bf16_hi_f32(xv[2 + d]) * w1[2 * d + 1];
      }
      const FragSplit b = split_f32x8(xw);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        FragBF av;
        av.v = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                              &s_bt[(nt * 16 + r16) * FLDW + off]));
        mma(acc[nt], av, b);
      }
    }
  };

  // ---- sequence structure of the range
  Chunk cfirst, clast;
  get_chunk(g, j0, cfirst);
  get_chunk(g, j1 - 1, clast);
  int f0, l0, fs, ls;
  seq_chunks(g, cfirst.seq, f0, l0);
  seq_chunks(g, clast.seq, fs, ls);
  const bool need_lb = f0 < j0;        // the first chunk continues a sequence
  const bool publish = j1 < ls;        // the next range continues the last sequence
  const bool reset = fs >= j0;         // the last sequence starts inside the range

  f32x4 carry[NT];

  // ---- pass 1: the range's aggregate
  if (publish) {
    const int js = reset ? fs : j0;
    if (reset) load_h0(carry, clast.seq);
    else {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) carry[nt] = zero4();
    }
    float E = 1.0f;
    for (int j = js; j < j1; ++j) {
      Chunk c;
      get_chunk(g, j, c);
      load_chunk(c, false);
      __syncthreads();
      stage_chunk(c);
      __syncthreads();
      f32x4 S[NT];
      state_mma(S);
      const float e = fast_exp(__uint_as_float(s_misc[1]));
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) carry[nt][i] = fmaf(e, carry[nt][i], S[nt][i]);
      E *= e;
    }
    float* dst = a.agg + slot(r);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) *reinterpret_cast<f32x4*>(dst + nt * 16) = carry[nt];
    if (tid == 0) a.edec[r * a.U + u] = E;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (tid == 0)
      __hip_atomic_store(a.sync + 2 + r * a.U + u, reset ? kFlagReset : kFlagAgg,
                         __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- carry-in: the decayed sum of the preceding ranges' aggregates, back
  // to the range where the sequence starts
  if (need_lb) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) carry[nt] = zero4();
    float dec = 1.0f;
    for (int rr = r - 1; rr >= 0; --rr) {
      if (tid == 0) {
        uint32_t f;
        int spins = 0;
        while ((f = __hip_atomic_load(a.sync + 2 + rr * a.U + u, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT)) == 0) {
          if (++spins > kSpinLimit) {
            __hip_atomic_fetch_or(a.sync + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            f = kFlagReset;
            break;
          }
          __builtin_amdgcn_s_sleep(2);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        s_misc[2] = f;
      }
      __syncthreads();
      const uint32_t f = s_misc[2];
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      const float* src = a.agg + slot(rr);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(src + nt * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) carry[nt][i] = fmaf(dec, v[i], carry[nt][i]);
      }
      const float e = a.edec[rr * a.U + u];
      __syncthreads();
      if (f == kFlagReset) break;
      dec *= e;
    }
  }

  // ---- pass 2: outputs, chunk by chunk
  for (int j = j0; j < j1; ++j) {
    Chunk c;
    get_chunk(g, j, c);
    load_chunk(c, true);
    __syncthreads();  // the previous chunk's epilogue is done with LDS
    stage_chunk(c);
    __syncthreads();
    f32x4 S[NT];
    state_mma(S);
    const float lam = __uint_as_float(s_misc[1]);
    __syncthreads();  // B^T is dead: its space takes the carry-in state

    int fj, lj;
    seq_chunks(g, c.seq, fj, lj);
    if (j == fj) load_h0(carry, c.seq);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      bf16x4 hi, lo;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16 hv = (bf16)carry[nt][i];
        hi[i] = hv;
        lo[i] = (bf16)(carry[nt][i] - (float)hv);
      }
      *reinterpret_cast<bf16x4*>(&s_hh[pl * HLD + nt * 16 + q * 4]) = hi;
      *reinterpret_cast<bf16x4*>(&s_hl[pl * HLD + nt * 16 + q * 4]) = lo;
    }
    const float e = fast_exp(lam);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) carry[nt][i] = fmaf(e, carry[nt][i], S[nt][i]);
    if (j == lj - 1 && a.hfinal && p_ok) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        if (nt * 16 < g.N)
          *reinterpret_cast<f32x4*>(a.hfinal + state_row(c.seq) + nt * 16 + q * 4) = carry[nt];
    }
    __syncthreads();

    // ---- Y for l-tiles w and 7 - w, all four p-tiles, one l-tile at a time
    f32x4 acc[2][4];
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int ui = 0; ui < 2; ++ui) {
      const int lt = ui ? 7 - wave : wave;
      const int lrow = lt * 16 + r16;
      const bool lok = lrow < c.len;
      // C fragments: the A operand of Y_off and the B operand of C.B^T
      u32x4 cfr[NKB];
      const bf16* crow = row_ptr<bf16>(a.C, c.b, c.t0 + min(lrow, c.len - 1), grp);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        cfr[kb] = *reinterpret_cast<const u32x4*>(crow + min(kb * 32 + q * 8, g.N - 8));
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) acc[ui][pt] = zero4();
      // Y_off = exp(cs_l) C_l . H_j
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const bool nok = kb * 32 + q * 8 < g.N;
        cfr[kb] = (lok && nok) ? cfr[kb] : zero;
        FragBF cf;
        cf.v = __builtin_bit_cast(bf16x8, cfr[kb]);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          FragSplit hs;
          hs.hi = *reinterpret_cast<const bf16x8*>(&s_hh[(pt * 16 + r16) * HLD + kb * 32 + q * 8]);
          hs.lo = *reinterpret_cast<const bf16x8*>(&s_hl[(pt * 16 + r16) * HLD + kb * 32 + q * 8]);
          mma(acc[ui][pt], cf, hs);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ex = fast_exp(s_cs[lt * 16 + q * 4 + i]);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) acc[ui][pt][i] *= ex;
      }
      // Y_diag = (L o C.B^T) x, two s-tiles (one 32-token k-block) at a time
      const float csl = s_cs[lrow];
      for (int kp = 0; kp <= lt / 2; ++kp) {
        const int sa = 2 * kp, sb = 2 * kp + 1;
        const int rowa = sa * 16 + r16, rowb = sb * 16 + r16;
        const bf16* pa = row_ptr<bf16>(a.B, c.b, c.t0 + min(rowa, c.len - 1), grp);
        const bf16* pb = row_ptr<bf16>(a.B, c.b, c.t0 + min(rowb, c.len - 1), grp);
        u32x4 ba[NKB], bb[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const int n = min(kb * 32 + q * 8, g.N - 8);
          ba[kb] = *reinterpret_cast<const u32x4*>(pa + n);
          bb[kb] = *reinterpret_cast<const u32x4*>(pb + n);
        }
        // rows past the chunk only reach M entries the token mask removes,
        // and columns past N meet zeros in the C operand
        f32x4 cba = zero4(), cbb = zero4();
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          FragBF A0, A1, Bc;
          A0.v = __builtin_bit_cast(bf16x8, ba[kb]);
          A1.v = __builtin_bit_cast(bf16x8, bb[kb]);
          Bc.v = __builtin_bit_cast(bf16x8, cfr[kb]);
          mma(cba, A0, Bc);
          mma(cbb, A1, Bc);
        }
        const f32x4 csa = *reinterpret_cast<const f32x4*>(&s_cs[sa * 16 + q * 4]);
        const f32x4 csb = *reinterpret_cast<const f32x4*>(&s_cs[sb * 16 + q * 4]);
        f32x8 m;
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const bool ka = lok && sa * 16 + q * 4 + e4 <= lrow;
          const bool kb2 = lok && sb * 16 + q * 4 + e4 <= lrow;
          const float xa = fast_exp(ka ? csl - csa[e4] : 0.0f);
          const float xb = fast_exp(kb2 ? csl - csb[e4] : 0.0f);
          m[e4] = ka ? xa * cba[e4] : 0.0f;
          m[4 + e4] = kb2 ? xb * cbb[e4] : 0.0f;
        }
        const FragSplit mf = split_f32x8(m);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          const uint32_t* xrow = &s_xt[(pt * 16 + r16) * FLDW];
          const u32x2 xa = *reinterpret_cast<const u32x2*>(xrow + sa * 8 + q * 2);
          const u32x2 xb = *reinterpret_cast<const u32x2*>(xrow + sb * 8 + q * 2);
          const u32x4 xv = {xa[0], xa[1], xb[0], xb[1]};
          FragBF xf;
          xf.v = __builtin_bit_cast(bf16x8, xv);
          mma(acc[ui][pt], mf, xf);
        }
      }
    }
    // D skip from x^T
    if (a.D) {
      const float Dh = a.D[h];
#pragma unroll
      for (int ui = 0; ui < 2; ++ui) {
        const int lt = ui ? 7 - wave : wave;
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          const u32x2 xv =
              *reinterpret_cast<const u32x2*>(&s_xt[(pt * 16 + r16) * FLDW + lt * 8 + q * 2]);
          acc[ui][pt][0] += Dh * bf16_lo_f32(xv[0]);
          acc[ui][pt][1] += Dh * bf16_hi_f32(xv[0]);
          acc[ui][pt][2] += Dh * bf16_lo_f32(xv[1]);
          acc[ui][pt][3] += Dh * bf16_hi_f32(xv[1]);
        }
      }
    }
    __syncthreads();  // every wave is done with the carry-in rows
#pragma unroll
    for (int ui = 0; ui < 2; ++ui) {
      const int lt = ui ? 7 - wave : wave;
#pragma unroll
      for (int pt = 0; pt < 4; ++pt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          s_y[(lt * 16 + q * 4 + i) * FYLD + pt * 16 + r16] = acc[ui][pt][i];
    }
    __syncthreads();
    // ---- epilogue: gate and store, coalesced 8-element rows
#pragma unroll
    for (int k = 0; k < FZV; ++k) {
      const int v = tid + 256 * k, l = v / 8, pp = (v % 8) * 8;
      if (l >= c.len || pp >= pw) continue;
      f32x8 y = Vec8<float>::load(s_y + l * FYLD + pp);
      if (a.z.p) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          y[2 * d] *= silu(bf16_lo_f32(zr[k][d]));
          y[2 * d + 1] *= silu(bf16_hi_f32(zr[k][d]));
        }
      }
      Vec8<TO>::store(row_ptr_mut<TO>(a.out, c.b, c.t0 + l, h) + p0 + pp, y);
    }
  }
}

// Resets the synchronisation words, builds the 128-token chunk table of a
// packed batch and writes the final state of every sequence without tokens.
__global__ __launch_bounds__(256) void k_fused_prep(Geo g, const int32_t* cu, int32_t* meta,
                                                    uint32_t* sync, int nsync, int nflag_blocks,
                                                    const float* h0, float* hfinal) {
  __shared__ int lds_waves[4];
  const int bid = blockIdx.x;
  if (bid == 0) {
    if (cu) varlen_meta_block(cu, g.nseq, g.T, g.C, g.K, meta, lds_waves);
    return;
  }
  if (bid <= nflag_blocks) {
    for (int i = (bid - 1) * 256 + threadIdx.x; i < nsync; i += nflag_blocks * 256) sync[i] = 0u;
    return;
  }
  const int seq = bid - 1 - nflag_blocks;
  bool empty;
  if (cu) {
    int st, L;
    seq_span(cu, seq, g.T, st, L);
    empty = L == 0;
  } else {
    empty = g.T == 0;
  }
  if (!empty) return;
  const int64_t n = (int64_t)g.H * g.P * g.N;
  float* dst = hfinal + (int64_t)seq * n;
  const float* src = h0 ? h0 + (int64_t)seq * n : nullptr;
  for (int64_t i = threadIdx.x; i < n; i += 256) dst[i] = src ? src[i] : 0.0f;
}

FusedPlan fused_plan(int64_t K, int H, int P, int N) {
  FusedPlan pl;
  pl.PS = (P + 63) / 64;
  pl.U = H * pl.PS;
  pl.NT = N <= 32 ? 2 : (N <= 64 ? 4 : 8);
  if (K <= 0) {
    pl.R = 1;
    pl.nr = 0;
    return pl;
  }
  int64_t nr = kFusedTargetWorkgroups / pl.U;
  nr = nr < 1 ? 1 : (nr > K ? K : nr);
  pl.R = (int)((K + nr - 1) / nr);
  pl.nr = (int)((K + pl.R - 1) / pl.R);
  return pl;
}

hipError_t launch_fused_fwd(const FusedLaunch& f, hipStream_t s) {
  const Geo& g = f.g;
  const FusedPlan& pl = f.plan;
  const int nsync = 2 + pl.nr * pl.U;
  const int nflag_blocks = min((nsync + 255) / 256, 64);
  const int nfinal = f.hfinal ? g.nseq : 0;
  hipLaunchKernelGGL(k_fused_prep, dim3(1 + nflag_blocks + nfinal), dim3(256), 0, s, g, f.cu,
                     f.meta, f.sync, nsync, nflag_blocks, f.h0, f.hfinal);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.nr == 0) return e;

  FusedArgs a;
  a.g = g;
  a.x = f.x; a.B = f.B; a.C = f.C; a.dt = f.dt; a.z = f.z; a.out = f.out;
  a.dt_bf16 = f.dt_dtype == DT_BF16;
  a.A = f.A; a.dt_bias = f.dt_bias; a.D = f.D; a.h0 = f.h0; a.hfinal = f.hfinal;
  a.softplus = f.softplus; a.clamp = f.clamp; a.dt_min = f.dt_min; a.dt_max = f.dt_max;
  a.U = pl.U; a.PS = pl.PS; a.R = pl.R;
  a.sync = f.sync; a.edec = f.edec; a.agg = f.agg;
  const dim3 grid((unsigned)(pl.nr * pl.U));
  const bool ob = f.out_dtype == DT_BF16;
#define SSD_FUSED(TO, NT) hipLaunchKernelGGL((k_fused_fwd<TO, NT>), grid, dim3(256), 0, s, a)
  switch (pl.NT) {
    case 2: if (ob) SSD_FUSED(bf16, 2); else SSD_FUSED(float, 2); break;
    case 4: if (ob) SSD_FUSED(bf16, 4); else SSD_FUSED(float, 4); break;
    default: if (ob) SSD_FUSED(bf16, 8); else SSD_FUSED(float, 8); break;
  }
#undef SSD_FUSED
  return hipGetLastError();
}

}  // namespace ssd
